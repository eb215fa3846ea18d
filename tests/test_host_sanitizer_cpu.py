"""The library's host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source of the library is compiled with its usual flags, the host code additionally
instrumented (`-Xarch_host -fsanitize=...`; device code is left as it is), and linked into
a plain C client.  The client calls every entry point of asa.h with arguments that the
host checks reject (NULL pointers, bad shapes and dtypes, unknown patterns, short CSR
capacity and workspace, out-of-range parameters, shapes beyond the static scratch), plus
the size queries and message functions.  Every rejected call returns before anything is
enqueued, so no GPU is needed.  The run must exit cleanly with no sanitizer report.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

CLIENT = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "asa.h"

static int fails = 0;
#define EXPECT(call, code) do { asa_status st_ = (call); if (st_ != (code)) { \
    printf("line %d: got %d want %d (%s)\n", __LINE__, (int)st_, (int)(code), asa_last_error()); ++fails; } \
    else if (strlen(asa_last_error()) == 0) { printf("line %d: empty message\n", __LINE__); ++fails; } } while (0)

int main(void) {
  void* F = (void*)0x10000;            /* never dereferenced: validation fails first */
  void* W = (void*)0x40000;            /* 256-byte aligned fake workspace */
  asa_shape s = {1, 2, 1024, 64, 64, ASA_BF16};
  asa_shape bad_d = {1, 2, 1024, 96, 64, ASA_BF16};
  asa_shape bad_b = {0, 2, 1024, 64, 64, ASA_BF16};
  asa_shape bad_t = {1, 2, 1024, 64, 64, 7};
  asa_shape many_blocks = {1, 1, 64 * 1025, 64, 64, ASA_BF16};
  asa_shape big = {2, 24, 75600, 128, 128, ASA_BF16};
  asa_shape f32 = {1, 2, 1024, 64, 64, ASA_F32};
  int64_t cap = asa_csr_capacity(&s);
  if (cap != 2 * 16 * 16) { printf("capacity %lld\n", (long long)cap); ++fails; }
  if (asa_csr_capacity(&bad_d) != -1 || asa_csr_capacity(NULL) != -1) { printf("capacity of a bad shape\n"); ++fails; }
  if (asa_build_mask_workspace_size(&bad_d) != 0 || asa_static_mask_workspace_size(&bad_b) != 0 ||
      asa_attention_bwd_workspace_size(&many_blocks) != 0 || asa_pattern_search_workspace_size(&s, 9) != 0 ||
      asa_attention_fwd_split_workspace_size(&s, -1) != 0) { printf("size of a bad call\n"); ++fails; }
  size_t need = asa_build_mask_workspace_size(&s);
  asa_csr csr = {(int32_t*)0x20000, (int32_t*)0x30000, cap, NULL};
  asa_csr small = {(int32_t*)0x20000, (int32_t*)0x30000, cap - 1, NULL};
  asa_csr nullcsr = {NULL, (int32_t*)0x30000, cap, NULL};
  asa_adaptive ad = {ASA_MODE_TOPK, 4, 0.0, 0, 0, 1};
  asa_adaptive bad_mode = {5, 4, 0.0, 0, 0, 1};
  asa_adaptive bad_k = {ASA_MODE_TOPK, -1, 0.0, 0, 0, 1};
  asa_adaptive bad_tau = {ASA_MODE_TAU, 0, NAN, 0, 0, 1};
  asa_adaptive bad_cap = {ASA_MODE_TAU, 0, 0.9, -2, 0, 1};
  asa_adaptive bad_text = {ASA_MODE_TOPK, 4, 0.0, 0, 5000, 1};
  asa_adaptive bad_diag = {ASA_MODE_TOPK, 4, 0.0, 0, 0, 2};
  asa_head_pattern unknown[2] = {{9, 0}, {0, 0}};
  asa_head_pattern md0[2] = {{ASA_PAT_MULTIDIAG, 0}, {0, 0}};
  asa_head_pattern vs[2] = {{ASA_PAT_VSTRIPE, -1}, {0, 0}};
  asa_head_pattern ft[2] = {{ASA_PAT_FRAME_TILE, 0}, {ASA_PAT_FULL, 0}};
  asa_head_pattern adapt[2] = {{ASA_PAT_ADAPTIVE, 0}, {ASA_PAT_FULL, 0}};
  asa_head_pattern good[2] = {{ASA_PAT_DIAG, 0}, {ASA_PAT_FULL, 0}};

  /* asa_build_mask */
  EXPECT(asa_build_mask(NULL, F, &s, &ad, NULL, &csr, W, need, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_build_mask(F, F, NULL, &ad, NULL, &csr, W, need, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_build_mask(F, F, &s, NULL, NULL, &csr, W, need, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_build_mask(F, F, &bad_b, &ad, NULL, &csr, W, need, NULL), ASA_ERR_BAD_SHAPE);
  EXPECT(asa_build_mask(F, F, &bad_d, &ad, NULL, &csr, W, need, NULL), ASA_ERR_UNSUPPORTED);
  EXPECT(asa_build_mask(F, F, &bad_t, &ad, NULL, &csr, W, need, NULL), ASA_ERR_BAD_DTYPE);
  EXPECT(asa_build_mask(F, F, &many_blocks, &ad, NULL, &csr, W, need, NULL), ASA_ERR_UNSUPPORTED);
  EXPECT(asa_build_mask(F, F, &s, &bad_mode, NULL, &csr, W, need, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask(F, F, &s, &bad_k, NULL, &csr, W, need, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask(F, F, &s, &bad_tau, NULL, &csr, W, need, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask(F, F, &s, &bad_cap, NULL, &csr, W, need, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask(F, F, &s, &bad_text, NULL, &csr, W, need, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask(F, F, &s, &bad_diag, NULL, &csr, W, need, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask(F, F, &s, &ad, unknown, &csr, W, need, NULL), ASA_ERR_BAD_PATTERN);
  EXPECT(asa_build_mask(F, F, &s, &ad, md0, &csr, W, need, NULL), ASA_ERR_BAD_PATTERN);
  EXPECT(asa_build_mask(F, F, &s, &ad, vs, &csr, W, need, NULL), ASA_ERR_BAD_PATTERN);
  EXPECT(asa_build_mask(F, F, &s, &ad, NULL, &small, W, need, NULL), ASA_ERR_CAPACITY);
  EXPECT(asa_build_mask(F, F, &s, &ad, NULL, &nullcsr, W, need, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_build_mask(F, F, &s, &ad, NULL, &csr, NULL, need, NULL), ASA_ERR_WORKSPACE);
  EXPECT(asa_build_mask(F, F, &s, &ad, NULL, &csr, W, need - 1, NULL), ASA_ERR_WORKSPACE);
  EXPECT(asa_build_mask(F, F, &s, &ad, NULL, &csr, (char*)W + 16, need, NULL), ASA_ERR_WORKSPACE);

  /* asa_build_mask_noalloc */
  asa_csr bigcsr = {(int32_t*)0x20000, (int32_t*)0x30000, asa_csr_capacity(&big), NULL};
  EXPECT(asa_build_mask_noalloc(NULL, F, &s, &ad, NULL, &csr, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_build_mask_noalloc(F, F, &bad_d, &ad, NULL, &csr, NULL), ASA_ERR_UNSUPPORTED);
  EXPECT(asa_build_mask_noalloc(F, F, &s, &bad_k, NULL, &csr, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_build_mask_noalloc(F, F, &s, &ad, NULL, &small, NULL), ASA_ERR_CAPACITY);
  EXPECT(asa_build_mask_noalloc(F, F, &big, &ad, NULL, &bigcsr, NULL), ASA_ERR_WORKSPACE);

  /* asa_static_mask */
  size_t sneed = asa_static_mask_workspace_size(&s);
  EXPECT(asa_static_mask(&s, NULL, &csr, W, sneed, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_static_mask(&s, adapt, &csr, W, sneed, NULL), ASA_ERR_BAD_PATTERN);
  EXPECT(asa_static_mask(&s, ft, &csr, W, sneed, NULL), ASA_ERR_BAD_PATTERN);
  EXPECT(asa_static_mask(&s, good, &small, W, sneed, NULL), ASA_ERR_CAPACITY);
  EXPECT(asa_static_mask(&s, good, &csr, W, 8, NULL), ASA_ERR_WORKSPACE);
  EXPECT(asa_static_mask(&bad_b, good, &csr, W, sneed, NULL), ASA_ERR_BAD_SHAPE);

  /* asa_attention_fwd, _lse, _split */
  EXPECT(asa_attention_fwd(F, F, F, NULL, ASA_F32, &s, &csr, NULL, 0.f, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_attention_fwd(F, F, F, F, 5, &s, &csr, NULL, 0.f, NULL), ASA_ERR_BAD_DTYPE);
  EXPECT(asa_attention_fwd(F, F, F, F, ASA_F32, &bad_d, &csr, NULL, 0.f, NULL), ASA_ERR_UNSUPPORTED);
  EXPECT(asa_attention_fwd(F, F, F, F, ASA_F32, &s, NULL, NULL, 0.f, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_attention_fwd(F, F, F, F, ASA_F32, &s, &nullcsr, NULL, 0.f, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_attention_fwd(F, F, F, F, ASA_F32, &s, &csr, NULL, INFINITY, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_attention_fwd(F, F, F, F, ASA_F32, &s, &csr, unknown, 0.f, NULL), ASA_ERR_BAD_PATTERN);
  EXPECT(asa_attention_fwd_lse(F, F, F, F, ASA_F32, &s, &csr, NULL, 0.f, NULL, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_attention_fwd_lse(F, F, F, F, 7, &s, &csr, NULL, 0.f, (float*)F, NULL), ASA_ERR_BAD_DTYPE);
  asa_shape wide = {1, 1, 64 * 1000, 64, 64, ASA_BF16};
  EXPECT(asa_attention_fwd_split(F, F, F, F, ASA_F32, &s, &csr, NULL, 0.f, NULL, -1, W, 1u << 30, NULL),
         ASA_ERR_BAD_PARAM);
  EXPECT(asa_attention_fwd_split(F, F, F, F, ASA_F32, &wide, &csr, NULL, 0.f, NULL, 10, W, 1u << 30, NULL),
         ASA_ERR_BAD_PARAM);
  EXPECT(asa_attention_fwd_split(F, F, F, F, ASA_F32, &s, &csr, NULL, 0.f, NULL, 4, NULL, 0, NULL),
         ASA_ERR_WORKSPACE);

  /* asa_attention_bwd */
  size_t bneed = asa_attention_bwd_workspace_size(&s);
  EXPECT(asa_attention_bwd(F, F, F, F, ASA_F32, F, NULL, (float*)F, (float*)F, (float*)F, &f32, &csr, NULL,
                           0.f, W, bneed, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_attention_bwd(F, F, F, F, ASA_F32, F, NULL, (float*)F, (float*)F, (float*)F, &s, &csr, NULL, 0.f, W,
                           bneed, NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_attention_bwd(F, F, F, F, 3, F, (float*)F, (float*)F, (float*)F, (float*)F, &s, &csr, NULL, 0.f, W,
                           bneed, NULL), ASA_ERR_BAD_DTYPE);
  EXPECT(asa_attention_bwd(F, F, F, F, ASA_F32, F, (float*)F, (float*)F, (float*)F, (float*)F, &s, &csr, NULL, 0.f,
                           W, bneed - 1, NULL), ASA_ERR_WORKSPACE);
  EXPECT(asa_attention_bwd(F, F, F, F, ASA_F32, F, (float*)F, (float*)F, (float*)F, (float*)F, &s, &csr, NULL, NAN,
                           W, bneed, NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_attention_bwd(F, F, F, F, ASA_F32, F, (float*)F, (float*)F, (float*)F, (float*)F, &s, &nullcsr, NULL,
                           0.f, W, bneed, NULL), ASA_ERR_NULL_ARG);

  /* asa_pattern_search */
  asa_head_pattern cands[2] = {{ASA_PAT_SKIP, 0}, {ASA_PAT_DIAG, 0}};
  asa_head_pattern cbad[1] = {{ASA_PAT_ADAPTIVE, 0}};
  size_t pneed = asa_pattern_search_workspace_size(&s, 2);
  EXPECT(asa_pattern_search(NULL, F, F, &s, cands, 2, 0.01, 0.1, 0.f, (double*)F, NULL, (int32_t*)F, W, pneed,
                            NULL), ASA_ERR_NULL_ARG);
  EXPECT(asa_pattern_search(F, F, F, &s, cands, 9, 0.01, 0.1, 0.f, (double*)F, NULL, (int32_t*)F, W, pneed, NULL),
         ASA_ERR_BAD_PARAM);
  EXPECT(asa_pattern_search(F, F, F, &s, cbad, 1, 0.01, 0.1, 0.f, (double*)F, NULL, (int32_t*)F, W, pneed, NULL),
         ASA_ERR_BAD_PATTERN);
  EXPECT(asa_pattern_search(F, F, F, &s, cands, 2, INFINITY, 0.1, 0.f, (double*)F, NULL, (int32_t*)F, W, pneed,
                            NULL), ASA_ERR_BAD_PARAM);
  EXPECT(asa_pattern_search(F, F, F, &s, cands, 2, 0.01, 0.1, 0.f, (double*)F, NULL, (int32_t*)F, W, pneed - 1,
                            NULL), ASA_ERR_WORKSPACE);
  EXPECT(asa_pattern_search(F, F, F, &bad_d, cands, 2, 0.01, 0.1, 0.f, (double*)F, NULL, (int32_t*)F, W, pneed,
                            NULL), ASA_ERR_UNSUPPORTED);

  /* messages */
  for (int st = 1; st >= -10; --st)
    if (asa_status_string((asa_status)st) == NULL) { printf("no status string %d\n", st); ++fails; }
  if (asa_version() < 10600) { printf("version %d\n", asa_version()); ++fails; }
  printf("fails %d\n", fails);
  return fails == 0 ? 0 : 1;
}
"""


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_asa_build_san", os.path.join(ROOT, "block_sparse_attention_asa_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(900)
def test_host_layer_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    b = _build_module()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    objs = []
    procs = []
    for src in b.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *b.COMMON, *b.EXTRA.get(src, []), *san, *lang, "-c", os.path.join(b.CSRC, src), "-o", obj]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src))
        objs.append(obj)
    for p, src in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"compiling {src}:\n{out[-3000:]}"
    client = tmp_path / "client.c"
    client.write_text(CLIENT)
    cobj = str(tmp_path / "client.o")
    subprocess.run([CLANG, "-std=c99", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", "-c", str(client), "-o", cobj],
                   check=True, capture_output=True)
    exe = str(tmp_path / "client")
    res = subprocess.run([HIPCC, "-fsanitize=address,undefined", cobj, *objs, "-o", exe,
                          "-Wl,-rpath,/opt/rocm/lib", "-L/opt/rocm/lib", "-lamdhip64", "-lm"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    text = run.stdout + run.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert run.returncode == 0, text[-4000:]
    assert "fails 0" in run.stdout
