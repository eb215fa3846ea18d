"""C-ABI library: loads, exports every declared symbol, validates arguments (no GPU needed).

Every call here fails validation on the host before anything is enqueued, so no
kernel runs and no device memory is touched (the fake addresses are never used).
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_asa_amd as asa
from block_sparse_attention_asa_amd import asa_shape, asa_adaptive, asa_head_pattern, asa_csr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "asa.h")
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, CAPACITY, WORKSPACE, BAD_PATTERN, BAD_PARAM = \
    0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(asa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("asa_build_mask", "asa_static_mask", "asa_attention_fwd"):
        assert must in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", asa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared in asa.h but not exported: {missing}"
    assert set(asa.EXPORTS) == set(declared_functions())


def _shape(B=1, H=2, N=1024, d=64, blk=64, dt=asa.ASA_BF16):
    return asa_shape(B, H, N, d, blk, dt)


def _csr(cap):
    return asa_csr(0x20000, 0x30000, cap)


def _build(shape, ad=None, pats=None, csr=None, ws_bytes=1 << 30, q=FAKE, k=FAKE, ws=0x40000):
    ad = ad or asa_adaptive(asa.TOPK, 4, 0.0, 0, 0, 1)
    csr = csr or _csr(asa.lib.asa_csr_capacity(ctypes.byref(shape)))
    return asa.lib.asa_build_mask(q, k, ctypes.byref(shape), ctypes.byref(ad), pats, ctypes.byref(csr),
                                  ctypes.c_void_p(ws), ws_bytes, None)


def test_capacity_and_workspace_sizes():
    s = _shape(N=1000, blk=64)                       # Nb = 16 (ragged)
    assert asa.lib.asa_csr_capacity(ctypes.byref(s)) == 2 * 16 * 16
    ws = asa.lib.asa_build_mask_workspace_size(ctypes.byref(s))
    rows = 2 * 16
    assert ws >= rows * 64 * 8 * 2 + rows * 4 + rows * 4   # pooled Q and K (float64), bitmasks, counts
    assert asa.lib.asa_static_mask_workspace_size(ctypes.byref(s)) >= rows * 8
    assert asa.lib.asa_build_mask_workspace_size(ctypes.byref(_shape(d=96))) == 0
    assert asa.lib.asa_csr_capacity(None) == -1
    assert asa.lib.asa_csr_capacity(ctypes.byref(_shape(d=96))) == -1          # shapes the builders reject
    assert asa.lib.asa_csr_capacity(ctypes.byref(_shape(N=64 * 1025, blk=64))) == -1   # Nb > 1024


@pytest.mark.parametrize("shape,code", [
    (_shape(B=0), BAD_SHAPE), (_shape(N=-5), BAD_SHAPE), (_shape(d=96), UNSUPPORTED),
    (_shape(blk=32), UNSUPPORTED), (_shape(dt=7), BAD_DTYPE), (_shape(H=300), UNSUPPORTED),
    (_shape(N=64 * 1025, blk=64), UNSUPPORTED),           # Nb > 1024 for the mask builders
])
def test_build_mask_rejects_shapes(shape, code):
    assert _build(shape) == code
    assert asa.lib.asa_last_error().decode() != ""


def test_build_mask_rejects_arguments():
    s = _shape()
    assert _build(s, q=None) == NULL_ARG
    assert _build(s, ad=asa_adaptive(5, 4, 0.0, 0, 0, 1)) == BAD_PARAM
    assert _build(s, ad=asa_adaptive(asa.TOPK, -1, 0.0, 0, 0, 1)) == BAD_PARAM
    assert _build(s, ad=asa_adaptive(asa.TAU, 0, float("nan"), 0, 0, 1)) == BAD_PARAM
    assert _build(s, ad=asa_adaptive(asa.TAU, 0, 0.9, -2, 0, 1)) == BAD_PARAM
    assert _build(s, ad=asa_adaptive(asa.TOPK, 4, 0.0, 0, 5000, 1)) == BAD_PARAM
    assert _build(s, ad=asa_adaptive(asa.TOPK, 4, 0.0, 0, 0, 2)) == BAD_PARAM
    assert _build(s, csr=_csr(10)) == CAPACITY
    assert _build(s, ws_bytes=100) == WORKSPACE
    assert _build(s, ws=0) == WORKSPACE
    assert _build(s, ws=0x40010) == WORKSPACE                # misaligned
    bad = (asa_head_pattern * 2)(asa_head_pattern(9, 0), asa_head_pattern(0, 0))
    assert _build(s, pats=bad) == BAD_PATTERN
    bad = (asa_head_pattern * 2)(asa_head_pattern(asa.MULTIDIAG, 0), asa_head_pattern(0, 0))
    assert _build(s, pats=bad) == BAD_PATTERN
    bad = (asa_head_pattern * 2)(asa_head_pattern(asa.VSTRIPE, -1), asa_head_pattern(0, 0))
    assert _build(s, pats=bad) == BAD_PATTERN


def test_build_mask_noalloc_rejects_arguments():
    """The variant without allocation validates like asa_build_mask, and rejects shapes whose
    workspace exceeds its static scratch before looking the scratch up."""
    assert asa.lib.asa_build_mask_noalloc.argtypes[-1] is ctypes.c_void_p
    s = _shape()
    ad = asa_adaptive(asa.TOPK, 4, 0.0, 0, 0, 1)
    csr = _csr(asa.lib.asa_csr_capacity(ctypes.byref(s)))
    call = lambda shape, c=csr, q=FAKE, a=ad: asa.lib.asa_build_mask_noalloc(
        q, FAKE, ctypes.byref(shape), ctypes.byref(a), None, ctypes.byref(c), None)
    assert call(s, q=None) == NULL_ARG
    assert call(_shape(d=96)) == UNSUPPORTED
    assert call(s, c=_csr(10)) == CAPACITY
    assert call(s, a=asa_adaptive(asa.TOPK, -1, 0.0, 0, 0, 1)) == BAD_PARAM
    big = _shape(B=2, H=24, N=75600, d=128, blk=128)
    need = asa.lib.asa_build_mask_workspace_size(ctypes.byref(big))
    assert need > asa.NOALLOC_SCRATCH_BYTES
    assert call(big, c=_csr(asa.lib.asa_csr_capacity(ctypes.byref(big)))) == WORKSPACE
    assert "static scratch" in asa.lib.asa_last_error().decode()
    # the five workload shapes fit (the largest is the 720p-like layer, 24 heads)
    for B, H, N, d in [(1, 2, 1024, 64), (1, 8, 8192, 64), (1, 48, 17776, 64), (1, 12, 32760, 128),
                       (1, 24, 75600, 128)]:
        sh = _shape(B=B, H=H, N=N, d=d, blk=128)
        assert 0 < asa.lib.asa_build_mask_workspace_size(ctypes.byref(sh)) <= asa.NOALLOC_SCRATCH_BYTES


def test_static_mask_rejects_arguments():
    s = _shape()
    cap = asa.lib.asa_csr_capacity(ctypes.byref(s))
    csr = _csr(cap)
    good = (asa_head_pattern * 2)(asa_head_pattern(asa.DIAG, 0), asa_head_pattern(asa.FULL, 0))
    adaptive = (asa_head_pattern * 2)(asa_head_pattern(asa.ADAPTIVE, 0), asa_head_pattern(asa.FULL, 0))
    call = asa.lib.asa_static_mask
    assert call(ctypes.byref(s), None, ctypes.byref(csr), ctypes.c_void_p(0x40000), 1 << 30, None) == NULL_ARG
    assert call(ctypes.byref(s), adaptive, ctypes.byref(csr), ctypes.c_void_p(0x40000), 1 << 30, None) == BAD_PATTERN
    small = _csr(cap - 1)
    assert call(ctypes.byref(s), good, ctypes.byref(small), ctypes.c_void_p(0x40000), 1 << 30, None) == CAPACITY
    assert call(ctypes.byref(s), good, ctypes.byref(csr), ctypes.c_void_p(0x40000), 8, None) == WORKSPACE
    nullcsr = asa_csr(0, 0x30000, cap)
    assert call(ctypes.byref(s), good, ctypes.byref(nullcsr), ctypes.c_void_p(0x40000), 1 << 30, None) == NULL_ARG
    for bad_f in (0, -5):
        tile = (asa_head_pattern * 2)(asa_head_pattern(asa.FRAME_TILE, bad_f), asa_head_pattern(asa.FULL, 0))
        assert call(ctypes.byref(s), tile, ctypes.byref(csr), ctypes.c_void_p(0x40000), 1 << 30, None) == BAD_PATTERN
        assert "frame-tile" in asa.lib.asa_last_error().decode()
    unknown = (asa_head_pattern * 2)(asa_head_pattern(7, 1), asa_head_pattern(asa.FULL, 0))
    assert call(ctypes.byref(s), unknown, ctypes.byref(csr), ctypes.c_void_p(0x40000), 1 << 30, None) == BAD_PATTERN


def test_attention_rejects_arguments():
    s = _shape()
    csr = _csr(10)
    call = asa.lib.asa_attention_fwd
    assert call(FAKE, FAKE, FAKE, None, asa.ASA_F32, ctypes.byref(s), ctypes.byref(csr), None, 0.0, None) == NULL_ARG
    assert call(FAKE, FAKE, FAKE, FAKE, 5, ctypes.byref(s), ctypes.byref(csr), None, 0.0, None) == BAD_DTYPE
    assert call(FAKE, FAKE, FAKE, FAKE, asa.ASA_F32, ctypes.byref(_shape(d=32)), ctypes.byref(csr), None, 0.0,
                None) == UNSUPPORTED
    assert call(FAKE, FAKE, FAKE, FAKE, asa.ASA_F32, ctypes.byref(s), None, None, 0.0, None) == NULL_ARG
    assert call(FAKE, FAKE, FAKE, FAKE, asa.ASA_F32, ctypes.byref(s), ctypes.byref(csr), None,
                float("inf"), None) == BAD_PARAM
    bad = (asa_head_pattern * 2)(asa_head_pattern(42, 0), asa_head_pattern(0, 0))
    assert call(FAKE, FAKE, FAKE, FAKE, asa.ASA_F32, ctypes.byref(s), ctypes.byref(csr), bad, 0.0,
                None) == BAD_PATTERN


def test_attention_lse_rejects_arguments():
    s = _shape()
    csr = _csr(10)
    call = asa.lib.asa_attention_fwd_lse
    assert call(FAKE, FAKE, FAKE, FAKE, asa.ASA_F32, ctypes.byref(s), ctypes.byref(csr), None, 0.0, None,
                None) == NULL_ARG                                   # lse NULL
    assert "lse" in asa.lib.asa_last_error().decode()
    assert call(FAKE, FAKE, FAKE, FAKE, 7, ctypes.byref(s), ctypes.byref(csr), None, 0.0, FAKE,
                None) == BAD_DTYPE


def _bwd(s, csr=None, ws=0x40000, ws_bytes=1 << 30, o_dtype=asa.ASA_F32, lse=FAKE, dq=FAKE, pats=None,
         scale=0.0):
    csr = csr or _csr(asa.lib.asa_csr_capacity(ctypes.byref(s)))
    return asa.lib.asa_attention_bwd(FAKE, FAKE, FAKE, FAKE, o_dtype, FAKE, lse, dq, FAKE, FAKE,
                                     ctypes.byref(s), ctypes.byref(csr), pats, scale, ctypes.c_void_p(ws),
                                     ws_bytes, None)


def test_attention_bwd_rejects_arguments():
    s = _shape()
    need = asa.lib.asa_attention_bwd_workspace_size(ctypes.byref(s))
    assert need > 0
    assert asa.lib.asa_attention_bwd_workspace_size(ctypes.byref(_shape(d=48))) == 0
    assert asa.lib.asa_attention_bwd_workspace_size(ctypes.byref(_shape(N=64 * 1025, blk=64))) == 0   # Nb > 1024
    assert _bwd(_shape(dt=asa.ASA_F32), lse=None) == NULL_ARG          # fp32 inputs pass the dtype check
    assert _bwd(s, lse=None) == NULL_ARG
    assert _bwd(s, dq=None) == NULL_ARG
    assert _bwd(s, o_dtype=3) == BAD_DTYPE
    assert _bwd(s, ws=0) == WORKSPACE
    assert _bwd(s, ws_bytes=need - 1) == WORKSPACE
    assert _bwd(s, ws=0x40010) == WORKSPACE                            # not 256-byte aligned
    assert _bwd(s, scale=float("nan")) == BAD_PARAM
    bad = (asa_head_pattern * 2)(asa_head_pattern(9, 0), asa_head_pattern(0, 0))
    assert _bwd(s, pats=bad) == BAD_PATTERN
    nullcsr = asa_csr(0, 0x30000, 10)
    assert _bwd(s, csr=nullcsr) == NULL_ARG


def _search(s, cands=None, n=None, lam=0.01, eps=0.1, scale=0.0, loss=FAKE, choice=FAKE, ws=0x40000,
            ws_bytes=1 << 30, q=FAKE):
    if cands is None:
        cands = [(asa.SKIP, 0), (asa.DIAG, 0)]
    arr = (asa_head_pattern * max(len(cands), 1))(*[asa_head_pattern(i, p) for i, p in cands])
    n = len(cands) if n is None else n
    return asa.lib.asa_pattern_search(q, FAKE, FAKE, ctypes.byref(s), arr, n, lam, eps, scale, loss, None,
                                      choice, ctypes.c_void_p(ws), ws_bytes, None)


def test_pattern_search_rejects_arguments():
    s = _shape()
    need = asa.lib.asa_pattern_search_workspace_size(ctypes.byref(s), 2)
    B, H, N, d, Nb = 1, 2, 1024, 64, 16
    # two fp32 outputs dominate the workspace
    assert need >= 2 * B * H * N * d * 4 + B * H * Nb * Nb * 4
    assert asa.lib.asa_pattern_search_workspace_size(ctypes.byref(s), 9) == 0
    assert asa.lib.asa_pattern_search_workspace_size(ctypes.byref(s), -1) == 0
    assert asa.lib.asa_pattern_search_workspace_size(ctypes.byref(_shape(N=64 * 1025, blk=64)), 2) == 0
    assert _search(s, q=None) == NULL_ARG
    assert _search(s, loss=None) == NULL_ARG
    assert _search(s, choice=None) == NULL_ARG
    assert _search(s, n=9) == BAD_PARAM
    assert _search(s, n=-1) == BAD_PARAM
    assert _search(s, cands=[(asa.ADAPTIVE, 0)]) == BAD_PATTERN
    assert "candidate 0" in asa.lib.asa_last_error().decode()
    assert _search(s, cands=[(asa.SKIP, 0), (asa.MULTIDIAG, 0)]) == BAD_PATTERN
    assert _search(s, cands=[(asa.VSTRIPE, -1)]) == BAD_PATTERN
    assert _search(s, cands=[(11, 0)]) == BAD_PATTERN
    assert _search(s, cands=[(asa.FRAME_TILE, 0)]) == BAD_PATTERN
    assert _search(s, lam=float("inf")) == BAD_PARAM
    assert _search(s, eps=float("nan")) == BAD_PARAM
    assert _search(s, scale=float("nan")) == BAD_PARAM
    assert _search(s, ws=0) == WORKSPACE
    assert _search(s, ws_bytes=need - 1) == WORKSPACE
    assert _search(s, ws=0x40010) == WORKSPACE
    assert _search(_shape(d=96)) == UNSUPPORTED


def _split(s, T=4, ws=0x40000, ws_bytes=1 << 30, lse=None, csr=None):
    csr = csr or _csr(asa.lib.asa_csr_capacity(ctypes.byref(s)))
    return asa.lib.asa_attention_fwd_split(FAKE, FAKE, FAKE, FAKE, asa.ASA_F32, ctypes.byref(s), ctypes.byref(csr),
                                           None, 0.0, lse, T, ctypes.c_void_p(ws), ws_bytes, None)


def test_attention_split_rejects_arguments():
    s = _shape()                                   # B1 H2 N1024 blk64: Nb 16, 32 rows
    B, H, Nb, blk, d = 1, 2, 16, 64, 64
    sz = lambda T: asa.lib.asa_attention_fwd_split_workspace_size(ctypes.byref(s), T)
    assert sz(4) >= 4 * B * H * Nb * blk * (d + 2) * 4     # 4 chunks per full row
    assert sz(16) == 0 and sz(100) == 0                    # T >= Nb: nothing to split
    assert sz(-1) == 0
    assert sz(0) == 0                                      # 16-block rows: never split automatically
    few = _shape(N=64 * 64)                                # 128 rows of 64 blocks: 4 chunks of 16
    assert asa.lib.asa_attention_fwd_split_workspace_size(ctypes.byref(few), 0) == \
        asa.lib.asa_attention_fwd_split_workspace_size(ctypes.byref(few), 16) > 0
    many = _shape(N=64 * 192)                              # 384 rows: not split automatically
    assert asa.lib.asa_attention_fwd_split_workspace_size(ctypes.byref(many), 0) == 0
    assert _split(s, T=-1) == BAD_PARAM
    big = _shape(N=64 * 1000, blk=64)                      # Nb 1000: T=10 would make 100 chunks
    assert _split(big, T=10) == BAD_PARAM
    assert "chunks" in asa.lib.asa_last_error().decode()
    assert _split(s, T=4, ws=0) == WORKSPACE
    assert _split(s, T=4, ws_bytes=sz(4) - 1) == WORKSPACE
    assert _split(s, T=4, ws=0x40010) == WORKSPACE
    nullcsr = asa_csr(0, 0x30000, 10)
    assert _split(s, csr=nullcsr) == NULL_ARG


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "asa.h"
int main(void) {
  asa_shape s = {1, 2, 1024, 64, 64, ASA_BF16};
  if (asa_version() < 10400) return 1;
  if (asa_csr_capacity(&s) != 2 * 16 * 16) return 2;
  asa_status st = asa_attention_fwd(NULL, NULL, NULL, NULL, ASA_F32, &s, NULL, NULL, 0.0f, NULL);
  if (st != ASA_ERR_NULL_ARG) return 3;
  if (strlen(asa_last_error()) == 0) return 4;
  printf("%s\n", asa_status_string(st));
  return 0;
}
"""


def test_plain_c_client_links_and_calls(tmp_path):
    """The header and the library are usable from plain C (no Python, no GPU work)."""
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(asa.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe),
                    f"-L{libdir}", "-lasa", f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, (res.returncode, res.stderr)
    assert res.stdout.strip() == "ASA_ERR_NULL_ARG"


def test_status_strings():
    assert asa.lib.asa_status_string(0) == b"ASA_OK"
    assert asa.lib.asa_status_string(-5) == b"ASA_ERR_CAPACITY"
    assert asa.lib.asa_version() >= 10700


def test_invalid_shape_left_to_the_builder():
    """For a shape the builders reject, the binding allocates no CSR of its own size: the
    builder call validates the shape first and raises AsaError with its status."""
    rp, ci = asa._alloc_csr(1, 1, 1560, 96, "cpu")
    assert rp.numel() == 1 and ci.numel() == 1
    rp, ci = asa._alloc_csr(1, 2, 1024, 64, "cpu")
    assert rp.numel() == 2 * 16 + 1 and ci.numel() == 2 * 16 * 16
