"""Static checks on the generated gfx950 assembly of the attention kernels, forward and
backward (CPU only).

The attention kernel issues its global -> LDS transfers from small inline-asm blocks.
The compiler does not see inside them, so they must not touch state it relies on:
  * only the whitelisted instructions appear inside asm blocks;
  * nothing in them writes SCC (an s_add into M0 once corrupted a later s_cselect);
  * M0 is written only inside those blocks (the compiler never reads a value it set);
  * no 64-bit base pointer is rebuilt with a sign-extending s_bfe_i64.
"""
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "block_sparse_attention_asa_amd", "csrc", f) for f in ("attn_fwd.hip", "attn_bwd.hip")]
HIPCC = "/opt/rocm/bin/hipcc"


def _build_module():
    """The library's build script, loaded by path (importing the package needs the built
    library), so that the checked assembly comes from the flags the library ships with."""
    spec = importlib.util.spec_from_file_location(
        "_asa_build_flags", os.path.join(ROOT, "block_sparse_attention_asa_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


ALLOWED = {"s_mov_b32", "s_nop", "global_load_lds_dwordx4", "v_max3_f32"}


@pytest.fixture(scope="module", params=SRCS, ids=lambda p: os.path.basename(p))
def asm_text(request, tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / (os.path.basename(request.param) + ".s")
    b = _build_module()
    flags = [f for f in b.COMMON if f != "-fPIC"] + b.EXTRA.get(os.path.basename(request.param), [])
    cmd = [HIPCC, *flags, "-x", "hip", "-S", "--offload-device-only", request.param, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _asm_blocks(text):
    return re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", text, flags=re.S)


def test_inline_asm_blocks_use_whitelisted_instructions(asm_text):
    blocks = _asm_blocks(asm_text)
    assert blocks, "expected inline asm blocks in the attention kernels"
    for b in blocks:
        for line in b.strip().splitlines():
            op = line.strip().split()[0] if line.strip() else ""
            if not op:
                continue
            assert op in ALLOWED, f"unexpected instruction in asm block: {line.strip()}"
            if op == "s_mov_b32":
                assert line.split()[1].rstrip(",") == "m0", line


def test_m0_written_only_by_transfer_blocks(asm_text):
    outside = re.sub(r";;#ASMSTART\n.*?;;#ASMEND", "", asm_text, flags=re.S)
    uses = [l for l in outside.splitlines() if re.search(r"\bm0\b", l) and not l.strip().startswith(";")]
    assert not uses, f"compiler-generated code touches m0: {uses[:3]}"


def test_no_sign_extended_pointer_rebuild(asm_text):
    assert "s_bfe_i64" not in asm_text
