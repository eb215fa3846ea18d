"""GPU: whole-output parity for the launch shape the benchmark times.

Launches with d = 128, blk = 128 and at least 768 query-block rows take the kernel
variant that consumes each kept key block in 32-key steps (three workgroups per compute
unit); smaller launches take 64-key steps.  The full-size layers reach the 32-key variant
but are checked on sampled tokens only, so this test runs a Wan-shaped layer with 12 heads
and 6 frames (N = 9360, Nb = 74, 888 rows, about 10 % of tiles kept) and compares the
entire output against the float64 oracle, for every variant of that kernel the ABI can
reach: bf16 inputs with fp32 output, bf16 inputs with bf16 output, fp32 inputs, and the
split-row forward (rows cut into chunks of 3 kept blocks, merged by the combine kernel).
The masked attention is the one of Sparse-vDiT, section 三 "核心公式".
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import compare_outputs, csr_to_device, oracle_inputs, say, to_device

pytestmark = pytest.mark.gpu

ROWS_32KEY = 768


def _layer(dtype):
    cfg = gen.scaled(gen.WAN, H=12, frames=6, name_suffix=f"_888rows_{dtype}")
    cfg.k = 7
    cfg.dtype = dtype
    assert cfg.B * cfg.H * cfg.Nb >= ROWS_32KEY and cfg.d == 128 and cfg.blk == 128
    return cfg


def _oracle(cfg):
    x = gen.make_inputs(cfg)
    q64, k64, v64 = oracle_inputs(x)
    M = O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, keep_diag=cfg.keep_diag)
    say(f"case {cfg.name}: N={cfg.N} Nb={cfg.Nb} rows={cfg.B * cfg.H * cfg.Nb} density {O.density(M):.4f}")
    return x, M, O.attention(q64, k64, v64, M, cfg.blk)


@pytest.fixture(scope="module")
def bf16_case():
    return _oracle(_layer("bf16"))


def test_bf16_in_fp32_out_whole(asa_lib, bf16_case):
    x, M, want = bf16_case
    cfg = _layer("bf16")
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
    torch.cuda.synchronize()
    compare_outputs(out.cpu().numpy(), want, False, "32-key bf16 -> fp32, whole output")


def test_bf16_in_bf16_out_whole(asa_lib, bf16_case):
    x, M, want = bf16_case
    cfg = _layer("bf16")
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, out_dtype=torch.bfloat16)
    ref = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    # the fp32-output bound plus half a bf16 ulp of the output magnitude
    bound = 2e-2 + np.abs(want) * 2.0 ** -8
    say(f"  [32-key bf16 -> bf16, whole output] max abs err {err.max():.3e}")
    assert np.all(np.isfinite(got)) and np.all(err <= bound)
    # the bf16 output is the fp32 output of the same kernel rounded to nearest even
    assert torch.equal(out, ref.to(torch.bfloat16))


def test_fp32_in_whole(asa_lib):
    cfg = _layer("f32")
    x, M, want = _oracle(cfg)
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
    torch.cuda.synchronize()
    compare_outputs(out.cpu().numpy(), want, True, "32-key fp32 inputs, whole output")


def test_split_rows_whole(asa_lib, bf16_case):
    x, M, want = bf16_case
    cfg = _layer("bf16")
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    out = asa_lib.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, split_blocks=3, lse=lse)
    plain = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
    torch.cuda.synchronize()
    compare_outputs(out.cpu().numpy(), want, False, "32-key split (3 blocks per chunk), whole output")
    q64, k64, _ = oracle_inputs(x)
    L = O.attention_lse(q64, k64, M, cfg.blk)
    err = float(np.abs(lse.cpu().numpy().astype(np.float64) - L).max())
    say(f"  [split lse] max abs err {err:.3e}")
    assert err <= 2.0 ** -8 + 1e-4
    # every row keeps more than 3 blocks here, so every row went through the combine
    assert (M.sum(axis=-1) > 3).all()
    say(f"  [split vs plain] max abs diff {float((out - plain).abs().max()):.3e}")
