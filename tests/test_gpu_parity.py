"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Masks: CSR bit-exact, except rows the oracle flags as ambiguous (near-tied block
scores), which are logged and checked for validity.  Attention: the GPU runs on the
oracle's own mask, so no oracle input comes from the HIP path; bf16 inputs must stay
within 2e-2 max / 2e-3 mean absolute error of the float64 oracle (fp32 output), fp32
inputs within 1e-4 max absolute error.
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import (compare_masks, compare_outputs, csr_to_device, gpu_csr_rows, oracle_inputs,
                         sample_rows, say, to_device)

pytestmark = pytest.mark.gpu


def _scaled_cases():
    cog = gen.scaled(gen.COGVIDEOX, H=4, frames=3)
    cog.k_cap = 8                       # floor(0.25 * Nb) at this size, so the cap binds
    wan = gen.scaled(gen.WAN, H=2, frames=3)
    wan.k = 4
    l720 = gen.scaled(gen.LONG720, H=3, frames=2)
    l720.k = 6
    l720.patterns = [(gen.MULTIDIAG, 3600), (gen.MULTIDIAG, 3600), (gen.SKIP, 0)]
    return [gen.TINY, cog, wan, l720]


def _oracle_mask(cfg, q64, k64, with_details=False):
    if cfg.kind == "static":
        return O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns()), None
    M, det = O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap,
                          n_text=cfg.n_text, keep_diag=cfg.keep_diag, patterns=cfg.patterns,
                          return_details=True)
    return M, det


def _gpu_mask(asa, cfg, xd):
    if cfg.kind == "static":
        return asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns(), "cuda:0")
    return asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                              k_cap=cfg.k_cap, n_text=cfg.n_text, keep_diag=cfg.keep_diag,
                              patterns=cfg.patterns)


def _check_mask(asa, cfg, x, xd, q64, k64):
    M, det = _oracle_mask(cfg, q64, k64)
    say(f"  mask: {cfg.name} B={cfg.B} H={cfg.H} N={cfg.N} blk={cfg.blk} Nb={cfg.Nb}")
    rp_t, ci_t = _gpu_mask(asa, cfg, xd)
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    amb = None
    if det is not None:
        amb = O.ambiguous_rows(det["S"], det["P"], mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap)
    diff = compare_masks(rp, ci, M, det, amb, cfg.mode, cfg.k, cfg.tau, cfg.k_cap)
    say(f"  mask: {int(rp[-1])} kept tiles, density {O.density(M):.4f}, "
        f"ambiguous rows {int(amb.sum()) if amb is not None else 0}, differing rows {len(diff)}")
    return M


@pytest.mark.parametrize("cfg", _scaled_cases(), ids=lambda c: c.name)
def test_scaled_mask_and_attention(asa_lib, cfg):
    asa = asa_lib
    say(f"case {cfg.name}: generating inputs")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M = _check_mask(asa, cfg, x, xd, q64, k64)
    rp, ci = csr_to_device(M)
    say(f"  attention: {cfg.name}")
    out = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, patterns=cfg.patterns)
    torch.cuda.synchronize()
    want = O.attention(q64, k64, v64, M, cfg.blk)
    compare_outputs(out.cpu().numpy(), want, cfg.dtype == "f32", cfg.name)


def test_static_patterns_full(asa_lib):
    cfg = gen.STATIC
    say(f"case {cfg.name}: generating inputs")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M = _check_mask(asa_lib, cfg, x, xd, q64, k64)
    counts = M.sum(axis=-1)[0]
    assert (counts[0:2] == 1).all() and (counts[2:4] == 8).all() and (counts[4:6] == 2).all()
    assert (counts[6] == cfg.Nb).all() and (counts[7] == 0).all()
    rp_t, ci_t = asa_lib.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns(), "cuda:0")
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp_t, ci_t, cfg.blk, patterns=cfg.patterns)
    torch.cuda.synchronize()
    want = O.attention(q64, k64, v64, M, cfg.blk)
    got = out.cpu().numpy()
    assert np.all(got[0, 7] == 0.0), "skipped head must be exactly zero"
    compare_outputs(got, want, False, cfg.name)


@pytest.mark.parametrize("cfg", [gen.COGVIDEOX, gen.WAN, gen.LONG720], ids=lambda c: c.name)
def test_full_size_mask_and_sampled_attention(asa_lib, cfg):
    """Full-size workloads: whole CSR compared; attention on sampled query tokens."""
    asa = asa_lib
    say(f"case {cfg.name} (full size): generating inputs")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M = _check_mask(asa, cfg, x, xd, q64, k64)
    rp, ci = csr_to_device(M)
    say(f"  attention: {cfg.name}")
    out = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, patterns=cfg.patterns)
    torch.cuda.synchronize()
    rows = sample_rows(cfg, 24, cfg.seed)
    want = O.attention_rows(q64, k64, v64, M, cfg.blk, rows)
    got = out[[r[0] for r in rows], [r[1] for r in rows], [r[2] for r in rows]].cpu().numpy()
    compare_outputs(got, want, False, cfg.name + " sampled")
    if cfg.patterns is not None:
        for h, (pid, _) in enumerate(cfg.patterns):
            if pid == gen.SKIP:
                assert torch.count_nonzero(out[:, h]).item() == 0


def test_dense_reference_run(asa_lib):
    """All-ones (FULL) mask of the same kernel equals dense attention."""
    cfg = gen.scaled(gen.WAN, H=2, frames=2)
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    pats = [(gen.FULL, 0)] * cfg.H
    rp, ci = asa_lib.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, pats, "cuda:0")
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
    torch.cuda.synchronize()
    compare_outputs(out.cpu().numpy(), O.dense_attention(q64, k64, v64), False, "dense")


@pytest.mark.parametrize("N,blk,d", [(1, 64, 64), (129, 128, 128), (100, 128, 128), (128, 128, 64), (640, 64, 128), (1000, 64, 64),
                                     (4097, 128, 128)])
def test_edge_shapes(asa_lib, N, blk, d):
    """One token, a one-token last block, a single partial block, exact multiples, ragged
    tails; adaptive top-k, bf16 and fp32."""
    for dtype in ("bf16", "f32"):
        cfg = gen.Config(name=f"edge_{N}_{blk}_{d}_{dtype}", seed=7, B=2, H=2, N=N, d=d, blk=blk,
                         dtype=dtype, frames=1, Hs=1, Ws=N, structure="none", mode=gen.TOPK, k=2)
        x = gen.make_inputs(cfg)
        xd = to_device(x)
        q64, k64, v64 = oracle_inputs(x)
        M = _check_mask(asa_lib, cfg, x, xd, q64, k64)
        rp, ci = csr_to_device(M)
        out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, blk)
        torch.cuda.synchronize()
        compare_outputs(out.cpu().numpy(), O.attention(q64, k64, v64, M, blk), dtype == "f32", cfg.name)


def test_empty_rows_and_skip_heads_are_zero(asa_lib):
    cfg = gen.Config(name="empty", seed=8, B=1, H=3, N=700, d=64, blk=64, dtype="bf16", frames=1,
                     Hs=1, Ws=700, structure="none")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    # k = 0 without the diagonal: every adaptive row is empty
    rp, ci = asa_lib.asa_build_mask(xd["q"], xd["k"], 64, gen.TOPK, k_top=0, keep_diag=0)
    torch.cuda.synchronize()
    assert int(rp[-1].item()) == 0
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, 64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    # a skip pattern zeroes the head even when its CSR rows are full
    pats = [(gen.FULL, 0), (gen.VSTRIPE, 0), (gen.FULL, 0)]
    rp, ci = asa_lib.asa_static_mask(1, 3, 700, 64, pats, "cuda:0")
    skip = [(gen.FULL, 0), (gen.VSTRIPE, 0), (gen.SKIP, 0)]
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, 64, patterns=skip)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[:, 1:]).item() == 0
    assert torch.count_nonzero(out[:, 0]).item() > 0


def test_bf16_output(asa_lib):
    cfg = gen.scaled(gen.WAN, H=2, frames=2)
    cfg.k = 4
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M, _ = _oracle_mask(cfg, q64, k64)
    rp, ci = csr_to_device(M)
    out = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = O.attention(q64, k64, v64, M, cfg.blk)
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    # fp32-path bound plus half a bf16 ulp of the output magnitude
    bound = 2e-2 + np.abs(want) * 2.0 ** -8
    say(f"  [bf16 out] max abs err {err.max():.3e}")
    assert np.all(err <= bound)


def test_determinism(asa_lib):
    cfg = gen.scaled(gen.COGVIDEOX, H=3, frames=2)
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    outs = []
    for _ in range(2):
        rp, ci = _gpu_mask(asa_lib, cfg, xd)
        o = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
        torch.cuda.synchronize()
        outs.append((rp.cpu(), ci[: int(rp[-1])].cpu(), o.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2])


def test_explicit_stream_and_errors(asa_lib):
    cfg = gen.scaled(gen.WAN, H=1, frames=1)
    cfg.k = 3
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rp, ci = asa_lib.asa_build_mask(xd["q"], xd["k"], cfg.blk, gen.TOPK, k_top=3)
        o1 = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk)
    s.synchronize()
    rp2, ci2 = asa_lib.asa_build_mask(xd["q"], xd["k"], cfg.blk, gen.TOPK, k_top=3)
    o2 = asa_lib.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp2, ci2, cfg.blk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    with pytest.raises(asa_lib.AsaError):
        asa_lib.asa_build_mask(xd["q"], xd["k"], 96, gen.TOPK, k_top=3)
