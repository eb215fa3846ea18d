"""GPU parity of the backward: asa_attention_fwd_lse + asa_attention_bwd against the float64
oracle (oracle.attention_lse, oracle.attention_bwd) on the oracle's own mask.

The GPU runs the whole training path: forward with lse (bf16 inputs, fp32 O), then the
backward on that O and lse.  The oracle computes everything from the same bf16 inputs in
float64.  Tolerances are relative to each gradient's scale:
  max |err| <= GRAD_MAX_REL  * max |ref|   and   mean |err| <= GRAD_MEAN_REL * mean |ref|.
They follow from the arithmetic: P and dS are rounded to bf16 (relative 2^-8) before the
matrix products, whose fp32 sums then carry errors of about 2^-8 relative to their scale.
Exact zeros are required where no kept tile contributes (skipped heads, empty rows).
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import csr_to_device, say, to_device

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 2e-2
GRAD_MEAN_REL = 5e-3
# The forward's normaliser sums the bf16-rounded weights (8 significant bits, so each is off
# by at most 2^-8 relative); the log of that sum is off by at most 2^-8, plus fp32 rounding.
LSE_MAX_ABS = 2.0 ** -8 + 1e-4


def _dout(shape, seed):
    g = np.random.default_rng(5000 + seed).standard_normal(shape).astype(np.float32)
    return torch.from_numpy(g).to(torch.bfloat16)


def _oracle_mask(cfg, q64, k64):
    if cfg.kind == "static":
        return O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns())
    return O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap,
                        n_text=cfg.n_text, keep_diag=cfg.keep_diag, patterns=cfg.patterns)


def _compare_grad(got: torch.Tensor, want: np.ndarray, label: str):
    g = got.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{label}: non-finite gradient"
    err = np.abs(g - want)
    scale_max, scale_mean = float(np.abs(want).max()), float(np.abs(want).mean())
    mx, mean = float(err.max()), float(err.mean())
    say(f"  [{label}] max abs err {mx:.3e} (ref max {scale_max:.3e}, rel {mx / max(scale_max, 1e-30):.2e})  "
        f"mean abs err {mean:.3e} (ref mean {scale_mean:.3e}, rel {mean / max(scale_mean, 1e-30):.2e})")
    assert mx <= GRAD_MAX_REL * scale_max, f"{label}: max abs err {mx} > {GRAD_MAX_REL} * {scale_max}"
    assert mean <= GRAD_MEAN_REL * scale_mean, f"{label}: mean abs err {mean} > {GRAD_MEAN_REL} * {scale_mean}"
    zero = want == 0.0
    if zero.any():
        assert np.all(g[zero] == 0.0), f"{label}: nonzero gradient where no tile contributes"


def _run_case(asa, cfg, x, M, pats, seed):
    B, H, N, d, blk = cfg.B, cfg.H, cfg.N, cfg.d, cfg.blk
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, blk, patterns=pats, lse=lse)
    dout = _dout((B, H, N, d), seed)
    dq, dk, dv = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout.to("cuda:0"), lse, rp, ci, blk,
                                       patterns=pats)
    torch.cuda.synchronize()
    q64, k64, v64 = (gen.as_float64(x[n]) for n in ("q", "k", "v"))
    g64 = dout.to(torch.float64).numpy()
    Meff = M.copy()
    if pats is not None:
        for h, (pid, _) in enumerate(pats):
            if pid == O.SKIP:
                Meff[:, h] = False
    L = O.attention_lse(q64, k64, Meff, blk)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(lg), ~fin), "lse: -inf pattern differs (empty rows / skipped heads)"
    err = float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0
    say(f"  [lse] max abs err {err:.3e}")
    assert err <= LSE_MAX_ABS
    rdq, rdk, rdv = O.attention_bwd(q64, k64, v64, g64, Meff, blk)
    _compare_grad(dq, rdq, "dQ")
    _compare_grad(dk, rdk, "dK")
    _compare_grad(dv, rdv, "dV")
    return dq, dk, dv


def _cases():
    cog = gen.scaled(gen.COGVIDEOX, H=3, frames=2)       # TAU, d=64, text rows and columns
    cog.k_cap = 8
    wan = gen.scaled(gen.WAN, H=2, frames=2)              # TOPK, d=128, ragged last block
    wan.k = 4
    l720 = gen.scaled(gen.LONG720, H=3, frames=1)         # multi-diagonal union and a skipped head
    l720.k = 6
    l720.patterns = [(gen.MULTIDIAG, 3600), (gen.MULTIDIAG, 3600), (gen.SKIP, 0)]
    return [cog, wan, l720]


@pytest.mark.parametrize("cfg", _cases(), ids=lambda c: c.name)
def test_backward_scaled(asa_lib, cfg):
    say(f"case {cfg.name}: backward")
    x = gen.make_inputs(cfg)
    q64, k64 = gen.as_float64(x["q"]), gen.as_float64(x["k"])
    M = _oracle_mask(cfg, q64, k64)
    say(f"  B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} blk={cfg.blk} density {O.density(M):.3f}")
    _run_case(asa_lib, cfg, x, M, cfg.patterns, seed=1)


def test_backward_static_patterns(asa_lib):
    cfg = gen.scaled(gen.STATIC, frames=2)   # full / skip / diagonal / multi-diag / stripes
    say(f"case {cfg.name}: backward N={cfg.N}")
    x = gen.make_inputs(cfg)
    M = _oracle_mask(cfg, None, None)
    _run_case(asa_lib, cfg, x, M, cfg.head_patterns(), seed=2)


@pytest.mark.parametrize("N,blk,d", [(100, 128, 128), (640, 64, 128), (1000, 64, 64), (700, 128, 64)])
def test_backward_edge_shapes(asa_lib, N, blk, d):
    cfg = gen.Config(name=f"bwd_edge_{N}_{blk}_{d}", seed=9, B=2, H=2, N=N, d=d, blk=blk, dtype="bf16",
                     frames=1, Hs=1, Ws=N, structure="none", mode=gen.TOPK, k=2)
    say(f"case {cfg.name}: backward edge shape")
    x = gen.make_inputs(cfg)
    Nb = O.num_blocks(N, blk)
    M = np.random.default_rng(77 + N).random((cfg.B, cfg.H, Nb, Nb)) < 0.5
    M[0, 0, 0] = False                      # an empty row
    M[0, -1, :, Nb - 1] = True              # the ragged last key block is kept everywhere
    _run_case(asa_lib, cfg, x, M, None, seed=3)


def test_backward_deterministic(asa_lib):
    asa = asa_lib
    cfg = gen.scaled(gen.WAN, H=2, frames=1)
    cfg.k = 3
    x = gen.make_inputs(cfg)
    q64, k64 = gen.as_float64(x["q"]), gen.as_float64(x["k"])
    M = _oracle_mask(cfg, q64, k64)
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, lse=lse)
    dout = _dout(tuple(x["q"].shape), 4).to("cuda:0")
    a = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout, lse, rp, ci, cfg.blk)
    b = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout, lse, rp, ci, cfg.blk)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_backward_schedules_change_nothing(asa_lib):
    """The dQ pass in the mask builder's row order, and the dK/dV pass in its own key-block
    order, give the same bits as row order: every gradient element is summed by one lane in
    a fixed order whatever the schedule."""
    asa = asa_lib
    cfg = gen.scaled(gen.COGVIDEOX, H=3, frames=2)   # text rows and popular key blocks: uneven lists
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    rp, ci, order = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                                       k_cap=cfg.k_cap, n_text=cfg.n_text, keep_diag=cfg.keep_diag,
                                       with_order=True)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, order=order, lse=lse)
    dout = _dout(tuple(x["q"].shape), 6).to("cuda:0")
    a = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout, lse, rp, ci, cfg.blk)
    b = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout, lse, rp, ci, cfg.blk, order=order)
    torch.cuda.synchronize()
    say(f"case {cfg.name}: backward with and without the row schedule")
    for name, u, w in zip(("dQ", "dK", "dV"), a, b):
        assert torch.equal(u, w), name


def test_backward_full_size_sampled(asa_lib):
    """Wan-shaped layer at full size (B=1, H=12, N=32760, d=128, top-26): the GPU computes all
    of dQ, dK, dV; the oracle checks sampled query blocks (dQ) and sampled key blocks (dK, dV:
    the sum over every query block that keeps them), including the ragged last blocks."""
    asa = asa_lib
    cfg = gen.WAN
    say(f"case {cfg.name}: full-size backward, sampled")
    x = gen.make_inputs(cfg)
    q64, k64, v64 = (gen.as_float64(x[n]) for n in ("q", "k", "v"))
    M = _oracle_mask(cfg, q64, k64)
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, lse=lse)
    dout = _dout((cfg.B, cfg.H, cfg.N, cfg.d), 6)
    dq, dk, dv = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout.to("cuda:0"), lse, rp, ci, cfg.blk)
    torch.cuda.synchronize()
    g64 = dout.to(torch.float64).numpy()
    dq_h, dk_h, dv_h = (t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    rng = np.random.default_rng(606)
    Nb, N = cfg.Nb, cfg.N
    got_q, ref_q, got_k, ref_k, got_v, ref_v = [], [], [], [], [], []
    for h in (0, 7, 11):
        for r in sorted(set(rng.integers(0, Nb, 2).tolist()) | {Nb - 1}):
            lo, hi = O.block_range(r, N, cfg.blk)
            a, _, _, _ = O.attention_bwd_block(q64, k64, v64, g64, M, cfg.blk, 0, h, r)
            got_q.append(dq_h[0, h, lo:hi])
            ref_q.append(a)
        for c in sorted(set(rng.integers(0, Nb, 2).tolist()) | {Nb - 1}):
            klo, khi = O.block_range(c, N, cfg.blk)
            sk = np.zeros((khi - klo, cfg.d))
            sv = np.zeros((khi - klo, cfg.d))
            for r in np.nonzero(M[0, h, :, c])[0]:
                _, J, bk, bv = O.attention_bwd_block(q64, k64, v64, g64, M, cfg.blk, 0, h, int(r))
                sel = (J >= klo) & (J < khi)
                sk[J[sel] - klo] += bk[sel]
                sv[J[sel] - klo] += bv[sel]
            got_k.append(dk_h[0, h, klo:khi])
            ref_k.append(sk)
            got_v.append(dv_h[0, h, klo:khi])
            ref_v.append(sv)
    _compare_grad(torch.from_numpy(np.concatenate(got_q)), np.concatenate(ref_q), "dQ sampled")
    _compare_grad(torch.from_numpy(np.concatenate(got_k)), np.concatenate(ref_k), "dK sampled")
    _compare_grad(torch.from_numpy(np.concatenate(got_v)), np.concatenate(ref_v), "dV sampled")


def test_backward_full_size_720p_sampled(asa_lib):
    """720p-like layer at full size (B=1, H=24, N=75600, d=128: Nb = 591, last block 80
    tokens; adaptive top-30 unioned with a one-frame multi-diagonal; heads 22-23 skipped):
    the largest mask the builders take in the workloads.  Sampled query blocks (dQ) and key
    blocks (dK, dV) against the oracle; skipped heads must be exactly zero."""
    asa = asa_lib
    cfg = gen.LONG720
    say(f"case {cfg.name}: full-size backward, sampled")
    x = gen.make_inputs(cfg)
    q64, k64, v64 = (gen.as_float64(x[n]) for n in ("q", "k", "v"))
    M = _oracle_mask(cfg, q64, k64)
    Meff = M.copy()
    for h, (pid, _) in enumerate(cfg.patterns):
        if pid == O.SKIP:
            Meff[:, h] = False
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, patterns=cfg.patterns, lse=lse)
    dout = _dout((cfg.B, cfg.H, cfg.N, cfg.d), 8)
    dq, dk, dv = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout.to("cuda:0"), lse, rp, ci, cfg.blk,
                                       patterns=cfg.patterns)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.all(t[:, 22:] == 0), "skipped heads must have zero gradients"
    g64 = dout.to(torch.float64).numpy()
    rng = np.random.default_rng(720)
    Nb, N = cfg.Nb, cfg.N
    got_q, ref_q, got_k, ref_k, got_v, ref_v = [], [], [], [], [], []
    for h in (0, 13, 21):
        dq_h, dk_h, dv_h = (t[0, h].cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
        for r in sorted(set(rng.integers(0, Nb, 2).tolist()) | {Nb - 1}):
            lo, hi = O.block_range(r, N, cfg.blk)
            a, _, _, _ = O.attention_bwd_block(q64, k64, v64, g64, Meff, cfg.blk, 0, h, r)
            got_q.append(dq_h[lo:hi])
            ref_q.append(a)
        for c in sorted(set(rng.integers(0, Nb, 1).tolist()) | {Nb - 1}):
            klo, khi = O.block_range(c, N, cfg.blk)
            sk = np.zeros((khi - klo, cfg.d))
            sv = np.zeros((khi - klo, cfg.d))
            for r in np.nonzero(Meff[0, h, :, c])[0]:
                _, J, bk, bv = O.attention_bwd_block(q64, k64, v64, g64, Meff, cfg.blk, 0, h, int(r))
                sel = (J >= klo) & (J < khi)
                sk[J[sel] - klo] += bk[sel]
                sv[J[sel] - klo] += bv[sel]
            got_k.append(dk_h[klo:khi])
            ref_k.append(sk)
            got_v.append(dv_h[klo:khi])
            ref_v.append(sv)
    _compare_grad(torch.from_numpy(np.concatenate(got_q)), np.concatenate(ref_q), "dQ sampled")
    _compare_grad(torch.from_numpy(np.concatenate(got_k)), np.concatenate(ref_k), "dK sampled")
    _compare_grad(torch.from_numpy(np.concatenate(got_v)), np.concatenate(ref_v), "dV sampled")


@pytest.mark.parametrize("B,H,N,d", [(1, 3, 2000, 128), (2, 3, 4000, 64)])
def test_backward_wide_score_range(asa_lib, B, H, N, d):
    """Scores that climb, fall or stay flat by 90 log2 units across each row's kept blocks
    (the inputs of the softmax-range forward test), through a key component of up to ~180
    shared by neighbouring keys.  P = exp2(S - lse) spans weights near 1 down to underflow.

    The backward gets the oracle's O and lse (rounded to fp32), so only its own rounding is
    measured.  It rounds P and dS to bf16 before the products, so each gradient element may
    be off by 2^-8 times the sum of the absolute values of its products
    (attention_bwd_terms), plus fp32 accumulation.  Each row of dS sums to zero, so with
    large shared key components dQ cancels far below that sum: the relative bound of the
    other backward tests does not apply to dQ here, the elementwise one does."""
    from test_gpu_softmax_range import _inputs as wide_inputs, _mask as spread_mask
    asa = asa_lib
    blk = 128
    x, x64 = wide_inputs(B, H, N, d, seed=81)
    Nb = (N + blk - 1) // blk
    M = spread_mask(B, H, Nb)
    say(f"case wide scores: B={B} H={H} N={N} d={d} rows={B * H * Nb}")
    xd = to_device(x)
    rp, ci = csr_to_device(M)
    o = torch.from_numpy(O.attention(x64["q"], x64["k"], x64["v"], M, blk).astype(np.float32)).to("cuda:0")
    lse = torch.from_numpy(O.attention_lse(x64["q"], x64["k"], M, blk).astype(np.float32)).to("cuda:0")
    dout = _dout((B, H, N, d), 81)
    dq, dk, dv = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, dout.to("cuda:0"), lse, rp, ci, blk)
    torch.cuda.synchronize()
    g64 = dout.to(torch.float64).numpy()
    refs = O.attention_bwd(x64["q"], x64["k"], x64["v"], g64, M, blk)
    terms = O.attention_bwd_terms(x64["q"], x64["k"], x64["v"], g64, M, blk)
    for got, ref, t, label in zip((dq, dk, dv), refs, terms, ("dQ", "dK", "dV")):
        g = got.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g)), label
        err = np.abs(g - ref)
        bound = 2.0 ** -8 * t + 1e-5 * float(np.abs(ref).max())
        say(f"  [{label}, wide scores] max abs err {err.max():.3e} (ref max {np.abs(ref).max():.3e}); "
            f"max err / bound {float((err / bound).max()):.3f}")
        assert np.all(err <= bound), f"{label}: {int((err > bound).sum())} elements over the rounding bound"
