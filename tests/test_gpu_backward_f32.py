"""GPU parity of the backward for fp32 inputs: asa_attention_fwd_lse + asa_attention_bwd
(fp32 Q, K, V, dO) against the float64 oracle (oracle.attention_bwd) on the oracle's own mask.

The fp32 path keeps P and dS in fp32 and runs every product on the fp32 matrix cores, so the
only error is fp32 rounding: the products' sums (unit roundoff 2^-24 per addition, over at
most a few thousand terms here), the hardware exp2 (about one ulp), and the forward's fp32 O
and lse.  Each gradient element is bounded by two parts:
  * 2^-12 times the sum of the absolute values of its products (oracle.attention_bwd_terms;
    2^-12 = 4096 additions at 2^-24): the rounding of the sums and of the weights;
  * 2^-14 of the gradient's largest magnitude: dP = dO.V and D = dO.O are fp32 dot products
    over d terms, and their rounding enters dS = P (dP - D) as P (err_dP - err_D) whatever
    the size of dS, so it is not proportional to the sums above.  Summed over a row it stays
    about 2^-17 of the gradient's scale (7e-6 measured); the floor leaves a factor of 8.
Inputs carry fp32 noise below the bf16 resolution, so a path that rounded them to bf16
fails the bound.  Exact zeros are required where no kept tile contributes (skipped heads,
empty rows).
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import csr_to_device, say

pytestmark = pytest.mark.gpu

TERMS_REL = 2.0 ** -12
SCALE_REL = 2.0 ** -14
# An lse error delta scales every weight P of its query by exp(-delta), a relative error
# of about delta, which the gradient bound above absorbs up to 2^-12.  The fp32 forward's
# lse carries the rounding of fp32 scores of magnitude up to ~100 (about 4e-5 measured).
LSE_MAX_ABS = 2.0 ** -12


def _f32_inputs(cfg, seed):
    """The config's generated tensors in fp32, plus N(0, 1e-3) noise that bf16 cannot hold."""
    x = gen.make_inputs(cfg)
    rng = np.random.default_rng(9000 + seed)
    out = {}
    for n in ("q", "k", "v"):
        a = x[n].to(torch.float32).numpy()
        out[n] = torch.from_numpy((a + 1e-3 * rng.standard_normal(a.shape)).astype(np.float32))
    return out


def _cases():
    cog = gen.scaled(gen.COGVIDEOX, H=3, frames=2)       # TAU, d=64, text rows and columns
    cog.k_cap = 8
    wan = gen.scaled(gen.WAN, H=2, frames=2)              # TOPK, d=128, ragged last block
    wan.k = 4
    l720 = gen.scaled(gen.LONG720, H=3, frames=1)         # multi-diagonal union and a skipped head
    l720.k = 6
    l720.patterns = [(gen.MULTIDIAG, 3600), (gen.MULTIDIAG, 3600), (gen.SKIP, 0)]
    return [cog, wan, l720]


def _mask(cfg, q64, k64):
    return O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap,
                        n_text=cfg.n_text, keep_diag=cfg.keep_diag, patterns=cfg.patterns)


@pytest.mark.parametrize("cfg", _cases(), ids=lambda c: c.name)
def test_backward_f32(asa_lib, cfg):
    say(f"case {cfg.name}: fp32 backward B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} blk={cfg.blk}")
    x = _f32_inputs(cfg, 1)
    q64, k64 = (x[n].numpy().astype(np.float64) for n in ("q", "k"))
    _check(asa_lib, cfg, x, _mask(cfg, q64, k64), cfg.patterns)


@pytest.mark.parametrize("N,blk,d", [(100, 128, 128), (640, 64, 128), (1000, 64, 64), (700, 128, 64)])
def test_backward_f32_edge_shapes(asa_lib, N, blk, d):
    """Ragged lengths, both block sizes and both head sizes on a random mask with an empty row
    and a ragged last key block kept by every row of one head."""
    cfg = gen.Config(name=f"bwd_f32_edge_{N}_{blk}_{d}", seed=9, B=2, H=2, N=N, d=d, blk=blk, dtype="bf16",
                     frames=1, Hs=1, Ws=N, structure="none", mode=gen.TOPK, k=2)
    say(f"case {cfg.name}: fp32 backward edge shape")
    x = _f32_inputs(cfg, 3)
    Nb = O.num_blocks(N, blk)
    M = np.random.default_rng(177 + N).random((cfg.B, cfg.H, Nb, Nb)) < 0.5
    M[0, 0, 0] = False
    M[0, -1, :, Nb - 1] = True
    _check(asa_lib, cfg, x, M, None)


def _check(asa, cfg, x, M, pats):
    B, H, N, d, blk = cfg.B, cfg.H, cfg.N, cfg.d, cfg.blk
    q64, k64, v64 = (x[n].numpy().astype(np.float64) for n in ("q", "k", "v"))
    Meff = M.copy()
    if pats is not None:
        for h, (pid, _) in enumerate(pats):
            if pid == O.SKIP:
                Meff[:, h] = False
    xd = {n: t.to("cuda:0") for n, t in x.items()}
    rp, ci = csr_to_device(M)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, blk, patterns=pats, lse=lse)
    g = np.random.default_rng(5100).standard_normal((B, H, N, d)).astype(np.float32)
    gd = torch.from_numpy(g).to("cuda:0")
    grads = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, gd, lse, rp, ci, blk, patterns=pats)
    again = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, gd, lse, rp, ci, blk, patterns=pats)
    torch.cuda.synchronize()

    L = O.attention_lse(q64, k64, Meff, blk)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(lg), ~fin), "lse: -inf pattern differs"
    lerr = float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0
    say(f"  [lse] max abs err {lerr:.3e}")
    assert lerr <= LSE_MAX_ABS

    g64 = g.astype(np.float64)
    refs = O.attention_bwd(q64, k64, v64, g64, Meff, blk)
    terms = O.attention_bwd_terms(q64, k64, v64, g64, Meff, blk)
    for got, rep, ref, t, label in zip(grads, again, refs, terms, ("dQ", "dK", "dV")):
        a = got.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), f"{label}: non-finite gradient"
        assert torch.equal(got, rep), f"{label}: two calls differ"
        err = np.abs(a - ref)
        scale = float(np.abs(ref).max())
        bound = TERMS_REL * t + SCALE_REL * scale
        say(f"  [{label}] max abs err {err.max():.3e} (ref max {scale:.3e}, rel {err.max() / max(scale, 1e-30):.2e}); "
            f"mean abs err {err.mean():.3e}; max err / bound {float((err / bound).max()):.3f}")
        assert np.all(err <= bound), f"{label}: {int((err > bound).sum())} elements over the fp32 rounding bound"
        zero = ref == 0.0
        if zero.any():
            assert np.all(a[zero] == 0.0), f"{label}: nonzero gradient where no tile contributes"


def test_backward_f32_schedule_changes_nothing(asa_lib):
    """The dQ pass follows the CSR's row order when one is given; fp32 gradients are
    bit-identical with and without it."""
    asa = asa_lib
    cfg = gen.scaled(gen.WAN, H=2, frames=2)
    cfg.k = 4
    say(f"case {cfg.name}: fp32 backward, with and without the row order")
    x = _f32_inputs(cfg, 2)
    xd = {n: t.to("cuda:0") for n, t in x.items()}
    rp, ci, od = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, asa.TOPK, k_top=cfg.k, keep_diag=1, with_order=True)
    lse = torch.empty(xd["q"].shape[:3], dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, order=od, lse=lse)
    gd = torch.randn(xd["q"].shape, generator=torch.Generator().manual_seed(7)).to("cuda:0")
    a = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, gd, lse, rp, ci, cfg.blk, order=od)
    b = asa.asa_attention_bwd(xd["q"], xd["k"], xd["v"], o, gd, lse, rp, ci, cfg.blk)
    torch.cuda.synchronize()
    for x1, x2, label in zip(a, b, ("dQ", "dK", "dV")):
        assert torch.equal(x1, x2), f"{label} depends on the schedule"
