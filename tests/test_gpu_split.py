"""GPU parity of the split-row forward (asa_attention_fwd_split) against the float64 oracle.

Rows keeping more than T key blocks are cut into chunks whose partial softmax states are
merged afterwards; the result must meet the forward's own bound against oracle.attention
(bf16 inputs: 2e-2 max / 2e-3 mean absolute error, fp32 inputs: 1e-4 max).  Rows of at
most T blocks take the unsplit code path and must equal asa_attention_fwd bit for bit;
skipped heads and empty rows must be exact zeros; lse must match oracle.attention_lse
within the backward's bound.  The GPU always runs on the oracle's own mask.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import compare_outputs, csr_to_device, oracle_inputs, say, to_device

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 2.0 ** -8 + 1e-4


def _oracle_mask(cfg, q64, k64):
    if cfg.kind == "static":
        return O.static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns())
    return O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, tau=cfg.tau, k_cap=cfg.k_cap,
                        n_text=cfg.n_text, keep_diag=cfg.keep_diag, patterns=cfg.patterns)


def _cases():
    dense = gen.Config(name="split_dense_ragged", seed=21, B=1, H=2, N=1000, d=128, blk=128, dtype="bf16",
                       frames=1, Hs=20, Ws=50, structure="smooth", kind="static",
                       patterns=[(gen.FULL, 0), (gen.FULL, 0)])
    cog = replace(gen.scaled(gen.COGVIDEOX, H=3, frames=2), name="split_text_rows")   # text rows keep all blocks
    cog.k_cap = 4
    st = replace(gen.scaled(gen.STATIC, frames=2), name="split_static_skip")          # full / skip / diag / ...
    f32 = gen.Config(name="split_f32_blk64", seed=22, B=2, H=2, N=700, d=64, blk=64, dtype="f32",
                     frames=1, Hs=20, Ws=35, structure="lowrank", kind="adaptive", mode=gen.TOPK, k=5)
    return [(dense, 2), (cog, 3), (st, 1), (f32, 2)]


@pytest.mark.parametrize("cfg,T", _cases(), ids=lambda c: c.name if hasattr(c, "name") else f"T{c}")
def test_split_against_oracle(asa_lib, cfg, T):
    asa = asa_lib
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M = _oracle_mask(cfg, q64, k64)
    counts = M.sum(axis=-1)
    say(f"case {cfg.name}: split T={T}, B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} blk={cfg.blk}, "
        f"row lengths {int(counts.min())}..{int(counts.max())}, split rows {int((counts > T).sum())}")
    assert (counts > T).any(), "the case must split some rows"
    rp, ci = csr_to_device(M)
    pats = cfg.patterns if cfg.kind == "adaptive" else cfg.head_patterns()
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda:0")
    o = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, split_blocks=T, patterns=pats,
                                    lse=lse)
    o_plain = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, patterns=pats)
    torch.cuda.synchronize()
    Meff = M.copy()
    if pats is not None:
        for h, (pid, _) in enumerate(pats):
            if pid == O.SKIP:
                Meff[:, h] = False
    want = O.attention(q64, k64, v64, Meff, cfg.blk)
    got = o.cpu().numpy()
    compare_outputs(got, want, cfg.dtype == "f32", cfg.name)
    # rows short enough to stay whole run the plain kernel's code: bit-identical
    plain = o_plain.cpu().numpy()
    Nb = cfg.Nb
    for b in range(cfg.B):
        for h in range(cfg.H):
            for r in range(Nb):
                lo, hi = O.block_range(r, cfg.N, cfg.blk)
                if Meff[b, h, r].sum() <= T:
                    assert np.array_equal(got[b, h, lo:hi], plain[b, h, lo:hi]), (b, h, r)
    assert np.all(got[~Meff.any(axis=-1).repeat(cfg.blk, axis=-1)[..., :cfg.N]] == 0.0)
    L = O.attention_lse(q64, k64, Meff, cfg.blk)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L)
    assert np.array_equal(np.isneginf(lg), ~fin)
    err = float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0
    say(f"  [lse] max abs err {err:.3e}")
    assert err <= LSE_MAX_ABS


def test_split_bf16_output_and_order(asa_lib):
    """bf16 O through the combine; a schedule from the mask builder changes nothing."""
    asa = asa_lib
    cfg = replace(gen.scaled(gen.COGVIDEOX, H=2, frames=2), name="split_order")
    cfg.k_cap = 4
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    rp, ci, order = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                                       k_cap=cfg.k_cap, n_text=cfg.n_text, keep_diag=cfg.keep_diag,
                                       with_order=True)
    a = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, split_blocks=2)
    b = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, split_blocks=2, order=order)
    c = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, split_blocks=2,
                                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "outputs depend on the processing order"
    # the bf16 output is the fp32 result rounded to nearest even
    assert torch.equal(c, a.to(torch.bfloat16))


def test_split_auto_full_size_dense_head(asa_lib):
    """One Wan-sized head attended in full (B=1, H=1, N=32760, d=128): 256 rows of 256
    blocks, too few rows to fill the chip.  The automatic plan splits them; sampled rows,
    including the ragged last block, against the oracle."""
    asa = asa_lib
    cfg = replace(gen.WAN, name="split_dense_head", H=1, kind="static", patterns=[(gen.FULL, 0)])
    x = gen.make_inputs(replace(cfg, patterns=None, kind="adaptive"))
    xd = to_device(x)
    rp, ci = asa.asa_static_mask(1, 1, cfg.N, cfg.blk, [(gen.FULL, 0)], "cuda:0")
    shp = asa.asa_shape(1, 1, cfg.N, cfg.d, cfg.blk, asa.ASA_BF16)
    import ctypes
    assert asa.lib.asa_attention_fwd_split_workspace_size(ctypes.byref(shp), 0) > 0, "auto plan must split"
    o = asa.asa_attention_fwd_split(xd["q"], xd["k"], xd["v"], rp, ci, cfg.blk, split_blocks=0)
    torch.cuda.synchronize()
    q64, k64, v64 = oracle_inputs(x)
    M = np.ones((1, 1, cfg.Nb, cfg.Nb), dtype=bool)
    rng = np.random.default_rng(31)
    rows = [(0, 0, int(i)) for i in rng.integers(0, cfg.N, 12)] + [(0, 0, cfg.N - 1), (0, 0, 0)]
    want = O.attention_rows(q64, k64, v64, M, cfg.blk, rows)
    got = np.stack([o[b, h, i].cpu().numpy() for b, h, i in rows])
    err = np.abs(got - want)
    say(f"  sampled rows: max abs err {err.max():.3e}")
    assert float(err.max()) <= 2e-2
