"""GPU: the attention schedule (asa_csr.order) that the mask builders emit.

The pages leave the work order open; the rule here is the one stated in asa.h.  Rows
split into 8 contiguous ranges, one per XCD.  Inside each range they come by length
class (0 for an empty row, else 1 + floor(log2 of the kept count)) descending, ties in
row order.  The test re-derives that rule on the host from the builder's own row_ptr and
requires the device order to match it exactly.  Attention must give bit-identical
outputs with and without the order: it changes when rows run, not what they compute.
"""
import numpy as np
import pytest
import torch

import gen
from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu

N_XCD = 8


def expected_order(row_ptr: np.ndarray) -> np.ndarray:
    counts = np.diff(row_ptr.astype(np.int64))
    rows = counts.size
    per, rem = divmod(rows, N_XCD)
    out = np.empty(rows, dtype=np.int64)
    for x in range(N_XCD):
        lo = x * per + min(x, rem)
        hi = lo + per + (1 if x < rem else 0)
        idx = np.arange(lo, hi)
        cls = np.array([int(c).bit_length() for c in counts[lo:hi]], dtype=np.int64)
        out[lo:hi] = idx[np.lexsort((idx, -cls))]
    return out


def _cases():
    cog = gen.scaled(gen.COGVIDEOX, H=4, frames=3)   # text rows: full length, first in each head
    cog.k_cap = 8
    l720 = gen.scaled(gen.LONG720, H=3, frames=2)    # multi-diagonal union and a skipped head
    l720.k = 6
    l720.patterns = [(gen.MULTIDIAG, 3600), (gen.MULTIDIAG, 3600), (gen.SKIP, 0)]
    return [cog, l720, gen.STATIC]


def _build(asa, cfg, xd):
    if cfg.kind == "static":
        return asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns(), "cuda:0",
                                   with_order=True)
    return asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                              k_cap=cfg.k_cap, n_text=cfg.n_text, keep_diag=cfg.keep_diag,
                              patterns=cfg.patterns, with_order=True)


@pytest.mark.parametrize("cfg", _cases(), ids=lambda c: c.name)
def test_order_follows_rule_and_keeps_outputs(asa_lib, cfg):
    asa = asa_lib
    say(f"case {cfg.name}: schedule")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    rp_t, ci_t, order_t = _build(asa, cfg, xd)
    torch.cuda.synchronize()
    rp = rp_t.cpu().numpy()
    order = order_t.cpu().numpy().astype(np.int64)
    assert np.array_equal(np.sort(order), np.arange(rp.size - 1)), "order is not a permutation"
    exp = expected_order(rp)
    assert np.array_equal(order, exp), f"first mismatch at {int(np.argmax(order != exp))}"
    counts = np.diff(rp)
    say(f"  rows {counts.size}, kept counts {counts.min()}..{counts.max()}, "
        f"classes {sorted(set(int(c).bit_length() for c in counts))}")
    # a builder's CSR arrays do not depend on whether the order is requested
    if cfg.kind == "static":
        rp2, ci2 = asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns(), "cuda:0")
    else:
        rp2, ci2 = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, tau=cfg.tau,
                                      k_cap=cfg.k_cap, n_text=cfg.n_text, keep_diag=cfg.keep_diag,
                                      patterns=cfg.patterns)
    n = int(rp[-1])
    assert torch.equal(rp2, rp_t) and torch.equal(ci2[:n], ci_t[:n])
    pats = cfg.head_patterns() if cfg.kind == "static" else cfg.patterns
    o_plain = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp_t, ci_t, cfg.blk, patterns=pats)
    o_sched = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp_t, ci_t, cfg.blk, patterns=pats,
                                    order=order_t)
    torch.cuda.synchronize()
    assert torch.equal(o_plain, o_sched), "outputs depend on the processing order"


def test_order_argument_checks(asa_lib):
    asa = asa_lib
    cfg = gen.STATIC
    rp, ci = asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns(), "cuda:0")
    x = to_device(gen.make_inputs(cfg))
    bad = torch.zeros(rp.numel() - 2, dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):
        asa.asa_attention_fwd(x["q"], x["k"], x["v"], rp, ci, cfg.blk, order=bad)
    with pytest.raises(ValueError):
        asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, cfg.head_patterns(), "cuda:0",
                            out=(rp, ci, bad))
