"""GPU: the attention schedule (asa_csr.order) that the mask builders emit.

The pages leave the work order open; the rule here is the one stated in asa.h.  Positions
split into 8 contiguous ranges, one per XCD.  Rows group by length class (0 for an empty
row, else 1 + floor(log2 of the kept count)); each class, in row order, is cut into 8
consecutive slices, and range x holds slice x of every class, longest class first.  The
s_c mod 8 one-row-larger slices of a class go to the XCDs from a cursor that starts at 0
and advances by s_c mod 8 after each class.  The test re-derives that rule on the host
from the builder's own row_ptr and requires the device order to match it exactly.
Attention must give bit-identical outputs with and without the order: it changes when
rows run, not what they compute.
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
    lo = [x * per + min(x, rem) for x in range(N_XCD)]
    hi = [lo[x] + per + (1 if x < rem else 0) for x in range(N_XCD)]
    cls = np.array([int(c).bit_length() for c in counts], dtype=np.int64)
    out = np.full(rows, -1, dtype=np.int64)
    fill = list(lo)
    cursor = 0
    for c in range(int(cls.max()) if rows else 0, -1, -1):
        members = np.nonzero(cls == c)[0]          # ascending row index
        b, e = divmod(members.size, N_XCD)
        taken = 0
        for x in range(N_XCD):
            size = b + (1 if (x - cursor) % N_XCD < e else 0)
            out[fill[x]:fill[x] + size] = members[taken:taken + size]
            fill[x] += size
            taken += size
        cursor = (cursor + e) % N_XCD
    assert fill == hi
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


@pytest.mark.gpu
def test_csr_and_output_buffer_checks(asa_lib):
    """Caller-supplied CSR and output buffers are checked before anything is launched:
    host tensors, wrong dtypes, a short row_ptr and a mis-shaped output all raise."""
    asa = asa_lib
    cfg = gen.STATIC
    pats = cfg.head_patterns()
    rp, ci = asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, pats, "cuda:0")
    x = to_device(gen.make_inputs(cfg))
    dev = "cuda:0"
    cases = [
        (rp.cpu(), ci),                                              # host row_ptr
        (rp, ci.cpu()),                                              # host col_idx
        (rp.to(torch.int64), ci),                                    # wrong dtype
        (rp, ci.to(torch.int64)),
        (torch.zeros(rp.numel() - 1, dtype=torch.int32, device=dev), ci),   # short row_ptr
    ]
    for out in cases:
        with pytest.raises((ValueError, TypeError)):
            asa.asa_static_mask(cfg.B, cfg.H, cfg.N, cfg.blk, pats, dev, out=out)
        with pytest.raises((ValueError, TypeError)):
            asa.asa_build_mask(x["q"], x["k"], cfg.blk, asa.TOPK, k_top=2, out=out)
    B, H, N, d = x["q"].shape
    for shape in [(B, H, N - 1, d), (B, H, N, d // 2), (B * H * N * d,)]:
        small = torch.empty(shape, dtype=torch.float32, device=dev)
        with pytest.raises(ValueError):
            asa.asa_attention_fwd(x["q"], x["k"], x["v"], rp, ci, cfg.blk, out=small)
        with pytest.raises(ValueError):
            asa.asa_attention_fwd_split(x["q"], x["k"], x["v"], rp, ci, cfg.blk, out=small)
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_order_rule_with_long_runs(asa_lib):
    """More than 1023 x 1024 rows: each of the builder's threads owns a run of 1024 rows or
    more, past the packed per-class counters, so the order takes the one-counter-per-class
    path.  A static mask (no Q or K needed) with four row-length classes."""
    asa = asa_lib
    B, H, blk = 4, 256, 128
    N = 1024 * blk                                    # Nb = 1024: 4 * 256 * 1024 rows
    cycle = [(gen.DIAG, 0), (gen.VSTRIPE, 3), (gen.MULTIDIAG, 16 * blk), (gen.SKIP, 0)]
    pats = [cycle[h % len(cycle)] for h in range(H)]
    say(f"case long runs: B={B} H={H} Nb={N // blk} rows {B * H * (N // blk)}")
    rp_t, ci_t, order_t = asa.asa_static_mask(B, H, N, blk, pats, "cuda:0", with_order=True)
    torch.cuda.synchronize()
    rp = rp_t.cpu().numpy()
    order = order_t.cpu().numpy().astype(np.int64)
    del ci_t
    torch.cuda.empty_cache()
    assert rp.size - 1 > 1023 * 1024
    counts = np.diff(rp.astype(np.int64))
    assert len(set(int(c).bit_length() for c in np.unique(counts))) >= 3
    exp = expected_order(rp)
    assert np.array_equal(order, exp), f"first mismatch at {int(np.argmax(order != exp))}"
