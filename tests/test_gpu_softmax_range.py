"""GPU: the online softmax over a wide range of scores.

The forward keeps a running max per query row and moves it lazily, only when a step's max
exceeds it by more than 32 (log2 units), so weights up to 2^32 accumulate between
rescales; the row sums of the bf16 weights run on the matrix cores.  These inputs push
each part of that.  A per-key offset along one direction, seen by every query, makes the
scores of a row climb by about 90 log2 units across its kept blocks (rescales on the way,
weights near 2^32 between them), fall by as much (the first step holds the max, later
weights shrink towards underflow), or stay flat.  Every row keeps 8 key blocks spread over
the sequence, N leaves a partial last block, and the whole output is compared with the
float64 oracle, for the 32-key kernel (888 rows), the 64-key kernel (a small launch) and
d = 64, plus lse for the first.  The masked attention and its softmax are those of
Sparse-vDiT, section 三 "核心公式".
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import compare_outputs, csr_to_device, say

pytestmark = pytest.mark.gpu

SPAN_LOG2 = 90.0   # rise (or fall) of a row's scores across the sequence, log2 units
QDIR = 4.0         # every query's component along the offset direction


def _inputs(B, H, N, d, seed, dtype=torch.bfloat16):
    """Q, K, V as the device dtype; head h rises (h % 3 == 0), falls (1) or stays flat (2)."""
    rng = np.random.default_rng(seed)
    q = (0.5 * rng.standard_normal((B, H, N, d))).astype(np.float32)
    k = (0.5 * rng.standard_normal((B, H, N, d))).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    q[..., 0] = QDIR
    # score offset of key j: QDIR * c_j / sqrt(d) = SPAN_LOG2 * ln 2 * j / N (natural units)
    c = (SPAN_LOG2 * math.log(2.0) * math.sqrt(d) / QDIR) * (np.arange(N, dtype=np.float32) / N)
    for h in range(H):
        k[:, h, :, 0] = (c, c[::-1], np.zeros_like(c))[h % 3]
    t = {n: torch.from_numpy(a).to(dtype) for n, a in (("q", q), ("k", k), ("v", v))}
    return t, {n: a.to(torch.float64).numpy() for n, a in t.items()}


def _mask(B, H, Nb):
    """Each row keeps its diagonal block and 7 more spread over the sequence."""
    M = np.zeros((B, H, Nb, Nb), dtype=bool)
    stride = max(1, Nb // 8)
    for r in range(Nb):
        for t in range(8):
            M[:, :, r, (r + t * stride) % Nb] = True
    return M


def _run(asa, B, H, N, d, blk, seed, expect_rows=None, with_lse=False):
    x, x64 = _inputs(B, H, N, d, seed)
    Nb = (N + blk - 1) // blk
    if expect_rows is not None:
        assert B * H * Nb >= expect_rows
    M = _mask(B, H, Nb)
    want = O.attention(x64["q"], x64["k"], x64["v"], M, blk)
    say(f"case B={B} H={H} N={N} d={d} blk={blk} rows={B * H * Nb} kept per row={int(M[0, 0, 0].sum())}")
    xd = {n: t.to("cuda:0").contiguous() for n, t in x.items()}
    rp, ci = csr_to_device(M)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0") if with_lse else None
    out = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rp, ci, blk, lse=lse)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # every row sees its whole range: the rising heads' scores span the full offset
    for h in range(min(H, 3)):
        kind = ("rising", "falling", "flat")[h]
        compare_outputs(got[:, h::3], want[:, h::3], False, f"{kind} heads, d={d}, whole output")
    compare_outputs(got, want, False, f"all heads, d={d}, whole output")
    if with_lse:
        L = O.attention_lse(x64["q"], x64["k"], M, blk)
        err = float(np.abs(lse.cpu().numpy().astype(np.float64) - L).max())
        say(f"  [lse] max abs err {err:.3e} (|lse| up to {float(np.abs(L).max()):.1f})")
        assert err <= 2.0 ** -8 + 1e-4


def test_wide_scores_32key_kernel(asa_lib):
    # d = 128, blk = 128 and 888 rows: the kernel variant with 32-key steps
    _run(asa_lib, 1, 12, 9360, 128, 128, seed=71, expect_rows=768, with_lse=True)


def test_wide_scores_64key_kernel(asa_lib):
    # a small d = 128 launch: 64-key steps
    _run(asa_lib, 1, 3, 2000, 128, 128, seed=72)


def test_wide_scores_d64(asa_lib):
    _run(asa_lib, 2, 3, 4000, 64, 128, seed=73)
