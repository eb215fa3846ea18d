"""Property tests of the oracle's mask rule and attention on random small shapes (CPU).

Random B, H, N (block multiples and ragged tails), d, blk, k, tau, k_cap and n_text drawn by
hypothesis; the invariants follow from the rule as the builders' header states it
(top-k or shortest tau-prefix of the rank order, capped, plus diagonal and text blocks):
  - the top-k and tau prefixes are nested: a larger k, tau or k_cap never drops a block;
  - the diagonal (keep_diag) and the key blocks holding text tokens are always kept, and a
    query block holding text tokens keeps every block;
  - an adaptive row keeps exactly min(k, Nb) ranked blocks plus the forced ones;
  - the tau prefix is the shortest whose probability mass reaches tau;
  - the CSR form lists each row's kept blocks once, ascending, and counts every kept tile;
  - attention outputs are convex combinations of the kept values (per coordinate between
    their minimum and maximum), and exactly zero for empty rows.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def shapes(draw):
    blk = draw(st.sampled_from([64, 128]))
    nb = draw(st.integers(1, 9))
    tail = draw(st.integers(0, blk - 1)) if nb > 1 else draw(st.integers(0, blk - 1))
    N = max(1, nb * blk - tail)
    B = draw(st.integers(1, 2))
    H = draw(st.integers(1, 3))
    d = draw(st.sampled_from([16, 64]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return B, H, N, d, blk, seed


def _qk(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + 0.5 * q   # some query/key correlation
    return q, k


def _forced(M, N, blk, n_text, keep_diag):
    Nb = M.shape[-1]
    text_blocks = O.num_blocks(n_text, blk) if n_text > 0 else 0
    for r in range(Nb):
        if keep_diag:
            assert M[..., r, r].all(), f"diagonal block {r} dropped"
        if text_blocks:
            assert M[..., r, :text_blocks].all(), "text key blocks dropped"
    if text_blocks:
        assert M[..., :text_blocks, :].all(), "a query block with text tokens is not full"


@SETTINGS
@given(shapes(), st.integers(0, 12), st.integers(0, 1))
def test_topk_nested_forced_and_counted(shape, k, keep_diag):
    B, H, N, d, blk, seed = shape
    q, kk = _qk(B, H, N, d, seed)
    Nb = O.num_blocks(N, blk)
    M1, det = O.build_mask(q, kk, blk, mode=O.TOPK, k=k, keep_diag=keep_diag, return_details=True)
    M2 = O.build_mask(q, kk, blk, mode=O.TOPK, k=k + 1, keep_diag=keep_diag)
    assert M1.shape == (B, H, Nb, Nb) and M1.dtype == bool
    assert np.all(M2 | ~M1), "a larger k dropped a block"
    _forced(M1, N, blk, 0, keep_diag)
    # exactly min(k, Nb) ranked blocks, plus the diagonal when it is not among them
    P = det["P"]
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                top = set(O.rank_order(P[b, h, r])[: min(k, Nb)].tolist())
                want = top | ({r} if keep_diag else set())
                assert set(np.nonzero(M1[b, h, r])[0].tolist()) == want


@SETTINGS
@given(shapes(), st.floats(0.0, 1.0), st.floats(0.0, 1.0), st.integers(0, 6))
def test_tau_prefix_nested_shortest_and_capped(shape, t1, t2, k_cap):
    B, H, N, d, blk, seed = shape
    lo, hi = min(t1, t2), max(t1, t2)
    q, kk = _qk(B, H, N, d, seed)
    Nb = O.num_blocks(N, blk)
    Ma, det = O.build_mask(q, kk, blk, mode=O.TAU, tau=lo, k_cap=k_cap, keep_diag=0, return_details=True)
    Mb = O.build_mask(q, kk, blk, mode=O.TAU, tau=hi, k_cap=k_cap, keep_diag=0)
    assert np.all(Mb | ~Ma), "a larger tau dropped a block"
    if k_cap > 0:
        Mc = O.build_mask(q, kk, blk, mode=O.TAU, tau=lo, k_cap=k_cap + 1, keep_diag=0)
        assert np.all(Mc | ~Ma), "a larger cap dropped a block"
        assert Ma.sum(axis=-1).max() <= k_cap
    P = det["P"]
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                order = O.rank_order(P[b, h, r])
                m = int(Ma[b, h, r].sum())
                assert m >= 1, "a tau prefix is never empty"
                assert set(np.nonzero(Ma[b, h, r])[0].tolist()) == set(order[:m].tolist())
                if k_cap == 0 or m < k_cap:
                    cs = np.cumsum(P[b, h, r][order])
                    # shortest prefix reaching tau (all blocks if none does)
                    if m < Nb:
                        assert cs[m - 1] >= lo
                    if m >= 2:
                        assert cs[m - 2] < lo


@SETTINGS
@given(shapes(), st.integers(1, 300), st.integers(0, 5))
def test_text_tokens_and_csr(shape, n_text, k):
    B, H, N, d, blk, seed = shape
    n_text = min(n_text, N)
    q, kk = _qk(B, H, N, d, seed)
    M = O.build_mask(q, kk, blk, mode=O.TOPK, k=k, n_text=n_text, keep_diag=1)
    _forced(M, N, blk, n_text, 1)
    rp, ci = O.to_csr(M)
    rows = M.reshape(-1, M.shape[-1])
    assert rp[0] == 0 and rp[-1] == M.sum() and len(rp) == rows.shape[0] + 1
    for n in range(rows.shape[0]):
        seg = ci[rp[n]:rp[n + 1]]
        assert np.all(np.diff(seg) > 0), "col_idx not strictly ascending"
        assert np.array_equal(seg, np.nonzero(rows[n])[0])
    assert abs(O.density(M) - M.sum() / M.size) < 1e-15


@SETTINGS
@given(shapes(), st.integers(0, 4), st.integers(0, 1))
def test_attention_is_convex_combination(shape, k, keep_diag):
    B, H, N, d, blk, seed = shape
    q, kk = _qk(B, H, N, d, seed)
    v = np.random.default_rng(seed + 1).standard_normal((B, H, N, d))
    M = O.build_mask(q, kk, blk, mode=O.TOPK, k=k, keep_diag=keep_diag)
    out = O.attention(q, kk, v, M, blk)
    Nb = M.shape[-1]
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                lo_q, hi_q = O.block_range(r, N, blk)
                cols = np.nonzero(M[b, h, r])[0]
                if cols.size == 0:
                    assert np.all(out[b, h, lo_q:hi_q] == 0.0)
                    continue
                keys = np.concatenate([np.arange(*O.block_range(int(c), N, blk)) for c in cols])
                vmin, vmax = v[b, h, keys].min(axis=0), v[b, h, keys].max(axis=0)
                o = out[b, h, lo_q:hi_q]
                assert np.all(o >= vmin - 1e-12) and np.all(o <= vmax + 1e-12)
