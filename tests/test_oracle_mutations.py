"""Plant plausible mistakes in the oracle (CPU only) and require a pin to catch each.

This guards the pins themselves: a mistake of the kind listed here (a dropped
term, a wrong scale, a wrong tie-break, an off-by-one, a zero-padded partial
block, a transposed operand) must fail at least one ``check_*`` function.
"""
import numpy as np
import pytest

import oracle
import oracle.asa_oracle as core
from oracle_pins import ALL_CHECKS


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(core, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _pool_sum(X, blk):
    B, H, N, d = X.shape
    Nb = core.num_blocks(N, blk)
    out = np.empty((B, H, Nb, d))
    for r in range(Nb):
        lo, hi = core.block_range(r, N, blk)
        out[:, :, r] = X[:, :, lo:hi].sum(axis=2)
    return out


def _pool_zero_padded(X, blk):
    B, H, N, d = X.shape
    Nb = core.num_blocks(N, blk)
    out = np.empty((B, H, Nb, d))
    for r in range(Nb):
        lo, hi = core.block_range(r, N, blk)
        out[:, :, r] = X[:, :, lo:hi].sum(axis=2) / blk
    return out


def _scores_unscaled(Qp, Kp):
    return np.matmul(Qp, np.swapaxes(Kp, -1, -2))


def _softmax_wrong_axis(S):
    e = np.exp(S - S.max(axis=-2, keepdims=True))
    return e / e.sum(axis=-2, keepdims=True)


def _rank_ties_larger_first(p):
    idx = np.arange(p.shape[0])
    return np.lexsort((-idx, -p))


_orig_count = core.adaptive_count


def _count_off_by_one(p, order, mode, k, tau, k_cap):
    m = _orig_count(p, order, mode, k, tau, k_cap)
    return min(m + 1, p.shape[0]) if mode == core.TAU else m


def _row_attention_noscale(q, k, v):
    s = q @ k.T
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e @ v) / e.sum(axis=1, keepdims=True)


def _kept_tokens_full_blocks_only(mask_row, N, blk):
    parts = [np.arange(c * blk, c * blk + blk) for c in np.nonzero(mask_row)[0]
             if c * blk + blk <= N]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


_orig_static = core.static_row


def _static_floor(pattern, param, r, N, blk):
    if pattern != core.MULTIDIAG:
        return _orig_static(pattern, param, r, N, blk)
    Nb = core.num_blocks(N, blk)
    row = np.zeros(Nb, dtype=bool)
    qlo, qhi = core.block_range(r, N, blk)
    for c in range(Nb):
        klo, khi = core.block_range(c, N, blk)
        lo, hi = klo - (qhi - 1), (khi - 1) - qlo
        row[c] = (lo // param) * param <= hi          # floor instead of ceiling
    return row


def _frame_tile_variant(which):
    def f(pattern, param, r, N, blk):
        if pattern != core.FRAME_TILE:
            return _orig_static(pattern, param, r, N, blk)
        Nb = core.num_blocks(N, blk)
        row = np.zeros(Nb, dtype=bool)
        qlo, qhi = core.block_range(r, N, blk)
        for c in range(Nb):
            klo, khi = core.block_range(c, N, blk)
            if which == "no_first_frame":
                row[c] = klo // param <= (qhi - 1) // param and qlo // param <= (khi - 1) // param
            else:   # frame of the block's end taken as qhi // F (one past the last token)
                row[c] = klo < param or (klo // param <= qhi // param and qlo // param <= khi // param)
        return row
    return f


def _row_attention_no_normalise(q, k, v):
    s = (q @ k.T) / np.sqrt(q.shape[-1])
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e @ v


def _bwd_variant(which):
    def f(q, k, v, g):
        d = q.shape[-1]
        s_ = (q @ k.T) / np.sqrt(d)
        e = np.exp(s_ - s_.max(axis=1, keepdims=True))
        P = e / e.sum(axis=1, keepdims=True)
        dv = (e.T @ g) if which == "dv_unnormalised" else P.T @ g
        dP = g @ v.T
        D = (P * dP).sum(axis=1, keepdims=True)
        ds = P * dP if which == "ds_missing_rowsum" else P * (dP - D)
        dq = (ds @ (v if which == "dq_uses_v" else k)) / np.sqrt(d)
        dk = (ds.T @ q) if which == "dk_missing_scale" else (ds.T @ q) / np.sqrt(d)
        return dq, dk, dv
    return f


_orig_lse = core.attention_lse


def _lse_unscaled(Q, K, M, blk):
    B, H, N, d = Q.shape
    return _orig_lse(Q * np.sqrt(d), K, M, blk)


def _loss_no_penalty(mse, sparsity, lam):
    return mse + 0.0 * lam


def _loss_sparsity_not_density(mse, sparsity, lam):
    return mse + lam * np.asarray(sparsity, dtype=np.float64)[None, :]


def _select_variant(which):
    def f(L, eps):
        H, n = L.shape
        out = np.zeros(H, dtype=np.int64)
        for h in range(H):
            if n == 0:
                continue
            if which == "ge" and np.all(L[h] >= eps):
                continue
            if which != "ge" and np.all(L[h] > eps):
                continue
            if which == "argmax":
                out[h] = 1 + int(np.argmax(L[h]))
            elif which == "last_tie":
                out[h] = n - int(np.argmin(L[h][::-1]))
            else:
                out[h] = 1 + int(np.argmin(L[h]))
        return out
    return f


def _mse_pooled_heads(O_i, O_0):
    diff = O_i - O_0
    return np.full(O_i.shape[1], (diff * diff).mean())


def _mse_sum(O_i, O_0):
    diff = O_i - O_0
    return (diff * diff).sum(axis=(0, 2, 3))


def _sparsity_tile_count(pattern, param, N, blk):
    Nb = core.num_blocks(N, blk)
    kept = sum(int(core.static_row(pattern, param, r, N, blk).sum()) for r in range(Nb))
    return 1.0 - kept / float(Nb * Nb)


def _ambiguous_variant(which):
    def f(S, P, *, mode, k=0, tau=0.0, k_cap=0, gap=core.AMBIGUITY_GAP):
        B, H, Nb, _ = S.shape
        amb = np.zeros((B, H, Nb), dtype=bool)
        if which == "all":
            amb[:] = True
            return amb
        for b in range(B):
            for h in range(H):
                for r in range(Nb):
                    p = P[b, h, r]
                    order = core.rank_order(p)
                    m = core.adaptive_count(p, order, mode, k, tau, k_cap)
                    vals = p if which == "gap_on_p" else S[b, h, r]
                    e = m + 1 if which == "edge_off_by_one" else m
                    flag = False
                    if 0 < e < Nb:
                        flag = abs(vals[order[e - 1]] - vals[order[e]]) < gap
                    if mode == core.TAU and not flag:
                        cs = np.cumsum(p[order])
                        ts = (m - 1, m) if which == "tau_index_off_by_one" else (m - 2, m - 1)
                        for t in ts:
                            if 0 <= t < Nb and abs(cs[t] - tau) < gap:
                                flag = True
                    amb[b, h, r] = flag
        return amb
    return f


def _attention_block_variant(which):
    def f(Q, K, V, M, blk, b, h, r):
        N, d = Q.shape[2], Q.shape[3]
        rr = min(r + 1, core.num_blocks(N, blk) - 1) if which == "next_block_queries" else r
        lo, hi = core.block_range(rr, N, blk)
        J = core.kept_tokens(M[b, h, r], N, blk)
        if J.size == 0:
            return np.zeros((hi - lo, d))
        q = Q[b, h, lo:hi]
        s = (q @ K[b, h, J].T) / (1.0 if which == "no_scale" else np.sqrt(d))
        e = np.exp(s - s.max(axis=1, keepdims=True))
        return (e @ V[b, h, J]) / e.sum(axis=1, keepdims=True)
    return f


def _bwd_terms_variant(which):
    def f(Q, K, V, dO, M, blk):
        B, H, N, d = Q.shape
        Nb = core.num_blocks(N, blk)
        tQ, tK, tV = (np.zeros((B, H, N, d)) for _ in range(3))
        sc = 1.0 if which == "missing_scale" else np.sqrt(d)
        for b in range(B):
            for h in range(H):
                for r in range(Nb):
                    J = core.kept_tokens(M[b, h, r], N, blk)
                    if J.size == 0:
                        continue
                    lo, hi = core.block_range(r, N, blk)
                    q, k, v, g = Q[b, h, lo:hi], K[b, h, J], V[b, h, J], dO[b, h, lo:hi]
                    P, ds = core._row_softmax_and_ds(q, k, v, g)
                    a = ds if which == "signed_ds" else np.abs(ds)
                    tQ[b, h, lo:hi] = (a @ np.abs(v if which == "dq_uses_v" else k)) / sc
                    tK[b, h, J] += (a.T @ np.abs(q)) / sc
                    tV[b, h, J] += P.T @ np.abs(g)
        return tQ, tK, tV
    return f


MUTATIONS = {
    "pool_sum_not_mean": ("pool", _pool_sum),
    "pool_zero_padded_partial_block": ("pool", _pool_zero_padded),
    "block_scores_missing_scale": ("block_scores", _scores_unscaled),
    "block_softmax_wrong_axis": ("block_softmax", _softmax_wrong_axis),
    "rank_ties_larger_index_first": ("rank_order", _rank_ties_larger_first),
    "tau_prefix_off_by_one": ("adaptive_count", _count_off_by_one),
    "attention_missing_scale": ("_row_attention", _row_attention_noscale),
    "attention_drops_partial_key_block": ("kept_tokens", _kept_tokens_full_blocks_only),
    "multidiag_floor_not_ceiling": ("static_row", _static_floor),
    "frame_tile_without_first_frame": ("static_row", _frame_tile_variant("no_first_frame")),
    "frame_tile_end_off_by_one": ("static_row", _frame_tile_variant("end_off_by_one")),
    "attention_not_normalised": ("_row_attention", _row_attention_no_normalise),
    "bwd_dk_missing_scale": ("_row_attention_bwd", _bwd_variant("dk_missing_scale")),
    "bwd_ds_missing_rowsum": ("_row_attention_bwd", _bwd_variant("ds_missing_rowsum")),
    "bwd_dq_uses_v": ("_row_attention_bwd", _bwd_variant("dq_uses_v")),
    "bwd_dv_unnormalised": ("_row_attention_bwd", _bwd_variant("dv_unnormalised")),
    "lse_missing_scale": ("attention_lse", _lse_unscaled),
    "search_loss_missing_penalty": ("pattern_loss", _loss_no_penalty),
    "search_loss_sparsity_for_density": ("pattern_loss", _loss_sparsity_not_density),
    "search_full_when_all_ge_eps": ("select_patterns", _select_variant("ge")),
    "search_argmax": ("select_patterns", _select_variant("argmax")),
    "search_last_index_on_ties": ("select_patterns", _select_variant("last_tie")),
    "search_mse_pooled_over_heads": ("pattern_mse", _mse_pooled_heads),
    "search_mse_sum_not_mean": ("pattern_mse", _mse_sum),
    "search_sparsity_counts_tiles": ("pattern_sparsity", _sparsity_tile_count),
    "near_tie_gap_on_p_not_s": ("ambiguous_rows", _ambiguous_variant("gap_on_p")),
    "near_tie_edge_off_by_one": ("ambiguous_rows", _ambiguous_variant("edge_off_by_one")),
    "near_tie_tau_prefix_off_by_one": ("ambiguous_rows", _ambiguous_variant("tau_index_off_by_one")),
    "near_tie_every_row_flagged": ("ambiguous_rows", _ambiguous_variant("all")),
    "attention_block_next_block_queries": ("attention_block", _attention_block_variant("next_block_queries")),
    "attention_block_missing_scale": ("attention_block", _attention_block_variant("no_scale")),
    "bwd_terms_signed_ds": ("attention_bwd_terms", _bwd_terms_variant("signed_ds")),
    "bwd_terms_dq_uses_v": ("attention_bwd_terms", _bwd_terms_variant("dq_uses_v")),
    "bwd_terms_missing_scale": ("attention_bwd_terms", _bwd_terms_variant("missing_scale")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    _patch(monkeypatch, attr, fn)
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"planted mistake {name} went unnoticed by every pin"
