"""Pins for the float64 oracle: closed forms, library routines and brute force.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
something fixed independently of it.  ``test_oracle_pins.py`` runs them on the
oracle as written; ``test_oracle_mutations.py`` plants plausible mistakes in the
oracle (on the CPU) and confirms that at least one check catches each.
"""
import itertools
import math

import numpy as np
import scipy.special
import torch

import oracle as O

RNG = np.random.default_rng


def _qkv(B, H, N, d, seed, scale=1.0):
    rng = RNG(seed)
    return tuple(rng.standard_normal((B, H, N, d)) * scale for _ in range(3))


def _sdpa(q, k, v):
    """torch scaled_dot_product_attention in float64 on the CPU (library routine)."""
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t).numpy()


# ------------------------------------------------------------------ attention pins
def check_dense_equals_sdpa():
    """All-ones block mask == full attention (torch SDPA, float64), ragged N."""
    q, k, v = _qkv(1, 2, 200, 16, 11)
    M = np.ones((1, 2, O.num_blocks(200, 64), O.num_blocks(200, 64)), dtype=bool)
    ref = _sdpa(q, k, v)
    assert np.allclose(O.attention(q, k, v, M, 64), ref, atol=1e-12, rtol=0)
    assert np.allclose(O.dense_attention(q, k, v), ref, atol=1e-12, rtol=0)


def check_block_diagonal_equals_independent_blocks():
    """Diagonal-only mask == attention run separately inside each block."""
    N, blk = 150, 32
    q, k, v = _qkv(1, 3, N, 8, 12)
    M = O.static_mask(1, 3, N, blk, [(O.DIAG, 0)] * 3)
    out = O.attention(q, k, v, M, blk)
    for r in range(O.num_blocks(N, blk)):
        lo, hi = O.block_range(r, N, blk)
        ref = _sdpa(q[:, :, lo:hi], k[:, :, lo:hi], v[:, :, lo:hi])
        assert np.allclose(out[:, :, lo:hi], ref, atol=1e-12, rtol=0)


def check_weights_sum_to_one():
    """With V = 1 every non-empty output row is exactly 1 (weights sum to 1)."""
    N, blk, d = 300, 64, 16
    rng = RNG(13)
    q = rng.standard_normal((1, 2, N, d)) * 3
    k = rng.standard_normal((1, 2, N, d)) * 3
    v = np.ones((1, 2, N, d))
    Nb = O.num_blocks(N, blk)
    M = rng.random((1, 2, Nb, Nb)) < 0.5
    M[0, 0, 1, :] = False                                   # one empty row
    out = O.attention(q, k, v, M, blk)
    for h in range(2):
        for r in range(Nb):
            lo, hi = O.block_range(r, N, blk)
            want = 1.0 if M[0, h, r].any() else 0.0
            assert np.allclose(out[0, h, lo:hi], want, atol=1e-12, rtol=0)


def check_identical_keys_give_mean_of_v():
    """One kept key block whose keys are identical => uniform weights => mean(V_block)."""
    N, blk, d = 256, 64, 16
    rng = RNG(14)
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    Nb = O.num_blocks(N, blk)
    for c in range(Nb):
        lo, hi = O.block_range(c, N, blk)
        k[0, 0, lo:hi] = rng.standard_normal(d)             # all keys of block c equal
    M = np.zeros((1, 1, Nb, Nb), dtype=bool)
    pick = [(r * 3 + 1) % Nb for r in range(Nb)]
    for r in range(Nb):
        M[0, 0, r, pick[r]] = True
    out = O.attention(q, k, v, M, blk)
    for r in range(Nb):
        lo, hi = O.block_range(r, N, blk)
        klo, khi = O.block_range(pick[r], N, blk)
        assert np.allclose(out[0, 0, lo:hi], v[0, 0, klo:khi].mean(axis=0), atol=1e-12, rtol=0)


def check_bruteforce_2head_n128():
    """2 heads, N=128, ragged blocks (48, 48, 32): pure-Python loops with math.exp."""
    N, blk, d, H = 128, 48, 8, 2
    rng = RNG(15)
    q, k, v = (rng.standard_normal((1, H, N, d)) for _ in range(3))
    Nb = O.num_blocks(N, blk)
    M = rng.random((1, H, Nb, Nb)) < 0.6
    M[0, 1, 2, :] = False
    out = O.attention(q, k, v, M, blk)
    for h in range(H):
        for i in range(N):
            r = i // blk
            js = [j for j in range(N) if M[0, h, r, j // blk]]
            if not js:
                assert all(out[0, h, i, t] == 0.0 for t in range(d))
                continue
            s = [sum(q[0, h, i, t] * k[0, h, j, t] for t in range(d)) / math.sqrt(d) for j in js]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            z = sum(w)
            for t in range(d):
                o = sum(w[n] * v[0, h, js[n], t] for n in range(len(js))) / z
                assert abs(o - out[0, h, i, t]) < 1e-12


def check_skip_and_empty_rows_are_zero():
    N, blk = 256, 64
    q, k, v = _qkv(1, 2, N, 8, 16)
    M = O.static_mask(1, 2, N, blk, [(O.SKIP, 0), (O.FULL, 0)])
    out = O.attention(q, k, v, M, blk)
    assert np.all(out[0, 0] == 0.0)
    assert np.allclose(out[0, 1], _sdpa(q[:, 1:2], k[:, 1:2], v[:, 1:2])[0, 0], atol=1e-12)


def check_attention_rows_match_full():
    N, blk = 200, 64
    q, k, v = _qkv(1, 2, N, 8, 17)
    Nb = O.num_blocks(N, blk)
    M = RNG(17).random((1, 2, Nb, Nb)) < 0.5
    full = O.attention(q, k, v, M, blk)
    rows = [(0, h, i) for h in range(2) for i in (0, 63, 64, 150, 199)]
    got = O.attention_rows(q, k, v, M, blk, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.allclose(got[n], full[b, h, i], atol=1e-13, rtol=0)


# ------------------------------------------------------------------ mask-rule pins
def check_pool_score_bilinearity():
    """S[r,c] == mean over token pairs (i in T_r, j in T_c) of q_i.k_j / sqrt(d)."""
    N, blk, d = 70, 16, 5                                   # last block has 6 tokens
    rng = RNG(21)
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d)) + 0.5
    S = O.block_scores(O.pool(q, blk), O.pool(k, blk))
    Nb = O.num_blocks(N, blk)
    for r in range(Nb):
        for c in range(Nb):
            tot, cnt = 0.0, 0
            for i in range(*O.block_range(r, N, blk)):
                for j in range(*O.block_range(c, N, blk)):
                    tot += sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) / math.sqrt(d)
                    cnt += 1
            assert abs(S[0, 0, r, c] - tot / cnt) < 1e-12


def check_block_softmax_matches_scipy():
    S = RNG(22).standard_normal((2, 3, 7, 7)) * 5
    assert np.allclose(O.block_softmax(S), scipy.special.softmax(S, axis=-1), atol=1e-15, rtol=1e-13)


def check_rank_order_ties():
    p = np.array([0.1, 0.3, 0.1, 0.3, 0.2])
    assert list(O.rank_order(p)) == [1, 3, 4, 0, 2]


def _subset_masses(p):
    Nb = len(p)
    for m in range(Nb + 1):
        for sub in itertools.combinations(range(Nb), m):
            yield m, sub, sum(p[list(sub)]) if sub else 0.0


def check_selection_bruteforce():
    """Top-k and tau-prefix against exhaustive subset enumeration (Nb <= 8)."""
    rng = RNG(23)
    for trial in range(40):
        Nb = int(rng.integers(1, 9))
        p = scipy.special.softmax(rng.standard_normal(Nb) * 2)
        for k in range(0, Nb + 2):
            got = set(O.adaptive_set(p, O.TOPK, k, 0.0, 0).tolist())
            kk = min(k, Nb)
            best = max((s for m, s, w in _subset_masses(p) if m == kk),
                       key=lambda s: sum(p[list(s)]) if s else 0.0)
            assert got == set(best)
        for tau in (0.05, 0.3, 0.5, 0.75, 0.9, 0.99):
            got = O.adaptive_set(p, O.TAU, 0, tau, 0)
            feasible = [(m, s, w) for m, s, w in _subset_masses(p) if w >= tau]
            mmin = min(m for m, s, w in feasible)
            assert len(got) == mmin
            best_w = max(w for m, s, w in feasible if m == mmin)
            assert abs(sum(p[got]) - best_w) < 1e-12
            for cap in (1, 2, 3):
                capped = O.adaptive_set(p, O.TAU, 0, tau, cap)
                assert len(capped) == min(mmin, cap)
                # the capped prefix is the top-`len` set
                assert set(capped.tolist()) == set(O.adaptive_set(p, O.TOPK, len(capped), 0, 0).tolist())


def check_selection_limits_and_monotone():
    rng = RNG(24)
    for trial in range(20):
        Nb = int(rng.integers(2, 40))
        p = scipy.special.softmax(rng.standard_normal(Nb) * 3)
        assert len(O.adaptive_set(p, O.TOPK, Nb, 0, 0)) == Nb
        assert len(O.adaptive_set(p, O.TOPK, Nb + 5, 0, 0)) == Nb
        assert len(O.adaptive_set(p, O.TAU, 0, 1.0 + 1e-9, 0)) == Nb
        prev = set()
        for k in range(Nb + 1):
            cur = set(O.adaptive_set(p, O.TOPK, k, 0, 0).tolist())
            assert prev <= cur and len(cur) == k
            prev = cur
        prev = set()
        for tau in np.linspace(0.01, 1.0, 30):
            cur = set(O.adaptive_set(p, O.TAU, 0, float(tau), 0).tolist())
            assert prev <= cur
            prev = cur


def check_forced_blocks():
    """Diagonal kept, text key blocks kept, text query rows full, skip head empty."""
    N, blk, n_text = 600, 64, 100                            # text spans blocks 0 and 1
    rng = RNG(25)
    q = rng.standard_normal((1, 3, N, 8))
    k = rng.standard_normal((1, 3, N, 8))
    M = O.build_mask(q, k, blk, mode=O.TOPK, k=1, n_text=n_text, keep_diag=1,
                     patterns=[(O.ADAPTIVE, 0), (O.VSTRIPE, 4), (O.SKIP, 0)])
    Nb = O.num_blocks(N, blk)
    for h in range(2):
        assert M[0, h, 0].all() and M[0, h, 1].all()         # text rows
        for r in range(Nb):
            assert M[0, h, r, r] and M[0, h, r, 0] and M[0, h, r, 1]
    assert M[0, 1, :, :4].all()                              # static stripe unioned
    assert not M[0, 2].any()
    # rows outside text keep exactly top-1 U diag U text columns (U stripe)
    M0 = O.build_mask(q, k, blk, mode=O.TOPK, k=1, n_text=0, keep_diag=0)
    assert (M0.sum(axis=-1) == 1).all()


def check_static_patterns_token_pairs():
    """Closed-form static rows vs token-pair enumeration, ragged and strided cases."""
    for N, blk in ((300, 32), (256, 64), (130, 16)):
        Nb = O.num_blocks(N, blk)
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        for S in (1, 5, 16, 32, 48, 100, 128, 1000):
            tok = ((j - i) % S) == 0
            for r in range(Nb):
                ql, qh = O.block_range(r, N, blk)
                want = np.array([tok[ql:qh, slice(*O.block_range(c, N, blk))].any()
                                 for c in range(Nb)])
                assert np.array_equal(O.static_row(O.MULTIDIAG, S, r, N, blk), want), (N, blk, S, r)
        tokd = (i == j)
        for r in range(Nb):
            ql, qh = O.block_range(r, N, blk)
            want = np.array([tokd[ql:qh, slice(*O.block_range(c, N, blk))].any() for c in range(Nb)])
            assert np.array_equal(O.static_row(O.DIAG, 0, r, N, blk), want)
            assert np.array_equal(O.static_row(O.MULTIDIAG, N + 7, r, N, blk), want)
            assert O.static_row(O.VSTRIPE, Nb, r, N, blk).all()
            assert O.static_row(O.FULL, 0, r, N, blk).all()
            assert not O.static_row(O.SKIP, 0, r, N, blk).any()
            s2 = O.static_row(O.VSTRIPE, 2, r, N, blk)
            assert s2[:2].all() and not s2[2:].any()


def check_frame_tile_token_pairs():
    """Frame tiles (own frame + first frame) against token-pair enumeration, ragged blocks,
    frame lengths that are and are not block multiples; F >= N is full attention and F = 1
    is the diagonal plus the first key block."""
    for N, blk in ((300, 32), (256, 64), (130, 16)):
        Nb = O.num_blocks(N, blk)
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        for F in (1, 5, 32, 48, 100, 128):
            tok = ((j // F) == (i // F)) | ((j // F) == 0)
            for r in range(Nb):
                ql, qh = O.block_range(r, N, blk)
                want = np.array([tok[ql:qh, slice(*O.block_range(c, N, blk))].any() for c in range(Nb)])
                assert np.array_equal(O.static_row(O.FRAME_TILE, F, r, N, blk), want), (N, blk, F, r)
        for r in range(Nb):
            assert O.static_row(O.FRAME_TILE, N, r, N, blk).all()
            d1 = O.static_row(O.FRAME_TILE, 1, r, N, blk)
            assert np.array_equal(d1, O.static_row(O.DIAG, 0, r, N, blk) | O.static_row(O.VSTRIPE, 1, r, N, blk))
    # frames of 1024 tokens at N = 8192, blk 128: 8 blocks per frame, rows of frame f > 0
    # keep their own 8 blocks and frame 0's 8
    M = O.static_mask(1, 1, 8192, 128, [(O.FRAME_TILE, 1024)])
    counts = M.sum(axis=-1)[0, 0]
    assert (counts[:8] == 8).all() and (counts[8:] == 16).all()
    assert abs(O.pattern_sparsity(O.FRAME_TILE, 1024, 8192, 128) - (1 - (8 * 1024 + 56 * 16 * 128) * 128 / 8192 ** 2)) < 1e-15


def check_static_counts_8192():
    """Frame-stride multi-diagonal at N=8192, blk=128: 8 tiles per row; stripe 2; diag 1."""
    pats = [(O.DIAG, 0), (O.MULTIDIAG, 1024), (O.VSTRIPE, 2), (O.FULL, 0), (O.SKIP, 0)]
    M = O.static_mask(1, 5, 8192, 128, pats)
    counts = M.sum(axis=-1)[0]
    assert (counts[0] == 1).all() and (counts[1] == 8).all() and (counts[2] == 2).all()
    assert (counts[3] == 64).all() and (counts[4] == 0).all()


def check_csr_layout():
    rng = RNG(26)
    M = rng.random((2, 3, 9, 9)) < 0.3
    row_ptr, col_idx = O.to_csr(M)
    rows = M.reshape(-1, 9)
    assert row_ptr[0] == 0 and len(row_ptr) == rows.shape[0] + 1
    for n in range(rows.shape[0]):
        cols = col_idx[row_ptr[n]:row_ptr[n + 1]]
        assert list(cols) == [c for c in range(9) if rows[n, c]]


def check_kept_tile_flops():
    N, blk, d = 100, 32, 4
    Nb = O.num_blocks(N, blk)
    M = RNG(27).random((1, 1, Nb, Nb)) < 0.5
    pairs = sum(1 for i in range(N) for j in range(N) if M[0, 0, i // blk, j // blk])
    assert O.kept_tile_flops(M, N, blk, d) == 4.0 * pairs * d


# ------------------------------------------------------------------ backward pins
def _token_mask(M, N, blk):
    """Block mask [B,H,Nb,Nb] -> token mask [B,H,N,N] (True = the pair is attended)."""
    idx = np.arange(N) // blk
    return M[:, :, idx][:, :, :, idx]


def _masked_loss(q, k, v, M, blk, g):
    return float((O.attention(q, k, v, M, blk) * g).sum())


def check_bwd_finite_differences():
    """dQ, dK, dV against central differences of sum(G * O) (ragged N, an empty row)."""
    B, H, N, d, blk = 1, 2, 40, 8, 16
    q, k, v = _qkv(B, H, N, d, 31)
    g = RNG(32).standard_normal((B, H, N, d))
    Nb = O.num_blocks(N, blk)
    M = RNG(33).random((B, H, Nb, Nb)) < 0.6
    M[0, 0, 0] = [True, False, True]
    M[0, 1, 1] = False                      # a query block with no kept key block
    dq, dk, dv = O.attention_bwd(q, k, v, g, M, blk)
    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _masked_loss(q, k, v, M, blk, g)
            x[i] = old - eps
            lm = _masked_loss(q, k, v, M, blk, g)
            x[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        assert np.allclose(grad, fd, atol=1e-7, rtol=1e-6), (name, np.abs(grad - fd).max())


def check_bwd_matches_torch_autograd():
    """Gradients of torch SDPA (float64, token-level boolean mask) through autograd."""
    B, H, N, d, blk = 1, 3, 200, 16, 64
    q, k, v = _qkv(B, H, N, d, 34)
    g = RNG(35).standard_normal((B, H, N, d))
    Nb = O.num_blocks(N, blk)
    M = RNG(36).random((B, H, Nb, Nb)) < 0.5
    M[..., np.arange(Nb), np.arange(Nb)] = True   # every row attends somewhere (SDPA needs it)
    t = [torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True) for x in (q, k, v)]
    mask = torch.from_numpy(_token_mask(M, N, blk))
    out = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=mask)
    (out * torch.from_numpy(g)).sum().backward()
    dq, dk, dv = O.attention_bwd(q, k, v, g, M, blk)
    for mine, ref in ((dq, t[0].grad), (dk, t[1].grad), (dv, t[2].grad)):
        assert np.allclose(mine, ref.numpy(), atol=1e-11, rtol=0)


def check_bwd_identical_keys_closed_form():
    """One kept block of identical keys: P is uniform, so dQ = 0 and dV_j = mean_i G_i."""
    B, H, N, d, blk = 1, 1, 96, 8, 32
    q, k, v = _qkv(B, H, N, d, 37)
    k[0, 0, 32:64] = k[0, 0, 40]            # key block 1: one repeated key
    g = RNG(38).standard_normal((B, H, N, d))
    M = np.zeros((B, H, 3, 3), dtype=bool)
    M[0, 0, 0, 1] = True                     # query block 0 attends key block 1 only
    dq, dk, dv = O.attention_bwd(q, k, v, g, M, blk)
    assert np.allclose(dq[0, 0, :32], 0.0, atol=1e-12)
    assert np.allclose(dv[0, 0, 32:64], np.broadcast_to(g[0, 0, :32].mean(axis=0), (32, d)), atol=1e-12)
    assert np.all(dq[0, 0, 32:] == 0) and np.all(dk[0, 0, :32] == 0) and np.all(dv[0, 0, 64:] == 0)


def _bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest even, through float32) and back to float64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def check_bwd_terms_bound_rounded_products():
    """attention_bwd_terms bounds the gradients of a computation that rounds P and dS to
    bf16 before the products, and the bound is tight enough to matter.

    Per query block, P and dS = dL/dS come from torch (softmax and autograd of
    sum(G * softmax(S) V), no formula retyped), are rounded to bf16, and give the gradients
    through plain matmuls.  Each element's error against attention_bwd must stay within
    2^-8 times its term sum (the rounding is at most 2^-9 relative).  Keys share a large
    component in one head, so there dQ cancels and its rounded error exceeds 2^-8 |dQ|
    by far while staying inside the term bound."""
    B, H, N, d, blk = 1, 2, 150, 16, 32
    q, k, v = _qkv(B, H, N, d, 42)
    k[0, 1] += 40.0                           # head 1: a large component shared by every key
    g = RNG(43).standard_normal((B, H, N, d))
    Nb = O.num_blocks(N, blk)
    M = RNG(44).random((B, H, Nb, Nb)) < 0.6
    M[0, 0, 2] = False                        # a query block with no kept key block
    M[0, 1, :, 0] = True
    dq, dk, dv = O.attention_bwd(q, k, v, g, M, blk)
    tq, tk, tv = O.attention_bwd_terms(q, k, v, g, M, blk)
    rq, rk, rv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for h in range(H):
        for r in range(Nb):
            J = O.kept_tokens(M[0, h, r], N, blk)
            if J.size == 0:
                continue
            lo, hi = O.block_range(r, N, blk)
            qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q[0, h, lo:hi], k[0, h, J], v[0, h, J]))
            S = (qt @ kt.T / math.sqrt(d)).requires_grad_(True)
            P = torch.softmax(S, dim=1)
            (P @ vt * torch.from_numpy(g[0, h, lo:hi])).sum().backward()
            Pr, dSr = _bf16(P.detach().numpy()), _bf16(S.grad.numpy())
            rq[0, h, lo:hi] = dSr @ k[0, h, J] / math.sqrt(d)
            rk[0, h, J] += dSr.T @ q[0, h, lo:hi] / math.sqrt(d)
            rv[0, h, J] += Pr.T @ g[0, h, lo:hi]
    u = 2.0 ** -8
    for name, r_, x, t in (("dq", rq, dq, tq), ("dk", rk, dk, tk), ("dv", rv, dv, tv)):
        err = np.abs(r_ - x)
        assert np.all(err <= u * t + 1e-12), (name, float((err - u * t).max()))
        assert np.all(np.abs(x) <= t * (1 + 1e-12) + 1e-12), name      # triangle inequality
        ratio = err[t > 0] / (u * t[t > 0])
        assert ratio.max() > 0.15, (name, ratio.max())                 # not a loose bound
    assert np.all(tq[0, 0, 64:96] == 0) and np.all(dq[0, 0, 64:96] == 0)
    err1, mag1 = np.abs(rq[0, 1] - dq[0, 1]), np.abs(dq[0, 1])
    assert err1.max() > 4 * u * mag1.max(), (err1.max(), mag1.max())  # cancellation in dQ


def check_bwd_blocks_assemble_full():
    """Per-row pieces (attention_bwd_block) add up to the whole-tensor gradients."""
    B, H, N, d, blk = 1, 2, 100, 8, 32
    q, k, v = _qkv(B, H, N, d, 39)
    g = RNG(40).standard_normal((B, H, N, d))
    Nb = O.num_blocks(N, blk)
    M = RNG(41).random((B, H, Nb, Nb)) < 0.5
    dq, dk, dv = O.attention_bwd(q, k, v, g, M, blk)
    dq2, dk2, dv2 = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for h in range(H):
        for r in range(Nb):
            lo, hi = O.block_range(r, N, blk)
            a, J, bk, bv = O.attention_bwd_block(q, k, v, g, M, blk, 0, h, r)
            dq2[0, h, lo:hi] = a
            dk2[0, h, J] += bk
            dv2[0, h, J] += bv
    assert np.allclose(dq, dq2, atol=1e-13) and np.allclose(dk, dk2, atol=1e-13)
    assert np.allclose(dv, dv2, atol=1e-13)


def check_lse_matches_scipy():
    """attention_lse == scipy logsumexp of the masked token scores; -inf for empty rows."""
    B, H, N, d, blk = 1, 2, 90, 8, 32
    q, k, _ = _qkv(B, H, N, d, 42)
    Nb = O.num_blocks(N, blk)
    M = RNG(43).random((B, H, Nb, Nb)) < 0.5
    M[0, 1, 2] = False
    L = O.attention_lse(q, k, M, blk)
    tm = _token_mask(M, N, blk)
    for h in range(H):
        s = q[0, h] @ k[0, h].T / math.sqrt(d)
        s = np.where(tm[0, h], s, -np.inf)
        ref = scipy.special.logsumexp(s, axis=1)
        assert np.allclose(L[0, h], ref, atol=1e-12, rtol=0, equal_nan=False)
    assert np.all(np.isneginf(L[0, 1, 64:]))


# ------------------------------------------------------------------ pattern search pins
def check_pattern_sparsity_token_pairs():
    """S_i = fraction of dropped token pairs, by enumerating the token-level mask (ragged
    blocks count at their true size), plus the closed forms of the mode table."""
    for N, blk in ((300, 32), (130, 16), (256, 64)):
        Nb = O.num_blocks(N, blk)
        blk_of = np.arange(N) // blk
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        for pid, prm in ((O.DIAG, 0), (O.VSTRIPE, 2), (O.MULTIDIAG, 5), (O.MULTIDIAG, 48),
                         (O.FULL, 0), (O.SKIP, 0)):
            if pid == O.MULTIDIAG:
                hit = ((j - i) % prm) == 0            # token pairs on the diagonals
                tile = np.zeros((Nb, Nb), dtype=bool)
                np.logical_or.at(tile, (blk_of[:, None].repeat(N, 1), blk_of[None, :].repeat(N, 0)), hit)
            elif pid == O.DIAG:
                tile = np.eye(Nb, dtype=bool)
            elif pid == O.VSTRIPE:
                tile = np.zeros((Nb, Nb), dtype=bool)
                tile[:, :prm] = True
            else:
                tile = np.full((Nb, Nb), pid == O.FULL)
            tok = tile[blk_of][:, blk_of]
            want = 1.0 - tok.sum() / float(N * N)
            got = O.pattern_sparsity(pid, prm, N, blk)
            assert abs(got - want) < 1e-15, (N, blk, pid, prm, got, want)
    assert O.pattern_sparsity(O.FULL, 0, 300, 32) == 0.0
    assert O.pattern_sparsity(O.SKIP, 0, 300, 32) == 1.0
    assert abs(O.pattern_sparsity(O.DIAG, 0, 1024, 64) - (1 - 1 / 16)) < 1e-15
    assert abs(O.pattern_sparsity(O.VSTRIPE, 3, 1000, 64) - (1 - 3 * 64 / 1000)) < 1e-15


def _masked_sdpa_or_zero(q, k, v, tok):
    """torch SDPA (float64, boolean token mask) per head; rows with no kept key -> 0."""
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = torch.from_numpy(np.ascontiguousarray(tok))
    out = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m)
    out = torch.where(m.any(dim=-1, keepdim=True), out, torch.zeros_like(out))
    return out.numpy()


def check_pattern_mse_matches_torch():
    """MSE(O_i - O_0) per head: candidates' outputs from torch SDPA with the token mask,
    the squared error from torch's mse_loss on each head's [B, N, d] slice."""
    B, H, N, d, blk = 2, 3, 200, 16, 64
    q, k, v = _qkv(B, H, N, d, 41)
    v[:, 1] *= 3.0                                     # heads on different scales
    cands = [(O.SKIP, 0), (O.DIAG, 0), (O.MULTIDIAG, 50), (O.VSTRIPE, 1)]
    choice, L, mse, S = O.pattern_search(q, k, v, blk, cands, lam=0.01, eps=0.1)
    o0 = _sdpa(q, k, v)
    for n, (pid, prm) in enumerate(cands):
        tok = _token_mask(O.static_mask(B, H, N, blk, [(pid, prm)] * H), N, blk)
        oi = _masked_sdpa_or_zero(q, k, v, tok)
        for h in range(H):
            want = torch.nn.functional.mse_loss(torch.from_numpy(oi[:, h]), torch.from_numpy(o0[:, h])).item()
            assert abs(mse[h, n] - want) <= 1e-13 * max(1.0, want), (n, h, mse[h, n], want)
    assert L.shape == (H, len(cands)) and choice.shape == (H,)


def check_pattern_uniform_attention_closed_form():
    """Q = 0 makes every row's weights uniform over its kept tokens, so each output row is
    the mean of V over those tokens: full -> mean over all N, diagonal -> mean over the
    query's own block, stripe(s) -> mean over the first s blocks, skip -> 0.  The losses
    and the choice follow from these means alone."""
    B, H, N, d, blk = 1, 4, 320, 8, 64                 # 5 blocks
    rng = RNG(43)
    k = rng.standard_normal((B, H, N, d))
    q = np.zeros((B, H, N, d))
    offs = rng.standard_normal((B, H, 5, d))
    v = np.repeat(offs, blk, axis=2) + 0.1 * rng.standard_normal((B, H, N, d))
    v[:, 0] *= 0.05                                    # tiny outputs: skipping is cheapest
    v[:, 1] *= 3.0                                     # large spread: every L_i > eps
    v[:, 2] *= 0.2
    v[:, 3] = np.repeat(offs[:, 3, :1], N, axis=1) * 0.5 + 0.3   # block-constant rows -> diag exact
    lam, eps = 0.01, 0.1
    cands = [(O.SKIP, 0), (O.DIAG, 0), (O.VSTRIPE, 1)]
    choice, L, mse, S = O.pattern_search(q, k, v, blk, cands, lam, eps)
    want = np.zeros((H, 3))
    for h in range(H):
        full = v[0, h].mean(axis=0)
        blockmean = np.stack([v[0, h, r * blk:(r + 1) * blk].mean(axis=0) for r in range(5)])
        diag_rows = np.repeat(blockmean, blk, axis=0)
        stripe = v[0, h, :blk].mean(axis=0)
        want[h, 0] = np.mean(full ** 2) + lam * 0.0
        want[h, 1] = np.mean((diag_rows - full) ** 2) + lam * (5 * blk * blk) / N ** 2
        want[h, 2] = np.mean((stripe - full) ** 2) + lam * (N * blk) / N ** 2
    assert np.allclose(L, want, rtol=1e-12, atol=1e-15), (L, want)
    assert np.allclose(S, [1.0, 1 - 1 / 5, 1 - 1 / 5], rtol=0, atol=1e-15)
    # the branches this case was built to reach
    assert choice[0] == 1 and choice[1] == 0 and choice[3] == 2, choice
    assert np.array_equal(choice, O.select_patterns(want, eps))


def check_select_rule_cases():
    """The selection formula on hand-made losses: full attention only when every L_i is
    strictly above eps; otherwise the smallest L_i, first index on ties."""
    cases = [
        ([[0.2, 0.3, 0.15]], 0.1, [0]),
        ([[0.2, 0.05, 0.07]], 0.1, [2]),
        ([[0.05, 0.05]], 0.1, [1]),
        ([[0.1, 0.2]], 0.1, [1]),
        ([[0.3, 0.09, 0.5]], 0.1, [2]),
        ([[0.2, 0.3], [0.01, 0.02], [0.5, 0.11]], 0.1, [0, 1, 0]),
        ([[0.12, 0.11]], 0.15, [2]),
    ]
    for L, eps, want in cases:
        got = O.select_patterns(np.array(L), eps)
        assert list(got) == want, (L, eps, got, want)
    assert list(O.select_patterns(np.zeros((3, 0)), 0.1)) == [0, 0, 0]
    # the loss adds lam * (1 - S_i): kept fraction 0.1 and 0.5 at lam 0.01
    L = O.pattern_loss(np.array([[0.01, 0.02]]), np.array([0.9, 0.5]), 0.01)
    assert np.allclose(L, [[0.011, 0.025]], rtol=0, atol=1e-15)


def check_search_follows_table3_trends():
    """The page's Table 3 (tests/golden/sparse_vdit_table3.json): a larger epsilon or a
    smaller lambda gives a larger speedup, i.e. sparser choices.  On heads whose losses
    spread across the thresholds (uniform attention, Q = 0, so each output row is a mean of
    V), the oracle's kept fraction of token pairs must order the settings the same way."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sparse_vdit_table3.json")
    rows = json.load(open(path))["rows"]
    B, H, N, d, blk = 1, 12, 320, 8, 64                 # 5 blocks
    rng = RNG(47)
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    offs = rng.standard_normal((B, H, 5, d))
    v = np.repeat(offs, blk, axis=2) + 0.3 * rng.standard_normal((B, H, N, d))
    v *= np.geomspace(0.1, 0.8, H)[None, :, None, None]    # pattern losses from ~0.01 to ~0.7
    v += 1.0                                               # large outputs: skipping never pays
    cands = [(O.SKIP, 0), (O.DIAG, 0), (O.VSTRIPE, 3)]
    kept = {}
    for row in rows:
        choice, L, mse, S = O.pattern_search(q, k, v, blk, cands, row["lambda"], row["epsilon"])
        dens = np.array([1.0] + [1.0 - x for x in S])         # choice 0 = full attention
        kept[(row["lambda"], row["epsilon"])] = float(dens[choice].mean())
    for a in rows:
        for b in rows:
            if a["speedup"] > b["speedup"]:
                ka, kb = kept[(a["lambda"], a["epsilon"])], kept[(b["lambda"], b["epsilon"])]
                assert ka <= kb, (a, b, ka, kb)
    # epsilon alone moves the choice on these heads
    assert kept[(0.01, 0.15)] < kept[(0.01, 0.1)] < kept[(0.01, 0.05)], kept


# ------------------------------------------------------------------ near-tie rule pins
def _row_from_sorted_scores(vals, perm):
    """A score row whose rank order is `perm` and whose sorted scores are `vals`."""
    s = np.empty(len(vals))
    s[np.asarray(perm)] = vals
    return s


def _filler_rows(nb):
    """Score rows with gaps of at least 0.5 everywhere (never near a tie)."""
    return np.stack([np.roll(np.arange(nb, dtype=np.float64) * 0.5, i) for i in range(nb)])


def _amb_single(s_row, **kw):
    """The near-tie flag of one planted row, placed as row 0 of a square score matrix."""
    s_row = np.asarray(s_row, dtype=np.float64)
    S = _filler_rows(s_row.shape[0])
    S[0] = s_row
    S = S[None, None]
    return bool(O.ambiguous_rows(S, O.block_softmax(S), **kw)[0, 0, 0])


def check_ambiguous_rows_planted():
    """The near-tie rule (a row may differ between two correct implementations only if the
    last kept and first dropped candidates differ in block score by under 1e-6, or the
    cumulative mass next to the stopping point is within 1e-6 of tau), on planted rows.

    Every expectation below follows from the rule's wording, not from the oracle: the
    gaps are placed in S (flag below 1e-6, none at 2e-6, including at small P where P
    gaps are far below 1e-6), only at the selection edge (near-ties one place before or
    after the edge do not flag), and at the prefix masses just before and at the stopping
    point in cumulative-mass mode.  Rows keeping no candidate or every candidate have no
    edge and never flag.
    """
    perm = [5, 2, 7, 0, 3, 6, 1, 4]                      # rank order of the planted rows
    base = np.array([4.0, 3.0, 2.0, 1.0, 0.0, -1.0, -2.0, -3.0])

    def topk_row(edge_gap, at=2, lift=0.0):
        v = base.copy() + lift
        v[at + 1] = v[at] - edge_gap                     # gap between rank `at` and `at`+1
        return _row_from_sorted_scores(v, perm)

    k = 3                                                # edge between rank 2 and rank 3
    assert _amb_single(topk_row(5e-7), mode=O.TOPK, k=k)
    assert not _amb_single(topk_row(2e-6), mode=O.TOPK, k=k)
    # the same gaps far down the softmax (P ~ 1e-6 and below): P gaps are ~1e-12, so
    # only gaps measured in S decide
    v = base.copy()
    v[2:] -= 14.0                                        # ranks 2.. at P ~ 1e-6 and below
    v[3] = v[2] - 2e-6
    assert not _amb_single(_row_from_sorted_scores(v, perm), mode=O.TOPK, k=k)
    v[3] = v[2] - 5e-7
    assert _amb_single(_row_from_sorted_scores(v, perm), mode=O.TOPK, k=k)
    # near-ties one place before and one place after the edge do not flag
    vb = base.copy()                                     # ranks 1, 2 (both kept)
    vb[2] = vb[1] - 1e-9
    assert not _amb_single(_row_from_sorted_scores(vb, perm), mode=O.TOPK, k=k)
    va = base.copy()
    va[4] = va[3] - 1e-9                                 # ranks 3, 4 (both dropped)
    assert not _amb_single(_row_from_sorted_scores(va, perm), mode=O.TOPK, k=k)
    # no edge: k = 0 keeps nothing, k >= Nb keeps everything (exact ties everywhere)
    flat = np.zeros(8)
    assert not _amb_single(flat, mode=O.TOPK, k=0)
    assert not _amb_single(flat, mode=O.TOPK, k=8)
    assert not _amb_single(flat, mode=O.TOPK, k=20)
    assert _amb_single(flat, mode=O.TOPK, k=4)

    # cumulative-mass mode: P chosen directly, S = log P (softmax gives P back)
    p = np.array([0.4, 0.25, 0.15, 0.1, 0.06, 0.04])
    perm6 = [3, 0, 5, 1, 4, 2]
    s6 = _row_from_sorted_scores(np.log(p), perm6)
    cs = np.cumsum(p)
    tau_far = cs[2] + 0.02                               # between cs[2] and cs[3], far from both
    assert not _amb_single(s6, mode=O.TAU, tau=tau_far)
    # mass at the stopping point within 3e-7 above tau: m = 3, cs[m-1] - tau = 3e-7
    assert _amb_single(s6, mode=O.TAU, tau=cs[2] - 3e-7)
    # mass just before the stopping point within 3e-7 below tau: m = 4, tau - cs[m-2] = 3e-7
    assert _amb_single(s6, mode=O.TAU, tau=cs[2] + 3e-7)
    # the same distances at 2e-6 do not flag
    assert not _amb_single(s6, mode=O.TAU, tau=cs[2] - 2e-6)
    assert not _amb_single(s6, mode=O.TAU, tau=cs[2] + 2e-6)
    # mass one place after the stopping point near tau is no edge: m = 2 here
    # (cs[1] >= tau), and cs[2] sits 3e-7 from a second threshold that is not tau
    assert not _amb_single(s6, mode=O.TAU, tau=cs[1] - 0.01)
    # tau above the total: every candidate kept, no edge
    assert not _amb_single(s6, mode=O.TAU, tau=1.5)
    # the cap sets the edge: natural m = 4, cap 2, ranks 1 and 2 within 5e-7 in S
    pc = np.array([0.4, 0.2, 0.2 * np.exp(-5e-7), 0.1, 0.06, 0.04])
    pc /= pc.sum()
    sc = _row_from_sorted_scores(np.log(pc), perm6)
    assert _amb_single(sc, mode=O.TAU, tau=0.85, k_cap=2)
    pc2 = np.array([0.4, 0.2, 0.2 * np.exp(-2e-6), 0.1, 0.06, 0.04])
    sc2 = _row_from_sorted_scores(np.log(pc2 / pc2.sum()), perm6)
    assert not _amb_single(sc2, mode=O.TAU, tau=0.85, k_cap=2)

    # many rows at once keep their own flags (no leakage across rows, heads, batches)
    rows = [topk_row(5e-7), topk_row(2e-6), topk_row(1e-3), topk_row(3e-7)]
    S = np.stack([_filler_rows(8)] * 4)
    for i, row in enumerate(rows):
        S[i, 5] = row
    S = S.reshape(2, 2, 8, 8)
    got = O.ambiguous_rows(S, O.block_softmax(S), mode=O.TOPK, k=k).reshape(4, 8)
    assert got[:, 5].tolist() == [True, False, False, True]
    assert not got[:, :5].any() and not got[:, 6:].any()


def check_attention_block_matches_sdpa_and_full():
    """attention_block (the outputs of one query block) equals torch SDPA run on that
    block's queries against the union of its kept key blocks (a library routine), and the
    matching slice of the full masked attention, on ragged blocks and an empty row."""
    B, H, N, d, blk = 2, 2, 230, 16, 64                  # 4 blocks, last one 38 tokens
    q, k, v = _qkv(B, H, N, d, 61, scale=1.5)
    Nb = O.num_blocks(N, blk)
    rng = RNG(62)
    M = rng.random((B, H, Nb, Nb)) < 0.5
    M[1, 0, 2, :] = False                                # an empty row
    M[0, 1, 3, :] = True                                 # a full ragged row
    full = O.attention(q, k, v, M, blk)
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                lo, hi = O.block_range(r, N, blk)
                got = O.attention_block(q, k, v, M, blk, b, h, r)
                assert got.shape == (hi - lo, d)
                cols = [c for c in range(Nb) if M[b, h, r, c]]
                if not cols:
                    assert np.all(got == 0.0)
                else:
                    J = np.concatenate([np.arange(*O.block_range(c, N, blk)) for c in cols])
                    ref = _sdpa(q[b, h, lo:hi][None], k[b, h, J][None], v[b, h, J][None])[0]
                    assert np.allclose(got, ref, atol=1e-12, rtol=0)
                assert np.array_equal(got, full[b, h, lo:hi])


ALL_CHECKS = [
    check_dense_equals_sdpa, check_block_diagonal_equals_independent_blocks,
    check_weights_sum_to_one, check_identical_keys_give_mean_of_v,
    check_bruteforce_2head_n128, check_skip_and_empty_rows_are_zero,
    check_attention_rows_match_full, check_pool_score_bilinearity,
    check_block_softmax_matches_scipy, check_rank_order_ties, check_selection_bruteforce,
    check_selection_limits_and_monotone, check_forced_blocks,
    check_static_patterns_token_pairs, check_frame_tile_token_pairs, check_static_counts_8192,
    check_csr_layout,
    check_kept_tile_flops,
    check_bwd_finite_differences, check_bwd_matches_torch_autograd,
    check_bwd_identical_keys_closed_form, check_bwd_blocks_assemble_full, check_lse_matches_scipy,
    check_bwd_terms_bound_rounded_products,
    check_pattern_sparsity_token_pairs, check_pattern_mse_matches_torch,
    check_pattern_uniform_attention_closed_form, check_select_rule_cases,
    check_search_follows_table3_trends,
    check_ambiguous_rows_planted, check_attention_block_matches_sdpa_and_full,
]
