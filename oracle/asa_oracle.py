"""Plain float64 CPU oracle for content-aware block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library and its
Python binding never call it, and it shares no code with them.

What it computes, in the order the method applies it:

* Attention, dense and masked -- Sparse-vDiT ("Sparse-vDiT: Sparse Attention
  Acceleration for Video Diffusion Transformers"), section 三 "核心公式":
  full attention softmax(Q_h K_h^T / sqrt(d)) V_h per head, and the masked form
  Attention(Q, K, V, M) whose mask M keeps or drops (query-block, key-block)
  tiles.
* Static mask sources -- same page, the "四种注意力模式" table: M0 full,
  M1 skip (output set to zero), M2 diagonal (intra-frame), M3 multi-diagonal
  (evenly spaced diagonals, cross-frame), M4 vertical stripe (global tokens).
  One more from "Efficient-vDiT: Efficient Video Diffusion Transformers With
  Attention Tile", section 3.1 (注意力图块化): the 3D attention map splits into
  frame-by-frame tiles that repeat, and a sparse tile set gives attention linear
  in the number of frames.  The page names no tile set; the one here keeps, for
  each query frame, its own frame and the first frame (frame tiles of F tokens).
* Adaptive mask source -- BLADE ("BLADE: Block-Sparse Attention Meets Step
  Distillation for Efficient Video Generation"), abstract: ASA generates a
  content-aware block mask per input.  The pages give no rule, so this oracle
  implements the stated rule: mean-pool Q and K per block, block scores
  Qp Kp^T / sqrt(d), row softmax, keep the top-k blocks (or the shortest prefix
  whose probability mass reaches tau, optionally capped), plus the diagonal
  block and any block holding text tokens.

* Backward of the masked attention -- the gradients (dQ, dK, dV) of
  sum(dO * O) by the chain rule through each row softmax, and the log of each
  row's softmax normaliser (what a training forward keeps for the backward).
  BLADE trains the sparse attention jointly with step distillation (abstract).

* Per-head pattern search -- Sparse-vDiT, section 三: the offline search loss
  L_i = MSE(O_i - O_0) + lambda (1 - S_i) over the candidate patterns, and the
  selection formula (full attention when every L_i exceeds epsilon, else the
  candidate with the smallest L_i), one layer of its offline search algorithm.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, library routines (torch SDPA and its autograd, scipy
softmax / logsumexp), finite differences and brute force.  The pooled-score rule and the tuned top-k are specification choices:
their fidelity to BLADE's own ASA is parity unpinned (the pages do not state
it).

All arithmetic is float64.  Tensors are NumPy arrays laid out [B, H, N, d].
"""
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Integer codes shared with the C ABI by convention (each side defines them).
ADAPTIVE, FULL, SKIP, DIAG, MULTIDIAG, VSTRIPE, FRAME_TILE = 0, 1, 2, 3, 4, 5, 6
TOPK, TAU = 0, 1

AMBIGUITY_GAP = 1e-6


# --------------------------------------------------------------------------- blocks
def num_blocks(N: int, blk: int) -> int:
    return (N + blk - 1) // blk


def block_range(r: int, N: int, blk: int) -> Tuple[int, int]:
    """Token range [lo, hi) of block r; the last block may be partial."""
    lo = r * blk
    return lo, min(lo + blk, N)


# --------------------------------------------------------------------------- mask rule
def pool(X: np.ndarray, blk: int) -> np.ndarray:
    """Per-block mean of X over the valid tokens of each block.

    X [B,H,N,d] -> [B,H,Nb,d].  A partial last block is averaged over its own
    token count (no zero padding).
    """
    B, H, N, d = X.shape
    Nb = num_blocks(N, blk)
    out = np.empty((B, H, Nb, d), dtype=np.float64)
    for r in range(Nb):
        lo, hi = block_range(r, N, blk)
        out[:, :, r, :] = X[:, :, lo:hi, :].astype(np.float64).mean(axis=2)
    return out


def block_scores(Qp: np.ndarray, Kp: np.ndarray) -> np.ndarray:
    """S[r, c] = Qp[r] . Kp[c] / sqrt(d), the same scale as token attention."""
    d = Qp.shape[-1]
    return np.matmul(Qp, np.swapaxes(Kp, -1, -2)) / np.sqrt(d)


def block_softmax(S: np.ndarray) -> np.ndarray:
    """Row softmax over all key blocks (max-subtracted)."""
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(axis=-1, keepdims=True)


def rank_order(p_row: np.ndarray) -> np.ndarray:
    """Key-block indices sorted by probability descending, ties by smaller index."""
    idx = np.arange(p_row.shape[0])
    return np.lexsort((idx, -p_row))


def adaptive_count(p_row: np.ndarray, order: np.ndarray, mode: int, k: int,
                   tau: float, k_cap: int) -> int:
    """How many leading entries of the rank order the adaptive source keeps."""
    Nb = p_row.shape[0]
    if mode == TOPK:
        return min(max(k, 0), Nb)
    if mode == TAU:
        mass = 0.0
        m = Nb
        for t in range(Nb):
            mass += p_row[order[t]]          # sequential prefix sum, rank order
            if mass >= tau:
                m = t + 1
                break
        if k_cap > 0:
            m = min(m, k_cap)
        return m
    raise ValueError(f"unknown adaptive mode {mode}")


def adaptive_set(p_row: np.ndarray, mode: int, k: int, tau: float, k_cap: int) -> np.ndarray:
    order = rank_order(p_row)
    m = adaptive_count(p_row, order, mode, k, tau, k_cap)
    return np.sort(order[:m])


def text_blocks(Nb: int, blk: int, n_text: int) -> int:
    """Number of leading blocks that hold at least one text token."""
    if n_text <= 0:
        return 0
    return min(Nb, num_blocks(n_text, blk))


def static_row(pattern: int, param: int, r: int, N: int, blk: int) -> np.ndarray:
    """Boolean row of kept key blocks for one static pattern (block level).

    MULTIDIAG(S): tile (r, c) is kept iff some query i in block r and key j in
    block c satisfy (j - i) = 0 mod S, i.e. the integer interval
    [min T_c - max T_r, max T_c - min T_r] contains a multiple of S.
    FRAME_TILE(F): with frame(t) = floor(t / F), tile (r, c) is kept iff some query i
    in block r and key j in block c have frame(j) == frame(i) or frame(j) == 0.
    """
    Nb = num_blocks(N, blk)
    row = np.zeros(Nb, dtype=bool)
    if pattern == FULL:
        row[:] = True
    elif pattern == SKIP:
        pass
    elif pattern == DIAG:
        row[r] = True
    elif pattern == VSTRIPE:
        row[:max(0, min(param, Nb))] = True
    elif pattern == MULTIDIAG:
        S = int(param)
        if S <= 0:
            raise ValueError("multi-diagonal stride must be positive")
        qlo, qhi = block_range(r, N, blk)
        for c in range(Nb):
            klo, khi = block_range(c, N, blk)
            lo = klo - (qhi - 1)
            hi = (khi - 1) - qlo
            # smallest multiple of S that is >= lo, compared with hi
            first = -((-lo) // S) * S
            row[c] = first <= hi
    elif pattern == FRAME_TILE:
        F = int(param)
        if F <= 0:
            raise ValueError("frame-tile frame length must be positive")
        qlo, qhi = block_range(r, N, blk)
        qframes = set(range(qlo // F, (qhi - 1) // F + 1))
        for c in range(Nb):
            klo, khi = block_range(c, N, blk)
            kframes = set(range(klo // F, (khi - 1) // F + 1))
            row[c] = 0 in kframes or bool(qframes & kframes)
    else:
        raise ValueError(f"unknown pattern id {pattern}")
    return row


def static_mask(B: int, H: int, N: int, blk: int,
                patterns: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Block mask [B,H,Nb,Nb] from per-head static patterns alone."""
    Nb = num_blocks(N, blk)
    M = np.zeros((B, H, Nb, Nb), dtype=bool)
    cache: Dict[Tuple[int, int], np.ndarray] = {}
    for h in range(H):
        pid, prm = patterns[h]
        if pid == ADAPTIVE:
            raise ValueError("the static call takes no adaptive heads")
        if (pid, prm) not in cache:
            cache[(pid, prm)] = np.stack([static_row(pid, prm, r, N, blk) for r in range(Nb)])
        M[:, h] = cache[(pid, prm)]
    return M


def build_mask(Q: np.ndarray, K: np.ndarray, blk: int, *, mode: int, k: int = 0,
               tau: float = 0.0, k_cap: int = 0, n_text: int = 0, keep_diag: int = 1,
               patterns: Optional[Sequence[Tuple[int, int]]] = None,
               return_details: bool = False):
    """Adaptive block mask [B,H,Nb,Nb] (bool), unioned with forced and static blocks.

    kept_r = A_r  U  {r if keep_diag}  U  {text key blocks}  U  static_r(head),
    a row whose query block holds text tokens is full, and a SKIP head is empty.
    """
    B, H, N, d = Q.shape
    Nb = num_blocks(N, blk)
    Qp, Kp = pool(Q, blk), pool(K, blk)
    S = block_scores(Qp, Kp)
    P = block_softmax(S)
    nt = text_blocks(Nb, blk, n_text)
    pats = list(patterns) if patterns is not None else [(ADAPTIVE, 0)] * H
    M = np.zeros((B, H, Nb, Nb), dtype=bool)
    counts = np.zeros((B, H, Nb), dtype=np.int64)
    static_cache: Dict[Tuple[int, int, int], np.ndarray] = {}
    for b in range(B):
        for h in range(H):
            pid, prm = pats[h]
            if pid == SKIP:
                continue
            for r in range(Nb):
                row = np.zeros(Nb, dtype=bool)
                order = rank_order(P[b, h, r])
                m = adaptive_count(P[b, h, r], order, mode, k, tau, k_cap)
                counts[b, h, r] = m
                row[order[:m]] = True
                if keep_diag:
                    row[r] = True
                row[:nt] = True
                if r < nt:
                    row[:] = True
                if pid != ADAPTIVE:
                    key = (pid, prm, r)
                    if key not in static_cache:   # static rows do not depend on the head
                        static_cache[key] = static_row(pid, prm, r, N, blk)
                    row |= static_cache[key]
                M[b, h, r] = row
    if return_details:
        return M, {"Qp": Qp, "Kp": Kp, "S": S, "P": P, "adaptive_count": counts}
    return M


def ambiguous_rows(S: np.ndarray, P: np.ndarray, *, mode: int, k: int = 0, tau: float = 0.0,
                   k_cap: int = 0, gap: float = AMBIGUITY_GAP) -> np.ndarray:
    """Rows whose adaptive selection could flip under rounding-order differences.

    A row is ambiguous if the last kept and first dropped candidates of the rank
    order differ in block score by less than ``gap``, or (cumulative-mass mode)
    the prefix mass just before or at the stopping point is within ``gap`` of tau.
    Returns a bool array [B,H,Nb].
    """
    B, H, Nb, _ = S.shape
    amb = np.zeros((B, H, Nb), dtype=bool)
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                p = P[b, h, r]
                order = rank_order(p)
                m = adaptive_count(p, order, mode, k, tau, k_cap)
                flag = False
                if 0 < m < Nb:
                    flag = abs(S[b, h, r, order[m - 1]] - S[b, h, r, order[m]]) < gap
                if mode == TAU and not flag:
                    cs = np.cumsum(p[order])
                    for t in (m - 2, m - 1):
                        if 0 <= t < Nb and abs(cs[t] - tau) < gap:
                            flag = True
                amb[b, h, r] = flag
    return amb


def to_csr(M: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-major CSR of a [B,H,Nb,Nb] block mask: row_ptr [B*H*Nb+1], col_idx ascending."""
    rows = M.reshape(-1, M.shape[-1])
    counts = rows.sum(axis=1)
    row_ptr = np.zeros(rows.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(rows)[1].astype(np.int64)   # row-major, ascending per row
    return row_ptr, col_idx


def density(M: np.ndarray, heads: Optional[Sequence[int]] = None) -> float:
    """Fraction of kept tiles."""
    if heads is not None:
        M = M[:, list(heads)]
    return float(M.mean())


# --------------------------------------------------------------------------- attention
def _row_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v for a set of query rows, two-pass per row."""
    d = q.shape[-1]
    s = (q @ k.T) / np.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def kept_tokens(mask_row: np.ndarray, N: int, blk: int) -> np.ndarray:
    """J = union of the token ranges of the kept key blocks (ascending)."""
    parts = [np.arange(*block_range(c, N, blk)) for c in np.nonzero(mask_row)[0]]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts)


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, M: np.ndarray, blk: int) -> np.ndarray:
    """Masked block-sparse attention, float64.  O_i = 0 where no key block is kept."""
    B, H, N, d = Q.shape
    Nb = num_blocks(N, blk)
    O = np.zeros((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                J = kept_tokens(M[b, h, r], N, blk)
                if J.size == 0:
                    continue
                lo, hi = block_range(r, N, blk)
                O[b, h, lo:hi] = _row_attention(
                    Q[b, h, lo:hi].astype(np.float64), K[b, h, J].astype(np.float64),
                    V[b, h, J].astype(np.float64))
    return O


def attention_block(Q: np.ndarray, K: np.ndarray, V: np.ndarray, M: np.ndarray, blk: int,
                    b: int, h: int, r: int) -> np.ndarray:
    """Outputs of the query tokens of block r of head (b, h): [n_r, d]."""
    N, d = Q.shape[2], Q.shape[3]
    lo, hi = block_range(r, N, blk)
    J = kept_tokens(M[b, h, r], N, blk)
    if J.size == 0:
        return np.zeros((hi - lo, d), dtype=np.float64)
    return _row_attention(Q[b, h, lo:hi].astype(np.float64), K[b, h, J].astype(np.float64),
                          V[b, h, J].astype(np.float64))


def attention_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, M: np.ndarray, blk: int,
                   rows: Sequence[Tuple[int, int, int]]) -> np.ndarray:
    """Outputs for selected query tokens (b, h, i) only: [len(rows), d]."""
    N, d = Q.shape[2], Q.shape[3]
    out = np.zeros((len(rows), d), dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        J = kept_tokens(M[b, h, i // blk], N, blk)
        if J.size == 0:
            continue
        out[n] = _row_attention(Q[b, h, i:i + 1].astype(np.float64),
                                K[b, h, J].astype(np.float64),
                                V[b, h, J].astype(np.float64))[0]
    return out


def dense_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Full attention (pattern M0) for every head."""
    B, H, N, d = Q.shape
    O = np.empty((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h] = _row_attention(Q[b, h].astype(np.float64), K[b, h].astype(np.float64),
                                     V[b, h].astype(np.float64))
    return O


def kept_tile_flops(M: np.ndarray, N: int, blk: int, d: int) -> float:
    """Sum over kept tiles of 4 * n_r * n_c * d (QK^T and PV multiply-adds, x2)."""
    Nb = M.shape[-1]
    sizes = np.array([block_range(c, N, blk)[1] - block_range(c, N, blk)[0]
                      for c in range(Nb)], dtype=np.float64)
    per_tile = 4.0 * np.outer(sizes, sizes) * d
    return float((M * per_tile).sum())


# ---------------------------------------------------------------------------- backward
# Gradients of the masked attention above.  BLADE ("BLADE: Block-Sparse Attention Meets
# Step Distillation for Efficient Video Generation", abstract) trains the sparse attention
# jointly with step distillation, so training needs the gradient through the same masked
# attention (Sparse-vDiT, section 三 "核心公式").  Derived by the chain rule through
# the row softmax of each query row, over the same kept token set J_i as the forward:
#   s = q k^T / sqrt(d),  P = softmax(s) per row,  O = P v
#   dv = P^T dO,  dP = dO v^T,  ds = P * (dP - rowsum(P * dP)),
#   dq = ds k / sqrt(d),  dk = ds^T q / sqrt(d).
# Query rows with no kept token have O = 0 and get dq = 0; they add nothing to dk, dv.

def attention_lse(Q: np.ndarray, K: np.ndarray, M: np.ndarray, blk: int) -> np.ndarray:
    """log of the softmax normaliser per query: log sum_{j in J_i} exp(q_i.k_j / sqrt(d)).

    [B, H, N] float64; -inf for queries whose row keeps no block.
    """
    B, H, N, d = Q.shape
    Nb = num_blocks(N, blk)
    L = np.full((B, H, N), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                J = kept_tokens(M[b, h, r], N, blk)
                if J.size == 0:
                    continue
                lo, hi = block_range(r, N, blk)
                s = (Q[b, h, lo:hi].astype(np.float64) @ K[b, h, J].astype(np.float64).T) / np.sqrt(d)
                mx = s.max(axis=1)
                L[b, h, lo:hi] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    return L


def _row_softmax_and_ds(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray):
    """For one set of query rows: P = softmax(q k^T / sqrt(d)) and dS = P (dP - D), where
    dP = g v^T and D = rowsum(P dP) (the chain rule through each row softmax)."""
    d = q.shape[-1]
    s = (q @ k.T) / np.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    P = e / e.sum(axis=1, keepdims=True)
    dP = g @ v.T
    D = (P * dP).sum(axis=1, keepdims=True)
    return P, P * (dP - D)


def _row_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray):
    """(dq, dk, dv) of sum(g * softmax(q k^T / sqrt(d)) v) for one set of query rows."""
    d = q.shape[-1]
    P, ds = _row_softmax_and_ds(q, k, v, g)
    dv = P.T @ g
    dq = (ds @ k) / np.sqrt(d)
    dk = (ds.T @ q) / np.sqrt(d)
    return dq, dk, dv


def attention_bwd(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, M: np.ndarray,
                  blk: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dQ, dK, dV) of sum(dO * attention(Q, K, V, M, blk)), float64."""
    B, H, N, d = Q.shape
    Nb = num_blocks(N, blk)
    dQ = np.zeros((B, H, N, d), dtype=np.float64)
    dK = np.zeros((B, H, N, d), dtype=np.float64)
    dV = np.zeros((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                J = kept_tokens(M[b, h, r], N, blk)
                if J.size == 0:
                    continue
                lo, hi = block_range(r, N, blk)
                dq, dk, dv = _row_attention_bwd(
                    Q[b, h, lo:hi].astype(np.float64), K[b, h, J].astype(np.float64),
                    V[b, h, J].astype(np.float64), dO[b, h, lo:hi].astype(np.float64))
                dQ[b, h, lo:hi] = dq
                dK[b, h, J] += dk
                dV[b, h, J] += dv
    return dQ, dK, dV


def attention_bwd_terms(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, M: np.ndarray,
                        blk: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per element of (dQ, dK, dV): the sum of the absolute values of the products that add
    up to it, float64.  dQ_i sums dS_ij K_j / sqrt(d) over kept keys j, dK_j sums
    dS_ij Q_i / sqrt(d) and dV_j sums P_ij dO_i over the queries i that keep j.

    A backward that rounds every weight P and every dS to relative precision u before its
    products is off by at most u times these sums, plus its own accumulation rounding.  For
    dQ they can exceed |dQ| by far: each row of dS sums to exactly zero, so keys that share a
    large component cancel in dQ but not in its rounding error."""
    B, H, N, d = Q.shape
    Nb = num_blocks(N, blk)
    tQ = np.zeros((B, H, N, d), dtype=np.float64)
    tK = np.zeros((B, H, N, d), dtype=np.float64)
    tV = np.zeros((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r in range(Nb):
                J = kept_tokens(M[b, h, r], N, blk)
                if J.size == 0:
                    continue
                lo, hi = block_range(r, N, blk)
                q = Q[b, h, lo:hi].astype(np.float64)
                k = K[b, h, J].astype(np.float64)
                g = dO[b, h, lo:hi].astype(np.float64)
                P, ds = _row_softmax_and_ds(q, k, V[b, h, J].astype(np.float64), g)
                tQ[b, h, lo:hi] = (np.abs(ds) @ np.abs(k)) / np.sqrt(d)
                tK[b, h, J] += (np.abs(ds).T @ np.abs(q)) / np.sqrt(d)
                tV[b, h, J] += P.T @ np.abs(g)
    return tQ, tK, tV


def attention_bwd_block(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, M: np.ndarray,
                        blk: int, b: int, h: int, r: int):
    """dQ of the query tokens of block r of head (b, h), and that row's contributions to dK
    and dV as (tokens J, dk [|J|, d], dv [|J|, d])."""
    N, d = Q.shape[2], Q.shape[3]
    lo, hi = block_range(r, N, blk)
    J = kept_tokens(M[b, h, r], N, blk)
    if J.size == 0:
        z = np.zeros((0, d), dtype=np.float64)
        return np.zeros((hi - lo, d), dtype=np.float64), J, z, z
    dq, dk, dv = _row_attention_bwd(Q[b, h, lo:hi].astype(np.float64), K[b, h, J].astype(np.float64),
                                    V[b, h, J].astype(np.float64), dO[b, h, lo:hi].astype(np.float64))
    return dq, J, dk, dv


def attention_bwd_flops(M: np.ndarray, N: int, blk: int, d: int) -> float:
    """Algorithmic backward flops: sum over kept tiles of 10 * n_r * n_c * d (the five
    products s, dP, dv, dq, dk at 2 flops per multiply-add)."""
    return 2.5 * kept_tile_flops(M, N, blk, d)


# ------------------------------------------------------------------------ pattern search
# Sparse-vDiT ("Sparse-vDiT: Sparse Attention Acceleration for Video Diffusion
# Transformers"), section 三: the offline search loss and the pattern-selection formula,
# and the per-layer step of "Algorithm 1: Offline Sparse Diffusion Search".  For one layer
# and one set of Q, K, V the search runs full attention (M0) and every candidate pattern,
# scores each candidate by how far its output is from full attention plus a penalty for
# the compute it keeps, and picks a pattern per head.
# Readings where the page is terse:
#   * MSE(O_i - O_0) of a head is the mean of the squared difference over the head's
#     B x N x d output elements (the page's attention output is B x N x d per head).
#   * S_i, the sparsity of pattern i, is the fraction of the N x N (query, key) token pairs
#     it drops, with each kept tile counted at its true size (so M0 -> 0 and M1 -> 1, as
#     the mode table lists).  When the pattern is the same for every batch element this
#     is the same for all heads.
#   * argmin ties go to the lowest candidate index; "L_i > epsilon" is strict.

def pattern_sparsity(pattern: int, param: int, N: int, blk: int) -> float:
    """S_i: fraction of the N*N token pairs that a static pattern does not attend."""
    Nb = num_blocks(N, blk)
    sizes = np.array([block_range(c, N, blk)[1] - block_range(c, N, blk)[0] for c in range(Nb)],
                     dtype=np.int64)
    kept = 0
    for r in range(Nb):
        row = static_row(pattern, param, r, N, blk)
        kept += int(sizes[r]) * int(sizes[row].sum())
    return 1.0 - kept / float(N * N)


def pattern_mse(O_i: np.ndarray, O_0: np.ndarray) -> np.ndarray:
    """MSE(O_i - O_0) per head: mean over (b, n, d) of the squared difference -> [H]."""
    diff = O_i.astype(np.float64) - O_0.astype(np.float64)
    return (diff * diff).mean(axis=(0, 2, 3))


def pattern_loss(mse: np.ndarray, sparsity: np.ndarray, lam: float) -> np.ndarray:
    """L_i = MSE(O_i - O_0) + lam * (1 - S_i); mse [H, n], sparsity [n] -> [H, n]."""
    return mse + lam * (1.0 - np.asarray(sparsity, dtype=np.float64))[None, :]


def select_patterns(L: np.ndarray, eps: float) -> np.ndarray:
    """Pattern choice per head: 0 (full attention, M0) when every candidate's L_i exceeds
    eps, else 1 + the index of the smallest L_i (first one on ties).  L is [H, n]."""
    H, n = L.shape
    choice = np.zeros(H, dtype=np.int64)
    for h in range(H):
        if n == 0 or np.all(L[h] > eps):
            continue
        choice[h] = 1 + int(np.argmin(L[h]))
    return choice


def pattern_search(Q: np.ndarray, K: np.ndarray, V: np.ndarray, blk: int,
                   candidates: Sequence[Tuple[int, int]], lam: float, eps: float,
                   O_0: Optional[np.ndarray] = None, outputs: Optional[Sequence[np.ndarray]] = None):
    """One layer of the offline search.  candidates: static (pattern id, param) pairs, the
    page's M1..M4.  Returns (choice [H], L [H, n], mse [H, n], S [n]).

    O_0 / outputs, when given, are used instead of computing full attention / each
    candidate's attention (to score outputs produced elsewhere with the same rule)."""
    B, H, N, d = Q.shape
    if O_0 is None:
        O_0 = dense_attention(Q, K, V)
    n = len(candidates)
    mse = np.zeros((H, n), dtype=np.float64)
    S = np.zeros(n, dtype=np.float64)
    for i, (pid, prm) in enumerate(candidates):
        S[i] = pattern_sparsity(pid, prm, N, blk)
        if outputs is not None:
            O_i = outputs[i]
        else:
            O_i = attention(Q, K, V, static_mask(B, H, N, blk, [(pid, prm)] * H), blk)
        mse[:, i] = pattern_mse(O_i, O_0)
    L = pattern_loss(mse, S, lam)
    return select_patterns(L, eps), L, mse, S
