"""Shared helpers for the GPU parity tests (comparison logic only; no method arithmetic)."""
import sys

import numpy as np
import torch

import gen
import oracle as O

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: dict, device="cuda:0"):
    return {k: v.to(device).contiguous() for k, v in x.items()}


def oracle_inputs(x: dict):
    return gen.as_float64(x["q"]), gen.as_float64(x["k"]), gen.as_float64(x["v"])


def gpu_csr_rows(row_ptr: torch.Tensor, col_idx: torch.Tensor):
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    return rp, ci


def csr_to_device(M: np.ndarray, device="cuda:0"):
    rp, ci = O.to_csr(M)
    if ci.size == 0:
        ci = np.zeros(1, dtype=np.int64)          # the ABI takes a non-NULL array
    return (torch.from_numpy(rp.astype(np.int32)).to(device),
            torch.from_numpy(np.ascontiguousarray(ci.astype(np.int32))).to(device))


def compare_masks(rp, ci, M, details=None, amb=None, mode=O.TOPK, k=0, tau=0.0, k_cap=0,
                  gap=O.AMBIGUITY_GAP):
    """GPU CSR vs oracle block mask: bit-exact except logged ambiguous rows.

    In an ambiguous row the GPU may keep a different one of the near-tied blocks.  Such
    a row must still hold every block the oracle keeps outside the adaptive prefix, and
    every block on which the two disagree must have a block score within `gap` of the
    oracle's last-kept or first-dropped candidate.  Returns the differing rows.
    """
    orp, oci = O.to_csr(M)
    rows = M.reshape(-1, M.shape[-1])
    Nb = M.shape[-1]
    assert rp.shape == orp.shape, "row_ptr length"
    assert rp[0] == 0
    if np.array_equal(rp, orp) and np.array_equal(ci, oci):
        return []
    diff_rows = []
    for n in range(rows.shape[0]):
        g = ci[rp[n]:rp[n + 1]]
        assert np.all(np.diff(g) > 0), f"row {n}: col_idx not strictly ascending"
        assert g.size == 0 or (g[0] >= 0 and g[-1] < Nb), f"row {n}: col_idx out of range"
        o = np.nonzero(rows[n])[0]
        if g.size == o.size and np.array_equal(g, o):
            continue
        assert amb is not None and details is not None and amb.reshape(-1)[n], \
            f"row {n}: GPU {g.tolist()} vs oracle {o.tolist()} (not an ambiguous row)"
        srow = details["S"].reshape(-1, Nb)[n]
        prow = details["P"].reshape(-1, Nb)[n]
        order = O.rank_order(prow)
        m = O.adaptive_count(prow, order, mode, k, tau, k_cap)
        edge = [srow[order[t]] for t in (m - 1, m) if 0 <= t < Nb]
        for c in np.setxor1d(g, o):
            assert min(abs(srow[c] - e) for e in edge) < gap, \
                f"row {n}: block {c} differs but is not near the selection boundary"
        if mode == O.TOPK:
            assert g.size == o.size, f"row {n}: kept count differs in top-k mode"
        else:
            assert abs(int(g.size) - int(o.size)) <= 1, f"row {n}: kept count differs by more than one"
        diff_rows.append(n)
    return diff_rows


def compare_outputs(got: np.ndarray, want: np.ndarray, fp32: bool, label: str):
    err = np.abs(got.astype(np.float64) - want)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say(f"  [{label}] max abs err {mx:.3e}  mean abs err {mean:.3e}  (n={err.size})")
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    if fp32:
        assert mx <= F32_MAX_ABS, f"{label}: max abs err {mx} > {F32_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{label}: max abs err {mx} > {BF16_MAX_ABS}"
        assert mean <= BF16_MEAN_ABS, f"{label}: mean abs err {mean} > {BF16_MEAN_ABS}"
    return mx, mean


def sample_rows(cfg, n_per_head: int, seed: int, heads=None):
    """Query tokens (b, h, i) to check at full size: random ones plus both ends and the ragged tail."""
    rng = np.random.default_rng(1000 + seed)
    heads = range(cfg.H) if heads is None else heads
    rows = []
    tail_lo = (cfg.Nb - 1) * cfg.blk
    for b in range(cfg.B):
        for h in heads:
            picks = set(rng.integers(0, cfg.N, n_per_head).tolist())
            picks |= {0, cfg.blk - 1, cfg.N - 1, tail_lo, min(cfg.N - 1, tail_lo + 7)}
            rows += [(b, h, int(i)) for i in sorted(picks)]
    return rows
