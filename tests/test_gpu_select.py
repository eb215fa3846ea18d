"""GPU parity of the adaptive selection in asa_build_mask over every padded row width and
the boundary values of k, tau and k_cap.

Each wavefront ranks one row: top-k by a pivot select for the k-th largest packed key, the
mass prefix by a bitonic sort of the packed keys.  Row widths Nb from 1 to 1024 cover every
padded width (64, 128, 256, 512, 1024 slots) with full and partly filled lanes.  Every case
compares the GPU CSR with oracle.build_mask bit for bit, except rows the oracle flags as
ambiguous (near-tied block scores, or a prefix mass within the gap of tau), which may differ
only among near-tied blocks (gpu_helpers.compare_masks).
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import compare_masks, gpu_csr_rows, oracle_inputs, say, to_device

pytestmark = pytest.mark.gpu

# (Nb, blk, d, structure): N = Nb * blk minus a ragged tail where Nb > 1
WIDTHS = [(1, 64, 64, "none"), (2, 128, 64, "none"), (63, 64, 64, "lowrank"), (64, 64, 128, "none"),
          (65, 64, 64, "smooth"), (200, 64, 64, "none"), (300, 64, 64, "lowrank"), (591, 64, 64, "none"),
          (1024, 64, 64, "none")]


def _config(Nb, blk, d, structure):
    N = Nb * blk - (13 if Nb > 1 else blk - 50)
    return gen.Config(name=f"select_nb{Nb}", seed=40 + Nb, B=1, H=2, N=N, d=d, blk=blk, dtype="bf16",
                      frames=1, Hs=1, Ws=N, structure=structure, mode=gen.TOPK, k=1)


def _check(asa, xd, q64, k64, blk, mode, k, tau, k_cap, keep_diag):
    M, det = O.build_mask(q64, k64, blk, mode=mode, k=k, tau=tau, k_cap=k_cap, n_text=0,
                          keep_diag=keep_diag, return_details=True)
    rp_t, ci_t = asa.asa_build_mask(xd["q"], xd["k"], blk, mode, k_top=k, tau=tau, k_cap=k_cap, n_text=0,
                                    keep_diag=keep_diag)
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    amb = O.ambiguous_rows(det["S"], det["P"], mode=mode, k=k, tau=tau, k_cap=k_cap)
    diff = compare_masks(rp, ci, M, det, amb, mode, k, tau, k_cap)
    return int(amb.sum()), len(diff)


@pytest.mark.parametrize("Nb,blk,d,structure", WIDTHS, ids=lambda v: str(v))
def test_selection_sweep(asa_lib, Nb, blk, d, structure):
    asa = asa_lib
    cfg = _config(Nb, blk, d, structure)
    assert cfg.Nb == Nb
    say(f"case {cfg.name}: N={cfg.N} blk={blk} d={d} {structure}")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, _ = oracle_inputs(x)
    ks = sorted({0, 1, 2, Nb // 3, max(Nb - 1, 0), Nb, Nb + 5})
    n_amb = n_diff = 0
    for i, k in enumerate(ks):
        a, b = _check(asa, xd, q64, k64, blk, gen.TOPK, k, 0.0, 0, i % 2)
        n_amb += a
        n_diff += b
    for i, (tau, k_cap) in enumerate([(0.0, 0), (0.5, 0), (0.9, 7), (0.999, 0), (1.0, 0), (0.99, Nb + 3)]):
        a, b = _check(asa, xd, q64, k64, blk, gen.TAU, 0, tau, k_cap, (i + 1) % 2)
        n_amb += a
        n_diff += b
    say(f"  {len(ks)} top-k and 6 mass-prefix settings: ambiguous rows {n_amb}, differing rows {n_diff}")


@pytest.mark.parametrize("d", [64, 128])
def test_selection_thirteen_row_tiles(asa_lib, d):
    """12 heads x 256 blocks is fewer than one 16-row workgroup per compute unit, so the
    builder takes 13 rows per workgroup: the last pass of a workgroup holds one real row
    (and at d = 64, where a wavefront sorts two rows side by side, one row of the next
    tile that it must not write).  Top-k and the mass prefix, bit for bit against the
    oracle except near-tie rows."""
    asa = asa_lib
    cfg = gen.Config(name=f"select_13rows_d{d}", seed=77 + d, B=1, H=12, N=256 * 64 - 13, d=d, blk=64,
                     dtype="bf16", frames=1, Hs=1, Ws=256 * 64 - 13, structure="smooth", mode=gen.TOPK, k=1)
    assert cfg.Nb == 256 and cfg.B * cfg.H * ((cfg.Nb + 15) // 16) < 256   # 16-row workgroups
    say(f"case {cfg.name}: N={cfg.N} blk=64 d={d}")
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, _ = oracle_inputs(x)
    n_amb = n_diff = 0
    for mode, k, tau, k_cap, diag in ((gen.TOPK, 26, 0.0, 0, 1), (gen.TOPK, 3, 0.0, 0, 0),
                                      (gen.TAU, 0, 0.9, 0, 1), (gen.TAU, 0, 0.5, 20, 0)):
        a, b = _check(asa, xd, q64, k64, 64, mode, k, tau, k_cap, diag)
        n_amb += a
        n_diff += b
    say(f"  ambiguous rows {n_amb}, differing rows {n_diff}")
