"""GPU parity of the frame-tile static pattern (ASA_PAT_FRAME_TILE: each query frame keeps its
own frame and the first frame) against the float64 oracle.

Masks must match oracle.static_mask / oracle.build_mask bit for bit (adaptive rows flagged
ambiguous by the oracle excepted, as for the other sources); attention on the oracle's
mask must meet the forward's bound; the pattern search must price the pattern with the
oracle's sparsity.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_helpers import (compare_masks, compare_outputs, csr_to_device, gpu_csr_rows, oracle_inputs, say,
                         to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,blk,F", [(1000, 64, 100), (4097, 128, 1024), (2600, 128, 300), (700, 64, 700)])
def test_frame_tile_static_mask(asa_lib, N, blk, F):
    asa = asa_lib
    pats = [(gen.FRAME_TILE, F), (gen.DIAG, 0), (gen.FRAME_TILE, 1), (gen.FRAME_TILE, 4 * N)]
    say(f"case frame tile static N={N} blk={blk} F={F}")
    rp_t, ci_t = asa.asa_static_mask(2, len(pats), N, blk, pats, "cuda:0")
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    M = O.static_mask(2, len(pats), N, blk, pats)
    orp, oci = O.to_csr(M)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


def test_frame_tile_with_adaptive_and_attention(asa_lib):
    """Adaptive top-k unioned with frame tiles of one latent frame, then attention."""
    asa = asa_lib
    cfg = replace(gen.scaled(gen.WAN, H=3, frames=3), name="frame_tile_union")
    cfg.k = 3
    frame = cfg.Hs * cfg.Ws
    cfg.patterns = [(gen.FRAME_TILE, frame), (gen.ADAPTIVE, 0), (gen.FRAME_TILE, frame)]
    x = gen.make_inputs(cfg)
    xd = to_device(x)
    q64, k64, v64 = oracle_inputs(x)
    M, det = O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, n_text=0, keep_diag=1,
                          patterns=cfg.patterns, return_details=True)
    rp_t, ci_t = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, keep_diag=1,
                                    patterns=cfg.patterns)
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    amb = O.ambiguous_rows(det["S"], det["P"], mode=cfg.mode, k=cfg.k)
    diff = compare_masks(rp, ci, M, det, amb, cfg.mode, cfg.k)
    say(f"  mask density {O.density(M):.4f}, differing (ambiguous) rows {len(diff)}")
    rpo, cio = csr_to_device(M)
    out = asa.asa_attention_fwd(xd["q"], xd["k"], xd["v"], rpo, cio, cfg.blk, patterns=cfg.patterns)
    torch.cuda.synchronize()
    compare_outputs(out.cpu().numpy(), O.attention(q64, k64, v64, M, cfg.blk), False, cfg.name)


def test_frame_tile_search_candidate(asa_lib):
    """The search accepts the pattern and charges lam * (1 - S) with the oracle's S."""
    asa = asa_lib
    cfg = replace(gen.scaled(gen.STATIC, H=2, frames=2), name="frame_tile_search")
    frame = cfg.Hs * cfg.Ws
    cands = [(gen.FRAME_TILE, frame), (gen.DIAG, 0)]
    x = to_device(gen.make_inputs(cfg))
    choice, loss, mse = asa.asa_pattern_search(x["q"], x["k"], x["v"], cfg.blk, cands)
    torch.cuda.synchronize()
    S = np.array([O.pattern_sparsity(p, q, cfg.N, cfg.blk) for p, q in cands])
    pen = (loss - mse).cpu().numpy()
    assert np.all(np.abs(pen - 0.01 * (1.0 - S)[None, :]) <= 1e-15)
    assert np.array_equal(choice.cpu().numpy(), O.select_patterns(loss.cpu().numpy(), 0.1))
