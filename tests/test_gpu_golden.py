"""GPU: the mask builder reproduces the stored oracle mask for the seeded 1024-token
adaptive case bit for bit (tests/golden/tiny_asa_mask.json, written from the oracle by
tests/golden/make_golden.py)."""
import json
import os

import numpy as np
import pytest
import torch

import gen
from gpu_helpers import gpu_csr_rows, say, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_gpu_mask_matches_stored_oracle_mask(asa_lib):
    asa = asa_lib
    want = json.load(open(os.path.join(GOLDEN, "tiny_asa_mask.json")))
    cfg = gen.TINY
    say(f"case {cfg.name}: GPU mask against the stored oracle mask")
    xd = to_device(gen.make_inputs(cfg))
    rp_t, ci_t = asa.asa_build_mask(xd["q"], xd["k"], cfg.blk, cfg.mode, k_top=cfg.k, keep_diag=cfg.keep_diag)
    torch.cuda.synchronize()
    rp, ci = gpu_csr_rows(rp_t, ci_t)
    assert np.array_equal(rp, np.array(want["row_ptr"]))
    assert np.array_equal(ci, np.array(want["col_idx"]))
