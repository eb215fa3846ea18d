"""Stored fixtures under tests/golden/ (CPU).

* sparse_vdit_table3.json holds the page's Table 3 settings; the search pins read it.
* tiny_asa_mask.json was written by tests/golden/make_golden.py from the float64 oracle;
  the oracle must still produce it exactly (the GPU mask builder is held to the same file
  by tests/test_gpu_golden.py).
"""
import json
import os

import numpy as np

import gen
import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_table3_fixture_is_well_formed():
    rows = json.load(open(os.path.join(GOLDEN, "sparse_vdit_table3.json")))["rows"]
    assert len(rows) == 4
    assert {(r["lambda"], r["epsilon"]) for r in rows} == {(0.01, 0.1), (0.005, 0.1), (0.01, 0.05), (0.01, 0.15)}
    assert all(r["speedup"] > 1.0 for r in rows)


def test_oracle_reproduces_the_stored_tiny_mask():
    want = json.load(open(os.path.join(GOLDEN, "tiny_asa_mask.json")))
    cfg = gen.TINY
    x = gen.make_inputs(cfg)
    M = O.build_mask(gen.as_float64(x["q"]), gen.as_float64(x["k"]), cfg.blk, mode=cfg.mode, k=cfg.k,
                     keep_diag=cfg.keep_diag)
    rp, ci = O.to_csr(M)
    assert rp.tolist() == want["row_ptr"]
    assert ci.tolist() == want["col_idx"]
    # top-4 plus the diagonal: 4 or 5 blocks per row
    assert set(np.diff(rp).tolist()) <= {4, 5}
