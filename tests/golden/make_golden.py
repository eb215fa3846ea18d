"""Write the stored oracle outputs under tests/golden/ (calls the oracle only).

Usage: python tests/golden/make_golden.py
Writes tiny_asa_mask.json: the float64 oracle's CSR mask for the seeded 1024-token
adaptive case (top-4 of 16 key blocks plus the diagonal, two heads).  The GPU mask
builder must reproduce it bit for bit; the CPU suite checks that the oracle still does.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import oracle as O  # noqa: E402


def tiny_mask():
    cfg = gen.TINY
    x = gen.make_inputs(cfg)
    q64, k64 = gen.as_float64(x["q"]), gen.as_float64(x["k"])
    M = O.build_mask(q64, k64, cfg.blk, mode=cfg.mode, k=cfg.k, keep_diag=cfg.keep_diag)
    rp, ci = O.to_csr(M)
    return {"config": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "blk": cfg.blk, "k": cfg.k,
            "row_ptr": [int(v) for v in rp], "col_idx": [int(v) for v in ci]}


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_asa_mask.json"), "w") as f:
        json.dump(tiny_mask(), f)
        f.write("\n")
    print("wrote tiny_asa_mask.json")
