"""GPU: asa_build_mask_noalloc (workspace in the library's static device scratch) against
asa_build_mask (caller workspace), through the C ABI.

Two calls in a row on one device, the second with a smaller input, so the second call
runs on scratch the first one filled: the CSR and the schedule must match asa_build_mask's
bit for bit each time (integer outputs).  A shape whose workspace exceeds the scratch is
rejected before anything runs.
"""
import pytest
import torch

import gen
from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


def _case(cfg, asa, mode_kw):
    x = to_device(gen.make_inputs(cfg))
    ref = asa.asa_build_mask(x["q"], x["k"], cfg.blk, cfg.mode, with_order=True, **mode_kw)
    rows = cfg.B * cfg.H * cfg.Nb
    out = (torch.full((rows + 1,), -7, dtype=torch.int32, device="cuda:0"),
           torch.full((ref[1].numel(),), -7, dtype=torch.int32, device="cuda:0"),
           torch.full((rows,), -7, dtype=torch.int32, device="cuda:0"))
    got = asa.asa_build_mask_noalloc(x["q"], x["k"], cfg.blk, cfg.mode, out=out, **mode_kw)
    torch.cuda.synchronize()
    n = int(ref[0][-1].item())
    assert torch.equal(got[0], ref[0]), "row_ptr differs"
    assert torch.equal(got[1][:n], ref[1][:n]), "col_idx differs"
    assert torch.equal(got[2], ref[2]), "order differs"
    say(f"  {cfg.name}: {n} kept tiles, identical to asa_build_mask")


def test_noalloc_matches_build_mask_twice(asa_lib):
    asa = asa_lib
    big = gen.scaled(gen.LONG720, H=6, frames=6, name_suffix="_noalloc_big")     # Nb = 169
    big.k = 9
    small = gen.scaled(gen.COGVIDEOX, H=3, frames=2, name_suffix="_noalloc_small")
    say(f"case noalloc: {big.name} then {small.name}")
    _case(big, asa, dict(k_top=big.k, patterns=big.patterns))
    _case(small, asa, dict(tau=small.tau, k_cap=8, n_text=small.n_text))


def test_noalloc_rejects_shapes_beyond_scratch(asa_lib):
    asa = asa_lib
    q = torch.zeros((2, 24, 75600, 128), dtype=torch.bfloat16, device="cuda:0")
    rows = 2 * 24 * 591
    out = (torch.zeros(rows + 1, dtype=torch.int32, device="cuda:0"),
           torch.zeros(rows * 591, dtype=torch.int32, device="cuda:0"))
    with pytest.raises(asa.AsaError) as ei:
        asa.asa_build_mask_noalloc(q, q, 128, asa.TOPK, k_top=4, out=out)
    assert ei.value.status == -6
    torch.cuda.synchronize()
