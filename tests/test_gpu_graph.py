"""GPU: the library's calls can be captured in a HIP graph and replayed.

Nothing in the library allocates, synchronizes or records a memset, so a step (adaptive
mask build + attention forward, then the backward) captured once must give, on every
replay, bit-identical results to the same calls run eagerly.  Replays are separated by
eager work that overwrites the outputs and by synchronizations.
"""
import pytest
import torch

import gen
from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_captured_step_replays_match_eager(asa_lib, dtype):
    """bf16 inputs take the LDS-ring kernels of both passes; fp32 inputs take the fp32
    matrix-core backward, which reads its operands straight from global memory."""
    asa = asa_lib
    cfg = gen.scaled(gen.WAN, H=2, frames=2)
    cfg.k = 4
    B, H, N, d, blk = cfg.B, cfg.H, cfg.N, cfg.d, cfg.blk
    say(f"case {cfg.name} ({dtype}): graph capture of mask build + forward + backward")
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = {k: v.to(tdt) for k, v in to_device(gen.make_inputs(cfg)).items()}
    g = torch.Generator().manual_seed(11)
    dout = torch.randn((B, H, N, d), generator=g).to(tdt).to(dev)
    rows = B * H * cfg.Nb
    rp = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(asa.asa_csr_capacity(B, H, N, blk), dtype=torch.int32, device=dev)
    order = torch.empty(rows, dtype=torch.int32, device=dev)
    shp = asa.asa_shape(B, H, N, d, blk, asa.ASA_BF16 if dtype == "bf16" else asa.ASA_F32)
    import ctypes
    mws = torch.empty(int(asa.lib.asa_build_mask_workspace_size(ctypes.byref(shp))), dtype=torch.uint8, device=dev)
    bws = torch.empty(int(asa.lib.asa_attention_bwd_workspace_size(ctypes.byref(shp))), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))

    def step():
        asa.asa_build_mask(x["q"], x["k"], blk, asa.TOPK, k_top=cfg.k, keep_diag=1, out=(rp, ci, order),
                           workspace=mws)
        asa.asa_attention_fwd(x["q"], x["k"], x["v"], rp, ci, blk, order=order, lse=lse, out=out)
        asa.asa_attention_bwd(x["q"], x["k"], x["v"], out, dout, lse, rp, ci, blk, grads=grads, workspace=bws)

    step()
    torch.cuda.synchronize()
    n = int(rp[-1].item())
    ref = [t.clone() for t in (rp, ci[:n], order, out, lse, *grads)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (rp, ci, order, out, lse, *grads):   # eager work between replays
            t.fill_(-7 if t.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [rp, ci[:n], order, out, lse, *grads]
        for name, a, b in zip(("row_ptr", "col_idx", "order", "O", "lse", "dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
    say("  3 replays bit-identical to the eager step")
