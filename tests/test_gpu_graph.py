"""The library's calls are capture-safe (no allocation, no memset node, no
host synchronization): a whole MoE layer step captured into a HIP graph and
replayed gives the same bits as the eager step, on every replay, with other
eager work on the device between the replays."""
import numpy as np
import pytest

from helpers import assert_bits_equal, to_gpu, to_np
from qat_nvfp4_quantize_amd import inputs

pytestmark = pytest.mark.gpu


def test_moe_layer_step_replays_match_eager():
    import torch

    from qat_nvfp4_quantize_amd import nvq

    s = inputs.small_moe(wid=106, T=200, H=256, E=8, I=128, topk=2, k=16)
    logits = to_gpu(inputs.logits(s))
    x = to_gpu(inputs.activations(s))
    qgu = nvq.nvfp4_quantize(to_gpu(inputs.weights(s, "gu")))[:3]
    qdn = nvq.nvfp4_quantize(to_gpu(inputs.weights(s, "dn")))[:3]
    L = nvq.load()
    dev = x.device
    ws_q1 = nvq.workspace(L.nvfp4_quantize_workspace_bytes(1, s.T, s.H), dev)
    ws_q2 = nvq.workspace(L.nvfp4_quantize_workspace_bytes(1, s.P, s.I), dev)
    ws_g = nvq.workspace(max(L.moe_gemm_workspace_bytes(s.P, s.E, 2 * s.I, s.k),
                             L.moe_gemm_workspace_bytes(s.P, s.E, s.H, s.k)), dev)
    h_amax = torch.zeros(1, dtype=torch.float32, device=dev)

    def step():
        ids, w = nvq.nvq_moe_route(logits, s.topk)
        sp, off, pos, _ = nvq.nvq_moe_permute(ids, s.E)
        qx = nvq.nvfp4_quantize(x, score=True, ws=ws_q1)
        idx1, r1, _ = nvq.residual_topk_channels(x, *qx[:3], s.k, scores=qx[3])
        h, _ = nvq.moe_grouped_gemm_w4a4_comp(qx[0], qx[1], qx[2], *qgu, off, rows=s.P, a_row=sp,
                                              a_row_div=s.topk, a_resid=r1, comp_idx=idx1,
                                              epilogue=nvq.NVQ_EPI_SWIGLU, ws=ws_g, h_amax=h_amax)
        qh = nvq.nvfp4_quantize(h, amax_in=h_amax, score=True, ws=ws_q2)
        idx2, r2, _ = nvq.residual_topk_channels(h, *qh[:3], s.k, scores=qh[3])
        y2, _ = nvq.moe_grouped_gemm_w4a4_comp(qh[0], qh[1], qh[2], *qdn, off, rows=s.P,
                                               a_resid=r2, comp_idx=idx2, ws=ws_g)
        return h, qh[0], nvq.nvq_moe_combine(y2, pos, w)

    eager = [to_np(t) for t in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the allocator outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for got, ref, what in zip(outs, eager, ("h", "codes of h", "layer output")):
            assert_bits_equal(to_np(got), ref, f"replay {rep}: {what}")
        # other eager work between replays, overwriting the shared workspaces
        step()
        torch.cuda.synchronize()
