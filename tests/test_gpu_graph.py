"""A call captured in a HIP graph against the same call made eagerly.

A call queues only kernels on the caller's stream (no memset, no host
synchronisation, no allocation), so it can be captured.  The replays must
reproduce the eager outputs and routing bit for bit, every time, with eager
work clobbering the outputs between replays.
"""
import numpy as np
import pytest

import sparse_moe_ffn_softmax_amd as cm
import workloads as W
from test_gpu_parity import FEW, MID

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl,layout", [
    (MID.with_(name="graph_mid_tiled", seed=131), "rows"),                     # tiled GEMMs (16 rows per expert)
    (FEW.with_(name="graph_few_register", seed=132), "rows"),                  # register GEMMs (one row tile)
    (MID.with_(name="graph_mid_noshared", shared_inter=0, seed=133), "rows"),  # no shared expert
    (MID.with_(name="graph_mid_tiled_panels", seed=134), "panels"),            # MFMA-panel weights
    (FEW.with_(name="graph_few_register_panels", seed=135), "panels"),
    # many-row kernels: 128-row tiles (16-wave gate/up, persistent down) and
    # fp8 weights on a few blocks (32-row tiles), with fp8 activations too
    (MID.with_(name="graph_t128_fp8", num_blocks=8, block_rows=32, num_experts=16, hidden=512, inter=512,
               shared_inter=512, weight_dtype=W.FP8, seed=136), "panels"),
    (MID.with_(name="graph_t128_fp8_act8", num_blocks=8, block_rows=32, num_experts=16, hidden=512, inter=512,
               shared_inter=512, weight_dtype=W.FP8, seed=137), "panels"),
    (MID.with_(name="graph_few_blocks_fp8", num_blocks=2, block_rows=32, num_experts=256, hidden=512, inter=512,
               shared_inter=512, weight_dtype=W.FP8, seed=138), "rows"),
], ids=lambda v: v.name if hasattr(v, "name") else v)
def test_graph_replay_matches_eager(wl, layout):
    import torch
    inp = W.generate(wl)
    K, tau = wl.top_k, wl.mass_threshold
    dp = cm.upload(inp, layout=layout)
    ws = cm.alloc_workspace(dp.problem, K)
    rt_t, rt = cm.alloc_routing(dp.problem, K)
    out = torch.empty((wl.rows, wl.hidden), dtype=torch.bfloat16, device="cuda")
    x = dp.tensors["x"]
    opts = cm.make_options(activation_fp8=1) if wl.name.endswith("_act8") else None

    cm.clover_moe_block_forward(dp.problem, dp.weights, x, tau, K, out, rt, ws, options=opts)
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_rt = {k: v.clone() for k, v in rt_t.items()}

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        cm.clover_moe_block_forward(dp.problem, dp.weights, x, tau, K, out, rt, ws, options=opts)
    torch.cuda.synchronize()

    for replay in range(3):
        # eager work between the replays: clobber every output
        out.fill_(768.0)
        for v in rt_t.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {replay}: out"
        for k, v in rt_t.items():
            a, b = v.cpu().numpy(), ref_rt[k].cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {replay}: {k}"
    # and an eager call after the replays still agrees
    out.fill_(768.0)
    cm.clover_moe_block_forward(dp.problem, dp.weights, x, tau, K, out, rt, ws, options=opts)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
