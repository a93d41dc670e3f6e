"""clover_moe_block_forward_noalloc, the entry point for callers that cannot
allocate: its workspace is the library's static per-GPU scratch array.  It
must give the workspace entry point's results bit for bit (same kernels, same
plan), call after call on the one shared array, largest call first so that the
later, smaller calls run over what the earlier ones left behind."""
import ctypes

import numpy as np
import pytest

import sparse_moe_ffn_softmax_amd as cm
import workloads as W
from parity import SENTINEL, assert_ffn_close, assert_routing_equal, bits

import oracle


def _call_both(inp, tau, top_k):
    """The same call through clover_moe_block_forward_ex (a fresh torch
    workspace) and through clover_moe_block_forward_noalloc; returns both
    outputs and routing dicts."""
    import torch
    wl = inp.wl
    dp = cm.upload(inp)
    opts = None
    if wl.expert_budget or dp.tensors.get("live_rows") is not None:
        opts = cm.make_options(wl.expert_budget, dp.tensors.get("live_rows"))
    odt = torch.bfloat16 if wl.act_dtype == W.BF16 else torch.float32
    res = []
    for noalloc in (False, True):
        rt_t, rt = cm.alloc_routing(dp.problem, top_k)
        out = torch.full((wl.rows, wl.hidden), SENTINEL, dtype=odt, device="cuda")
        if noalloc:
            cm.clover_moe_block_forward_noalloc(dp.problem, dp.weights, dp.tensors["x"], tau, top_k, out,
                                                rt, options=opts)
        else:
            ws = cm.alloc_workspace(dp.problem, top_k)
            cm.clover_moe_block_forward(dp.problem, dp.weights, dp.tensors["x"], tau, top_k, out, rt, ws,
                                        options=opts)
        torch.cuda.synchronize()
        res.append((out.double().cpu().numpy(), {k: v.cpu().numpy() for k, v in rt_t.items()}))
    return res


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_on_successive_smaller_calls(require_gpu):
    """64 blocks of fp8 (92 MiB of workspace), then one 32-row bf16 block, then
    a one-row decode with live rows and a budget-free full route: each through
    both entry points, in that order on the one scratch array."""
    calls = [
        (W.generate(W.WORKLOADS["blocks64_fp8"]), None, None),
        (W.generate(W.WORKLOADS["block32_bf16"]), None, None),
        (W.generate(W.WORKLOADS["block32_budget64_live50"]), None, None),
        (W.generate(W.WORKLOADS["decode1_bf16"]), 1.0, 8),
    ]
    for inp, tau, k in calls:
        wl = inp.wl
        tau = wl.mass_threshold if tau is None else tau
        k = wl.top_k if k is None else k
        print(f"[noalloc] {wl.name} B={wl.num_blocks} R={wl.block_rows} tau={tau} k={k}", flush=True)
        (out_ws, rt_ws), (out_na, rt_na) = _call_both(inp, tau, k)
        assert_routing_equal(rt_na, rt_ws)
        np.testing.assert_array_equal(bits(out_na), bits(out_ws))
    # the last (smallest) call against the oracle, to the parity bar
    ref = oracle.forward(inp, tau=tau, top_k=k)
    assert_routing_equal(rt_na, ref)
    assert_ffn_close(out_na, ref["out"], inp.wl.weight_dtype)


@pytest.mark.gpu
def test_noalloc_repeated_calls_are_identical(require_gpu):
    """Two calls in a row on the same inputs give the same bytes: nothing of
    the earlier call's scratch contents leaks into the next."""
    inp = W.generate(W.WORKLOADS["tiny_fp32"].with_(num_blocks=3, seed=301))
    (_, _), (o1, r1) = _call_both(inp, 0.9, 4)
    (_, _), (o2, r2) = _call_both(inp, 0.9, 4)
    assert_routing_equal(r2, r1)
    np.testing.assert_array_equal(bits(o2), bits(o1))


def test_noalloc_rejects_problems_beyond_its_scratch():
    """512 blocks at the model's shapes need about 740 MB of workspace: refused
    with CMOE_ERR_WORKSPACE before any HIP call (fake device addresses)."""
    p = cm.make_problem(2048, 256, 512, 512, 32, 512, "bf16", "fp8_e4m3")
    assert cm.clover_moe_workspace_size(p, 8) > cm.NOALLOC_MAX_WORKSPACE
    base, step = 0x7F0000000000, 1 << 36
    w = cm.make_weights(router_w=base + step, w13=base + 2 * step, w2=base + 3 * step,
                        shared_w13=base + 4 * step, shared_w2=base + 5 * step, w13_scale=base + 6 * step,
                        w2_scale=base + 7 * step, shared_w13_scale=base + 8 * step,
                        shared_w2_scale=base + 9 * step)
    lib = cm.load_library()
    st = lib.clover_moe_block_forward_noalloc(ctypes.byref(p), ctypes.byref(w), base + 10 * step,
                                              ctypes.c_float(0.9), 8, None, base + 11 * step, None, None)
    assert st == cm.CMOE_ERR_WORKSPACE
    assert "no-allocation" in cm.clover_moe_last_error()
    # an invalid problem is refused the same way as by the other entry points
    bad = cm.make_problem(2048, 256, 512, 512, 24, 1, "bf16", "bf16")
    st = lib.clover_moe_block_forward_noalloc(ctypes.byref(bad), ctypes.byref(w), base + 10 * step,
                                              ctypes.c_float(0.9), 8, None, base + 11 * step, None, None)
    assert st == cm.CMOE_ERR_UNSUPPORTED
