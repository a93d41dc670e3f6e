"""GPU parity at the limits the C ABI accepts and at the method's degenerate
cases: the largest hidden size, intermediate size and block count, a single
expert, k = E, and a coreset of one expert.  Routing bit-exact and the FFN
within the bars of tests/parity.py, as everywhere else."""
import numpy as np
import pytest

import sparse_moe_ffn_softmax_amd as cm
import workloads as W
from parity import bits, check, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    pass


def _wl(name, B, R, H, E, k, I, Is, tau=0.9, wt=W.BF16, seed=0):
    return W.Workload(name, B, R, H, E, k, I, Is, W.BF16, wt, tau, seed=seed)


def test_max_hidden():
    # H = 16384: router chunks of 2048 in 32 slices (the loop schedule), the
    # gate/up waves take 4096 of H each (32 stages)
    check(W.generate(_wl("max_hidden", 1, 8, 16384, 16, 4, 128, 128, seed=201)), threads=16)


def test_max_inter():
    # I = Is = 8192: the down GEMM runs 64 stages; gate/up 1024 column slices
    check(W.generate(_wl("max_inter", 2, 8, 128, 16, 4, 8192, 8192, seed=202)), threads=16)


@pytest.mark.parametrize("name,shape", [
    ("max_hidden_panels", (1, 8, 16384, 16, 4, 128, 128)),
    ("max_inter_panels", (2, 8, 128, 16, 4, 8192, 8192)),
    ("max_hidden_fp4_panels", (1, 8, 16384, 16, 4, 128, 128)),
])
def test_limits_on_panel_weights(name, shape):
    """The largest panel shapes (rows of 16384 bf16 elements, 8192-row down
    matrices, 4-bit rows of 8 KiB) give the row-major call's output bit for
    bit."""
    wt = W.FP4 if "fp4" in name else W.BF16
    wl = _wl(name, *shape, wt=wt, seed=205)
    inp = W.generate(wl)
    out_r, rt_r = run_gpu(inp, wl.mass_threshold, wl.top_k)
    out_p, rt_p = run_gpu(inp, wl.mass_threshold, wl.top_k, dp=cm.upload(inp, layout="panels"))
    np.testing.assert_array_equal(bits(rt_p["topk_idx"]), bits(rt_r["topk_idx"]))
    np.testing.assert_array_equal(bits(out_p), bits(out_r))


def test_max_blocks():
    # 1024 blocks of 8 rows (8192 rows): 1024 routing workgroups, the
    # many-block permutation, 128-row tiles; FFN on every row
    inp = W.generate(_wl("max_blocks", 1024, 8, 128, 16, 2, 128, 128, seed=203))
    check(inp, threads=16)


def test_max_blocks_fp8():
    inp = W.generate(_wl("max_blocks_fp8", 1024, 8, 256, 16, 2, 128, 128, wt=W.FP8, seed=204))
    check(inp, threads=16)


def test_single_expert():
    # E = k = 1: every row takes expert 0 with gate 1
    _, _, ref = check(W.generate(_wl("single_expert", 2, 8, 128, 1, 1, 128, 128, seed=205)))
    assert np.all(ref["topk_idx"] == 0) and np.all(ref["gates"] == 1.0)


@pytest.mark.parametrize("tau", [1.0, 0.5])
def test_k_equals_e(tau):
    # k = E = 8: at tau 1 every row takes every expert
    _, _, ref = check(W.generate(_wl("k_eq_e", 2, 16, 256, 8, 8, 128, 128, tau=tau, seed=206)))
    if tau == 1.0:
        assert np.all(np.sort(ref["topk_idx"], axis=1) == np.arange(8))


def test_coreset_of_one_expert():
    # a threshold far below one expert's share: the coreset is the heaviest
    # expert alone, every row takes it with gate 1 and the other slots are empty
    _, _, ref = check(W.generate(_wl("coreset_one", 2, 32, 256, 32, 8, 128, 128, tau=1e-6, seed=207)))
    assert np.all(ref["coreset_size"] == 1)
    assert np.all(ref["gates"][:, 0] == 1.0) and np.all(ref["topk_idx"][:, 1:] == -1)
