"""GPU parity of the opt-in fp8-activation path (cmoe_options.activation_fp8:
MXFP8 activations into the fp8-weight expert GEMMs).  Each call is held to
the oracle's fp8-activation reading at the bf16 bar (max|d| <= 2e-2
max|ref|, sum|d| <= 5e-3 sum|ref|) and to the exact oracle at the fp8-weight bar (max|d| <= 6e-2
max|ref|); see tests/parity.py.  Routing is unchanged by the option and
stays bit-exact."""
import pytest

import sparse_moe_ffn_softmax_amd as cm
import workloads as W
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    pass


def _report(name, mx, mean, ref):
    print(f"[w8a8] {name}: max_rel {mx:.3e} mean_rel {mean:.3e} "
          f"pairs {int(ref['expert_counts'].sum())} experts {int((ref['expert_counts'] > 0).sum())}", flush=True)


# many rows per expert at I = 512 with fp8 weights; hidden 512, 1024, 2048
# (4, 8, 16 k stages of the gate/up GEMM), 32..128-row work tiles
A8 = W.Workload("w8a8_res", 8, 32, 512, 16, 4, 512, 512, W.BF16, W.FP8, 0.9, seed=141)


@pytest.mark.parametrize("wl,layout", [
    (A8, "rows"),
    (A8.with_(name="w8a8_res_panels", seed=142), "panels"),
    (A8.with_(name="w8a8_H1024", hidden=1024, seed=143), "panels"),
    (A8.with_(name="w8a8_H2048", hidden=2048, seed=144), "rows"),
    (A8.with_(name="w8a8_noshared", shared_inter=0, seed=145), "panels"),
    (A8.with_(name="w8a8_mt1", num_blocks=4, num_experts=64, top_k=8, seed=146), "rows"),
    (A8.with_(name="w8a8_mt1_H1024", num_blocks=4, num_experts=64, top_k=8, hidden=1024, seed=152), "panels"),
    (A8.with_(name="w8a8_mt2", num_experts=32, seed=153), "panels"),
    (A8.with_(name="w8a8_mt2_H2048_rows", num_experts=32, hidden=2048, seed=154), "rows"),
    (A8.with_(name="w8a8_mt4", num_experts=8, seed=147), "panels"),
    (A8.with_(name="w8a8_mt4_rows", num_experts=8, seed=148), "rows"),
    (A8.with_(name="w8a8_mt4_H2048", num_experts=8, hidden=2048, seed=155), "panels"),
    (A8.with_(name="w8a8_hot", bias_sigma=3.0, seed=149), "rows"),
    (A8.with_(name="w8a8_live_budget", live_fraction=0.6, expert_budget=6, seed=150), "panels"),
    (A8.with_(name="w8a8_rows8", block_rows=8, num_blocks=32, seed=151), "rows"),
], ids=lambda v: v if isinstance(v, str) else v.name)
def test_w8a8_shapes(wl, layout):
    inp = W.generate(wl)
    mx, mean, ref = check(inp, threads=16, dp=cm.upload(inp, layout=layout), act_fp8=True)
    _report(wl.name, mx, mean, ref)
    if wl.name == "w8a8_hot":
        assert ref["expert_counts"].max() > 96   # an expert spans several tiles


@pytest.mark.parametrize("layout", ["panels", "rows"])
def test_w8a8_blocks64_full(layout):
    """The 64-block fp8 call at full size, every row."""
    inp = W.generate(W.WORKLOADS["blocks64_fp8"])
    mx, mean, ref = check(inp, threads=16, dp=cm.upload(inp, layout=layout), act_fp8=True)
    _report(f"blocks64_fp8 ({layout})", mx, mean, ref)


@pytest.mark.parametrize("nb", [2, 4])
def test_w8a8_few_blocks_full(nb):
    """Two and four 32-row blocks at full size: 32-row work tiles that mostly
    hold one or two rows."""
    inp = W.generate(W.WORKLOADS["blocks64_fp8"].with_(name=f"blocks64_fp8_x{nb}", num_blocks=nb, seed=180 + nb))
    mx, mean, ref = check(inp, threads=16, dp=cm.upload(inp, layout="panels"), act_fp8=True)
    _report(f"blocks64_fp8 x{nb}", mx, mean, ref)
