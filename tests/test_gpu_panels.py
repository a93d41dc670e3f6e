"""MFMA-panel weight storage (CMOE_LAYOUT_PANELS): the pack entry point
against the layout's definition in include/clover_moe.h, and calls on packed
weights against the same calls on row-major weights -- bit for bit, since a
lane receives the same weight bytes into the same registers in both layouts
and only their addresses differ -- and against the oracle."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_softmax_amd as cm
import workloads as W
from parity import bits, check, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(require_gpu):
    pass


def panels_by_definition(a: np.ndarray, gate_up: bool) -> np.ndarray:
    """[count, rows, row_bytes] uint8 -> panel bytes, written out unit by unit
    from the definition: byte 16l + b of unit q of panel p is byte
    64q + 16(l // 16) + b of panel row l % 16."""
    count, rows, rb = a.shape
    out = np.empty(count * rows * rb, np.uint8)
    o = 0
    for m in range(count):
        for p in range(rows // 16):
            for q in range(rb // 64):
                for l in range(64):
                    i = l % 16
                    if gate_up:
                        row = 8 * p + i if i < 8 else rows // 2 + 8 * p + i - 8
                    else:
                        row = 16 * p + i
                    c = 64 * q + 16 * (l // 16)
                    out[o:o + 16] = a[m, row, c:c + 16]
                    o += 16
    return out


@pytest.mark.parametrize("count,rows,row_bytes,gate_up", [
    (3, 32, 128, 1), (2, 48, 192, 0), (1, 64, 256, 1), (4, 16, 64, 0), (2, 256, 64, 1)])
def test_pack_matches_the_definition(count, rows, row_bytes, gate_up):
    rng = np.random.default_rng(count * 1000 + rows + row_bytes + gate_up)
    a = rng.integers(0, 256, size=(count, rows, row_bytes), dtype=np.uint8)
    src = torch.from_numpy(a).cuda()
    # dst inside a larger buffer, with 4 KiB canaries on both sides
    n = a.size
    buf = torch.full((n + 8192,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = buf[4096:4096 + n]
    cm.clover_moe_pack_weights(src, dst, count, rows, row_bytes, gate_up)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    np.testing.assert_array_equal(got[4096:4096 + n], panels_by_definition(a, bool(gate_up)))
    assert np.all(got[:4096] == 0xA5) and np.all(got[4096 + n:] == 0xA5), "write outside dst"
    np.testing.assert_array_equal(src.cpu().numpy(), a)  # the source is left alone


MID = W.Workload("mid_bf16", 4, 16, 256, 32, 8, 256, 128, W.BF16, W.BF16, 0.9, seed=21)
FEW = MID.with_(name="few_E256", num_experts=256, seed=61)
DEC = W.WORKLOADS["decode1_bf16"].with_(hidden=512, num_experts=64, inter=256, shared_inter=256)

CASES = [
    # register-operand GEMMs (one 16-row tile per expert)
    FEW.with_(name="p_few_bf16", seed=301),
    FEW.with_(name="p_few_fp8", weight_dtype=W.FP8, seed=302),
    FEW.with_(name="p_few_f32", act_dtype=W.F32, weight_dtype=W.F32, seed=303),
    FEW.with_(name="p_few_fp4", weight_dtype=W.FP4, seed=304),
    FEW.with_(name="p_few_fp4_H384_I512", weight_dtype=W.FP4, hidden=384, inter=512, seed=305),
    FEW.with_(name="p_few_fp4_H2048", weight_dtype=W.FP4, hidden=2048, inter=512, num_experts=64, seed=306),
    FEW.with_(name="p_few_Is_ne_I", inter=128, shared_inter=384, seed=307),
    # the fused down + combine kernel (one row)
    DEC.with_(name="p_dec_bf16", seed=311),
    DEC.with_(name="p_dec_fp8", weight_dtype=W.FP8, seed=312),
    DEC.with_(name="p_dec_fp4", weight_dtype=W.FP4, seed=313),
    # LDS-tiled GEMMs (many rows per expert)
    MID.with_(name="p_mid_bf16", seed=321),
    MID.with_(name="p_mid_fp8", weight_dtype=W.FP8, seed=322),
    MID.with_(name="p_mid_f32", act_dtype=W.F32, weight_dtype=W.F32, seed=323),
    MID.with_(name="p_mid_fp4", weight_dtype=W.FP4, seed=324),
    MID.with_(name="p_mid_Is_ne_I", inter=128, shared_inter=384, seed=325),
    MID.with_(name="p_mid_rows32_fp8", block_rows=32, num_blocks=3, weight_dtype=W.FP8, seed=326),
    # expert budget and live rows, a skewed router at a low threshold and k 4,
    # and a two-row verification call
    MID.with_(name="p_mid_budget6_live50", live_fraction=0.5, expert_budget=6, seed=331),
    FEW.with_(name="p_few_skewed_tau08_k4", bias_sigma=1.0, mass_threshold=0.8, top_k=4, seed=332),
    FEW.with_(name="p_few_rows2", block_rows=2, num_blocks=3, seed=333),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_panels_give_the_row_major_result_bit_for_bit(wl):
    print(f"[panels] {wl.name}", flush=True)
    inp = W.generate(wl)
    tau = wl.mass_threshold
    out_r, rt_r = run_gpu(inp, tau, wl.top_k)
    out_p, rt_p = run_gpu(inp, tau, wl.top_k, dp=cm.upload(inp, layout="panels"))
    for k in rt_r:
        np.testing.assert_array_equal(bits(rt_p[k]), bits(rt_r[k]), err_msg=k)
    np.testing.assert_array_equal(bits(out_p), bits(out_r))


@pytest.mark.parametrize("wl", [CASES[0], CASES[3], CASES[8], CASES[11], CASES[16]], ids=lambda w: w.name)
def test_panels_against_the_oracle(wl):
    inp = W.generate(wl)
    check(inp, dp=cm.upload(inp, layout="panels"))
