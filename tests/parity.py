"""Helpers shared by the GPU parity tests: run one call through the C ABI,
run the oracle on the same bytes, compare.

Bars (the operation's accuracy contract):
  routing (logits, block mass, coreset, top-k indices, gates, counts,
  offsets, permutation): bit-exact;
  FFN output, bf16 weights: max|d| <= 2e-2 max|ref| and sum|d| <= 5e-3 sum|ref|;
  FFN output, fp8 weights:  max|d| <= 6e-2 max|ref|;
  FFN output, fp32 (no bf16 rounding anywhere): max|d| <= 1e-4 max|ref|.  The
  only error sources are fp32 accumulation over at most max(H, I) terms and
  fp32 SiLU, both below 2^-24 * 2048 ~ 1.2e-4 relative in the worst case and
  ~1e-6 in practice.
  FFN output with fp8 activations (cmoe_options.activation_fp8), two checks:
  against the oracle's own fp8-activation reading (x and bf16 h rounded to
  MXFP8, everything else fp64) at the bf16 bar, max|d| <= 2e-2 max|ref| and
  sum|d| <= 5e-3 sum|ref| -- both sides take the same MXFP8 codes except where
  the kernel's fp32 h falls on the other side of a bf16 rounding boundary
  (a few codes in a million), so what remains are the bf16 roundings the
  bf16 path also has (each pair's down output y and the combined output;
  measured max 5-12e-3, mean 2.2-2.4e-3); and against the exact oracle at the
  fp8-weight bar, max|d| <= 6e-2 max|ref| (MXFP8 rounds each activation by up
  to 2^-4 relative; measured about 4.6e-2 sum|d|/sum|ref|).
"""
from __future__ import annotations

import numpy as np

import oracle
import sparse_moe_ffn_softmax_amd as cm
import workloads as W

ROUTING_KEYS = ("logits", "block_mass", "coreset_ids", "coreset_size", "topk_idx", "gates",
                "expert_counts", "expert_offsets", "perm")

TOL_ACT8 = dict(max_rel=2e-2, mean_rel=5e-3)

TOL = {
    W.BF16: dict(max_rel=2e-2, mean_rel=5e-3),
    W.FP8: dict(max_rel=6e-2, mean_rel=None),
    # 4-bit weights widen to bf16 exactly (code times a power of two): the bf16 bar
    W.FP4: dict(max_rel=2e-2, mean_rel=5e-3),
    W.F32: dict(max_rel=1e-4, mean_rel=5e-3),
}


# value `out` is filled with before a call: rows the call must not write
# (resolved rows) still hold it afterwards; exact in bf16 and fp32
SENTINEL = 768.0


def run_gpu(inp, tau: float, top_k: int, dp=None, workspace=None, outputs=None, act_fp8=False):
    """One call through the C ABI; returns (out as fp64 numpy, routing dict).
    Workloads with an expert budget or live rows, and calls with fp8
    activations, go through the _ex entry point with those options.
    `outputs`: the routing outputs requested (None = all)."""
    import torch
    wl = inp.wl
    dp = dp or cm.upload(inp)
    ws = workspace if workspace is not None else cm.alloc_workspace(dp.problem, top_k)
    rt_t, rt = cm.alloc_routing(dp.problem, top_k, names=outputs)
    odt = torch.bfloat16 if wl.act_dtype == W.BF16 else torch.float32
    out = torch.full((wl.rows, wl.hidden), SENTINEL, dtype=odt, device="cuda")
    opts = None
    if wl.expert_budget or dp.tensors.get("live_rows") is not None or act_fp8:
        opts = cm.make_options(wl.expert_budget, dp.tensors.get("live_rows"), int(act_fp8))
    cm.clover_moe_block_forward(dp.problem, dp.weights, dp.tensors["x"], tau, top_k, out, rt, ws,
                                options=opts)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in rt_t.items()}
    return out.double().cpu().numpy(), res


def bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float64:
        return a.view(np.uint64)
    return a


def assert_routing_equal(gpu: dict, ref: dict):
    for k in ROUTING_KEYS:
        if k not in gpu:
            continue
        g, r = bits(gpu[k]), bits(ref[k])
        assert g.shape == r.shape, (k, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"routing output {k} differs at {len(bad)} places, first {bad[:5].tolist()}")


def ffn_errors(out: np.ndarray, ref: np.ndarray, rows=None):
    if rows is not None:
        out, ref = out[rows], ref[rows]
    d = np.abs(out - ref)
    return float(d.max() / np.abs(ref).max()), float(d.sum() / np.abs(ref).sum())


def assert_ffn_close(out, ref, weight_dtype, rows=None, tol=None):
    assert np.all(np.isfinite(out if rows is None else out[rows]))
    mx, mean = ffn_errors(out, ref, rows)
    tol = tol or TOL[weight_dtype]
    assert mx <= tol["max_rel"], f"max|d|/max|ref| = {mx:.3e} > {tol['max_rel']}"
    if tol["mean_rel"] is not None:
        assert mean <= tol["mean_rel"], f"sum|d|/sum|ref| = {mean:.3e} > {tol['mean_rel']}"
    return mx, mean


def check(inp, tau=None, top_k=None, rows=None, threads=0, dp=None, outputs=None, act_fp8=False):
    """Full parity check of one call; returns (max_rel, mean_rel, oracle result).
    `outputs`: the routing outputs the call requests (None = all).  With
    act_fp8 the call runs with MXFP8 activations and its FFN output is held
    to the fp8-weight bar against the exact oracle."""
    wl = inp.wl
    tau = wl.mass_threshold if tau is None else tau
    top_k = wl.top_k if top_k is None else top_k
    print(f"[parity] {wl.name} B={wl.num_blocks} R={wl.block_rows} H={wl.hidden} E={wl.num_experts} "
          f"I={wl.inter} Is={wl.shared_inter} {wl.act_dtype}/{wl.weight_dtype} tau={tau} k={top_k}"
          f"{' act_fp8' if act_fp8 else ''}", flush=True)
    out, gpu = run_gpu(inp, tau, top_k, dp=dp, outputs=outputs, act_fp8=act_fp8)
    ref = oracle.forward(inp, tau=tau, top_k=top_k, rows=rows, threads=threads)
    assert_routing_equal(gpu, ref)
    if act_fp8:
        ref8 = oracle.forward(inp, tau=tau, top_k=top_k, rows=rows, threads=threads, act_fp8=True)
        sel = rows
        if inp.live_rows is not None:
            live = np.flatnonzero(inp.live_rows.astype(bool))
            sel = live if rows is None else np.intersect1d(np.asarray(rows), live)
        mx8, mean8 = assert_ffn_close(out, ref8["out"], wl.weight_dtype, sel, tol=TOL_ACT8)
        print(f"[parity] against the fp8-activation oracle: max_rel {mx8:.3e} mean_rel {mean8:.3e}", flush=True)
    if inp.live_rows is not None:
        # resolved rows keep the caller's cached output; compare the live ones
        live = inp.live_rows.astype(bool)
        assert np.all(out[~live] == SENTINEL), "a resolved row of out was written"
        sel = np.flatnonzero(live)
        rows = sel if rows is None else np.intersect1d(np.asarray(rows), sel)
        if rows.size == 0:
            return 0.0, 0.0, ref
    mx, mean = assert_ffn_close(out, ref["out"], wl.weight_dtype, rows)
    return mx, mean, ref
