"""Benchmark of the block-restricted sparse-MoE FFN on one MI355X.

One step = one call of the whole hot path (router, per-block routing,
permutation, gate/up GEMM + SwiGLU, down GEMM, combine with the shared
expert) over one batch of synthetic blocks, with every input already resident
in HBM.  The default workload is one 32-row bf16 block at the model's routing
shape (H 2048, 256 experts, top-8, I 512, shared expert I 512, mass threshold
0.9) -- the weight-streaming bound case.

The expert weights are stored as MFMA panels (clover_moe_pack_weights, run
once at load, before any timing), the library's fast layout; `--layout rows`
times the row-major layout instead.

Successive steps cycle through `--layers` copies of the weights placed at
different addresses (the experts of copy j are rotated by j*E/L, router
included, so every copy routes to the same number of experts): like the
consecutive MoE layers of a denoising pass, no step finds its weights in the
256 MB MALL left by the previous one.

Prints ONE JSON line (see the keys below).  `value` is the wall-clock rate of
plain clover_moe_block_forward calls over the timed steps (synchronised on
both sides).  Per-stage device times, and the dominant kernel's duration in
`roofline`, come from a second pass over the same steps through
clover_moe_block_forward_staged, which records HIP events on the call's stream
between its kernels.  The events are created without the system-scope fence
(timing only); each still costs about a microsecond of device time, so the
stage times are slight overestimates and the roofline fraction a slight
underestimate (one block: gate/up 96.8 us by events, 95.9 us in the kernel
trace).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)
# dense MFMA datasheet peaks (TFLOP/s) by the operand type the matrix cores run
MFMA_DATASHEET_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
# the MFMA operand type of each weight format: fp8 (W8A16) and 4-bit weights
# are widened to bf16 in registers and run on the bf16 MFMA
MFMA_KIND = {"bf16": "bf16", "fp8_e4m3": "bf16", "fp4_e2m1": "bf16", "f32": "f32"}


def hip():
    L = ctypes.CDLL("libamdhip64.so")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return L


def layer_copies(dp, n_layers, E, layout):
    """Weight copies at new addresses with experts rotated by j*E/n_layers
    (an expert's panels are its own contiguous bytes, so rotating packed
    weights by experts is packing the rotated ones)."""
    import torch
    import sparse_moe_ffn_softmax_amd as cm
    layers = [dp.weights]
    keep = []
    t = dp.tensors
    for j in range(1, n_layers):
        sh = (j * E) // n_layers

        def rot(a):
            if a is None:
                return None
            if a.dtype == torch.float8_e4m3fn:  # roll the raw bytes
                return torch.roll(a.view(torch.uint8), shifts=sh, dims=0).contiguous().view(a.dtype)
            return torch.roll(a, shifts=sh, dims=0).contiguous()

        def cp(a):
            return None if a is None else a.clone()

        c = dict(router_w=rot(t["router_w"]), router_b=rot(t["router_b"]), w13=rot(t["w13"]),
                 w13_scale=rot(t["w13_scale"]), w2=rot(t["w2"]), w2_scale=rot(t["w2_scale"]),
                 shared_w13=cp(t["shared_w13"]), shared_w13_scale=cp(t["shared_w13_scale"]),
                 shared_w2=cp(t["shared_w2"]), shared_w2_scale=cp(t["shared_w2_scale"]))
        keep.append(c)
        layers.append(cm.make_weights(**c, layout=layout))
    return layers, keep


def source_digest(name: str) -> str:
    """SHA-256 (16 hex digits) of a kernel source with its // comments and
    blank lines removed: the counters stay valid across comment edits, not
    across code changes."""
    p = os.path.join(ROOT, "sparse_moe_ffn_softmax_amd", "csrc", name)
    code = []
    for line in open(p).read().splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line.strip():
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, src: str, layout: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source and weight layout; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("code_sha256_16") != source_digest(src) or d.get("weight_layout", "rows") != layout:
        return None
    return d.get("hbm_bytes_per_launch")


def measure_peaks(H_, stream_ptr):
    """Achievable HBM read bandwidth and bf16 / fp8 MFMA rates of this GPU,
    from the probes of libclover_moe_peaks.so (a streaming read of 4 GiB with
    the panel loads' pattern; waves issuing independent MFMAs back to back)."""
    import torch
    from sparse_moe_ffn_softmax_amd import _build
    P = ctypes.CDLL(_build.PEAKS_LIB)
    P.cmoe_peak_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    P.cmoe_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    P.cmoe_peak_mfma_flop.restype = ctypes.c_longlong
    ev = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert H_.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
        ev.append(e.value)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            assert H_.hipEventRecord(ev[0], stream_ptr) == 0
            fn()
            assert H_.hipEventRecord(ev[1], stream_ptr) == 0
            torch.cuda.synchronize()
            f = ctypes.c_float()
            assert H_.hipEventElapsedTime(ctypes.byref(f), ev[0], ev[1]) == 0
            best = f.value if best is None else min(best, f.value)
        return best * 1e-3

    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    reads = {}
    for pattern, blocks_rd in ((0, 2048), (1, 2048), (1, 4096)):
        sink = torch.empty(blocks_rd, dtype=torch.int32, device="cuda")
        t_rd = timed(lambda: P.cmoe_peak_read(pattern, buf.data_ptr(), nbytes, sink.data_ptr(), blocks_rd,
                                              stream_ptr), 5)
        reads[f"pattern{pattern}_wg{blocks_rd}"] = round(nbytes / t_rd / 1e9, 1)
    del buf
    blocks, iters = 1024, 2000
    out = torch.empty(blocks * 256 * 4, dtype=torch.float32, device="cuda")
    res = {"hbm_read_gbps": max(reads.values()), "hbm_read_by_pattern": reads}
    for kind, name in ((0, "mfma_bf16_16x16x32_tflops"), (2, "mfma_bf16_32x32x16_tflops"),
                       (1, "mfma_fp8_16x16x128_tflops"), (3, "mfma_fp8_32x32x64_tflops")):
        t = timed(lambda: P.cmoe_peak_mfma(kind, out.data_ptr(), blocks, iters, stream_ptr), 3)
        flop = P.cmoe_peak_mfma_flop(kind) * iters * blocks * 4
        res[name] = round(flop / t / 1e12, 1)
    res["mfma_bf16_tflops"] = max(res["mfma_bf16_16x16x32_tflops"], res["mfma_bf16_32x32x16_tflops"])
    res["mfma_fp8_tflops"] = max(res["mfma_fp8_16x16x128_tflops"], res["mfma_fp8_32x32x64_tflops"])
    for e in ev:
        H_.hipEventDestroy(e)
    res["probe"] = ("streaming read of 4 GiB (each wave load 1 KiB of consecutive lines, non-temporal; "
                    "grid-strided or one slab per workgroup; the best); 1024 workgroups x 4 waves x 2000 "
                    "rounds of MFMAs on independent chains (16x16 and 32x32 bf16 and fp8 e4m3 with unit "
                    "scales); best of repeated runs")
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentiles(a):
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2)}


def cpu_baseline(inp, B, N, budget_s):
    """The oracle timed on this host: all cores (OpenMP over rows), then one
    thread on a bounded sample.  Full calls when they fit the budget;
    otherwise the FFN of the first blocks' rows only (routing still covers
    every row), scaled to block-passes/s by the blocks computed."""
    import oracle
    wl = inp.wl
    R = wl.block_rows
    nproc = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS") or min(16, nproc))

    def leg(nthreads, budget):
        t1 = time.perf_counter()
        oracle.forward(inp, threads=nthreads, rows=np.arange(min(N, R)))
        one_block = time.perf_counter() - t1
        # blocks whose rows fit the budget (one-block time includes all routing)
        nb = int(max(1, min(B, budget / max(one_block, 1e-4))))
        rows = None if nb >= B else np.arange(nb * R)
        reps = 1
        if nb >= B:
            t1 = time.perf_counter()
            oracle.forward(inp, threads=nthreads)
            one = time.perf_counter() - t1
            reps = max(1, min(500, int(budget / max(one, 1e-3))))
        t1 = time.perf_counter()
        for _ in range(reps):
            oracle.forward(inp, threads=nthreads, rows=rows)
        el = time.perf_counter() - t1
        blocks = nb if rows is not None else B
        what = (f"{reps} full call(s) (routing and fp64 FFN for all {N} rows)" if rows is None else
                f"one call with routing for all {N} rows and the fp64 FFN for the first {nb} of {B} "
                f"blocks ({nb * R} rows)")
        return reps * blocks / el, el, what

    import numpy as np
    v_all, el_all, what_all = leg(threads, budget_s * 0.6)
    v_one, el_one, what_one = leg(1, budget_s * 0.4)
    return {
        "value": round(v_all, 4), "unit": "block-passes/s", "cores": threads, "kind": "oracle",
        "sample": f"{wl.name}: {what_all}, {el_all:.1f} s wall, {threads} OpenMP threads over rows",
        "single_thread": {"value": round(v_one, 4), "unit": "block-passes/s", "cores": 1,
                          "sample": f"{what_one}, {el_one:.1f} s wall"},
        "host": {"nproc": nproc, "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model()},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="block32_bf16")
    ap.add_argument("--tau", type=float, default=None, help="mass threshold (default: the workload's)")
    ap.add_argument("--top-k", type=int, default=None, help="top-k (default: the workload's)")
    ap.add_argument("--layout", default="panels", choices=["panels", "rows"],
                    help="expert weight storage: MFMA panels (packed once at load) or row-major")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="rough budget of the oracle CPU-baseline leg (0 disables it)")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip measuring the achievable HBM read and MFMA rates of the GPU")
    ap.add_argument("--act-fp8", action="store_true",
                    help="fp8 weights only: MXFP8 activations into the expert GEMMs (W8A8, "
                         "cmoe_options.activation_fp8)")
    ap.add_argument("--blocks", type=int, default=None,
                    help="blocks per call (default: the workload's); the workload is then named "
                         "<workload>@<blocks>")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="copy a device buffer of this many bytes once before the workload: "
                         "a plain copy kernel of known size for calibrating HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_moe_ffn_softmax_amd as cm
    import workloads as W

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = W.WORKLOADS[args.workload]
    if args.blocks is not None and args.blocks != wl.num_blocks:
        wl = wl.with_(name=f"{wl.name}@{args.blocks}", num_blocks=args.blocks)
    K = wl.top_k if args.top_k is None else args.top_k
    tau = wl.mass_threshold if args.tau is None else args.tau
    N, H, E, I, Is, B = wl.rows, wl.hidden, wl.num_experts, wl.inter, wl.shared_inter, wl.num_blocks
    t0 = time.time()
    inp = W.generate(wl)
    print(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dp = cm.upload(inp, layout=args.layout)
    layers, _keep = layer_copies(dp, args.layers, E, args.layout)
    ws = cm.alloc_workspace(dp.problem, K)
    odt = torch.bfloat16 if wl.act_dtype == W.BF16 else torch.float32
    out = torch.empty((N, H), dtype=odt, device="cuda")
    total = args.warmup + args.steps
    counts = torch.zeros((total, E), dtype=torch.int32, device="cuda")
    routings = [cm.make_routing(expert_counts=counts[i]) for i in range(total)]

    H_ = hip()
    n_ev = cm.NUM_STAGES + 1
    events = []
    for _ in range(args.steps):
        row = []
        for _ in range(n_ev):
            e = ctypes.c_void_p()
            # timing-only events: no system-scope fence (cache writeback and
            # invalidation) when they complete, which would otherwise add to
            # the kernels between them
            assert H_.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
            row.append(e.value)
        events.append(row)

    stream = torch.cuda.current_stream()
    x = dp.tensors["x"]
    # expert budget / live rows: the _ex entry point with the workload's options
    opts = None
    if wl.expert_budget or dp.tensors.get("live_rows") is not None or args.act_fp8:
        opts = cm.make_options(wl.expert_budget, dp.tensors.get("live_rows"), int(args.act_fp8))
    for i in range(args.warmup):
        cm.clover_moe_block_forward(dp.problem, layers[i % len(layers)], x, tau, K, out,
                                    routings[i], ws, stream=stream, options=opts)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # timed region: plain calls, as a caller makes them
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        i = args.warmup + s
        cm.clover_moe_block_forward(dp.problem, layers[i % len(layers)], x, tau, K, out,
                                    routings[i], ws, stream=stream, options=opts)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    print(f"[bench] timed {args.steps} steps", file=sys.stderr, flush=True)

    # per-call pass: the same steps again, one event between consecutive calls
    call_ev = []
    for _ in range(args.steps + 1):
        e = ctypes.c_void_p()
        assert H_.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
        call_ev.append(e.value)
    sp = stream.cuda_stream
    torch.cuda.synchronize()
    for s in range(args.steps):
        i = args.warmup + s
        assert H_.hipEventRecord(call_ev[s], sp) == 0
        cm.clover_moe_block_forward(dp.problem, layers[i % len(layers)], x, tau, K, out,
                                    routings[i], ws, stream=stream, options=opts)
    assert H_.hipEventRecord(call_ev[args.steps], sp) == 0
    torch.cuda.synchronize()
    call_us = []
    f = ctypes.c_float()
    for s in range(args.steps):
        assert H_.hipEventElapsedTime(ctypes.byref(f), call_ev[s], call_ev[s + 1]) == 0
        call_us.append(f.value * 1e3)
    for e in call_ev:
        H_.hipEventDestroy(e)

    # single-call latency: one call on an idle GPU, from the host's issue to
    # its completion seen by the host (argument marshalling, launch, kernels)
    lat_us = []
    for s in range(min(args.steps, 20)):
        i = args.warmup + s
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        cm.clover_moe_block_forward(dp.problem, layers[i % len(layers)], x, tau, K, out,
                                    routings[i], ws, stream=stream, options=opts)
        torch.cuda.synchronize()
        lat_us.append((time.perf_counter() - t0) * 1e6)
    print(f"[bench] per-call and latency passes done", file=sys.stderr, flush=True)

    # stage pass: the same steps again, with HIP events between the kernels
    torch.cuda.synchronize()
    for s in range(args.steps):
        i = args.warmup + s
        cm.clover_moe_block_forward_staged(dp.problem, layers[i % len(layers)], x, tau, K, out,
                                           routings[i], ws, events[s], stream=stream, options=opts)
    torch.cuda.synchronize()
    print(f"[bench] stage pass done", file=sys.stderr, flush=True)

    peaks = measure_peaks(H_, sp) if args.peaks else None
    if peaks:
        print(f"[bench] peaks measured: {peaks['hbm_read_gbps']} GB/s read", file=sys.stderr, flush=True)

    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    stage_ms = np.zeros((args.steps, cm.NUM_STAGES))
    f = ctypes.c_float()
    for s in range(args.steps):
        for k in range(cm.NUM_STAGES):
            assert H_.hipEventElapsedTime(ctypes.byref(f), events[s][k], events[s][k + 1]) == 0
            stage_ms[s, k] = f.value
    for row in events:
        for e in row:
            H_.hipEventDestroy(e)

    cnt = counts[args.warmup:].cpu().numpy().astype(np.int64)  # [steps, E]
    touched = (cnt > 0).sum(1)
    pairs = cnt.sum(1)
    wsz = {W.F32: 4, W.BF16: 2, W.FP8: 1, W.FP4: 0.5}[wl.weight_dtype]
    asz = {W.F32: 4, W.BF16: 2}[wl.act_dtype]
    hsz = 4 if wl.act_dtype == W.F32 else 2
    fp8 = wl.weight_dtype == W.FP8
    fp4 = wl.weight_dtype == W.FP4

    def scale_bytes(rows, cols):
        if fp8:
            return (rows // 128) * (cols // 128) * 4
        if fp4:
            return rows * (cols // 32)
        return 0
    sc_up, sc_dn = scale_bytes(2 * I, H), scale_bytes(H, I)
    sc_up_s = scale_bytes(2 * Is, H) if Is else 0
    sc_dn_s = scale_bytes(H, Is) if Is else 0
    n_sh = N if Is else 0
    # algorithmic bytes per launch of the gate/up kernel: weights of the touched
    # experts (+ shared), x once, h written once
    up_bytes = (touched * (2 * I * H * wsz + sc_up) + (2 * Is * H * wsz + sc_up_s) + N * H * asz
                + (pairs * I + n_sh * Is) * hsz)
    # the library's kernel choice for this call, and the width of its per-pair
    # down outputs y (fp32, or bf16 on the taller-tile paths)
    plan = cm.clover_moe_plan_info(dp.problem, K, opts)
    ysz = plan["y_bytes"]
    dn_bytes = (touched * (H * I * wsz + sc_dn) + (H * Is * wsz + sc_dn_s) + (pairs * I + n_sh * Is) * hsz
                + (pairs + n_sh) * H * ysz)
    # whole call (weights, router, x in, out)
    call_bytes = (touched * (3 * H * I * wsz + sc_up + sc_dn) + (3 * H * Is * wsz + sc_up_s + sc_dn_s)
                  + 4 * E * H + N * H * 2 * asz)
    mfma_flops = 6.0 * H * I * pairs + 6.0 * H * Is * N
    up_flops = 4.0 * H * I * pairs + 4.0 * H * Is * n_sh
    dn_flops = 2.0 * H * I * pairs + 2.0 * H * Is * n_sh
    router_flops = 2.0 * N * H * E

    mean_stage = stage_ms.mean(0)
    dom = int(np.argmax(mean_stage))
    dom_name = cm.STAGE_NAMES[dom]
    dom_bytes = {2: up_bytes, 3: dn_bytes}.get(dom)
    device_ms = stage_ms.sum(1)
    if dom_bytes is not None:
        achieved = float(dom_bytes.sum() / (stage_ms[:, dom].sum() * 1e-3) / 1e9)
        # the kernel of the dominant stage, by the library's own choice
        if dom == 2:
            kname, src = {"register": ("expert_up_kernel", "expert_gemm.hip"),
                          "lds_tiled": ("expert_up_tiled_kernel", "expert_tiled.hip"),
                          "persistent": ("expert_up_mx_kernel", "expert_many.hip")}[plan["gate_up"]]
        else:
            kname, src = {"register": ("expert_down_kernel", "expert_gemm.hip"),
                          "lds_tiled": ("expert_down_tiled_kernel", "expert_tiled.hip"),
                          "persistent": ("expert_down_many_kernel", "expert_many.hip"),
                          "down_combine": ("expert_down_combine_kernel", "expert_gemm.hip")}[plan["down"]]
        wl_key = wl.name + ("_w8a8" if args.act_fp8 else "")
        traffic = measured_traffic(kname, wl_key, src, args.layout)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic, "kernel": kname,
                    "algorithmic_bytes_per_launch": int(dom_bytes.mean()),
                    "avg_launch_us": round(float(stage_ms[:, dom].mean() * 1e3), 2)}
        # past the ridge (MFMA peak / HBM peak flop per byte) the kernel's
        # roof is the matrix cores: report it against the MFMA peak instead
        dom_flops = up_flops if dom == 2 else dn_flops
        mfma_peak = MFMA_DATASHEET_TFLOPS["fp8" if args.act_fp8 else MFMA_KIND[wl.weight_dtype]]
        if peaks:
            roofline["frac_of_measured_peak"] = round(achieved / peaks["hbm_read_gbps"], 4)
            roofline["measured_peak"] = peaks["hbm_read_gbps"]
        if dom_flops.mean() / dom_bytes.mean() > mfma_peak * 1e12 / (HBM_PEAK_GBPS * 1e9):
            tflops = float(dom_flops.sum() / (stage_ms[:, dom].sum() * 1e-3) / 1e12)
            roofline.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak,
                             "unit": "TFLOP/s", "frac": round(tflops / mfma_peak, 4),
                             "algorithmic_flops_per_launch": float(dom_flops.mean()),
                             "hbm_gbps": round(achieved, 1)})
    else:
        roofline = {"bound": "alu", "achieved": None, "peak": None, "unit": None, "frac": None,
                    "traffic": None, "kernel": dom_name}

    value = B / (ms_per_step * 1e-3)
    rate = mfma_flops.mean() / (ms_per_step * 1e-3) / 1e12
    mk = "fp8" if args.act_fp8 else MFMA_KIND[wl.weight_dtype]
    mfma_util = {f"vs_{mk}_datasheet": round(float(rate / MFMA_DATASHEET_TFLOPS[mk]), 5)}
    if wl.weight_dtype == W.FP8:
        mfma_util["vs_fp8_datasheet"] = round(float(rate / MFMA_DATASHEET_TFLOPS["fp8"]), 5)
        mfma_util["vs_bf16_datasheet"] = round(float(rate / MFMA_DATASHEET_TFLOPS["bf16"]), 5)
    if peaks and mk in ("bf16", "fp8"):
        mfma_util[f"vs_{mk}_measured"] = round(float(rate / peaks[f"mfma_{mk}_tflops"]), 5)
        if wl.weight_dtype == W.FP8:
            mfma_util["vs_fp8_measured"] = round(float(rate / peaks["mfma_fp8_tflops"]), 5)
            mfma_util["vs_bf16_measured"] = round(float(rate / peaks["mfma_bf16_tflops"]), 5)
    call_gbps = float(call_bytes.mean() / (ms_per_step * 1e-3) / 1e9)
    res = {
        "metric": "MoE block-passes/s + achieved HBM GB/s & MFMA util vs peak, 32-row block",
        "value": round(value, 2),
        "unit": "block-passes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8_e4m3 weights, MXFP8 activations into the expert GEMMs (W8A8)" if args.act_fp8 else
                  {W.BF16: "bf16", W.F32: "f32", W.FP8: "fp8_e4m3 weights, bf16 activations",
                   W.FP4: "fp4_e2m1 (MXFP4) weights, bf16 activations"}[wl.weight_dtype]),
        "data": "synthetic (seeded normal inputs and random-init weights of the stated shapes)",
        "config": {"workload": wl.name, "num_blocks": B, "block_rows": wl.block_rows, "hidden": H,
                   "experts": E, "top_k": K, "inter": I, "shared_inter": Is,
                   "mass_threshold": tau, "weight_copies_rotated": args.layers,
                   "weight_layout": args.layout, "activation_fp8": bool(args.act_fp8)},
        "roofline": roofline,
        "call": {
            "kernels": plan,
            "device_us_staged": round(float(device_ms.mean() * 1e3), 2),
            "algorithmic_bytes": int(call_bytes.mean()),
            "hbm_gbps": round(call_gbps, 1),
            "hbm_frac": round(call_gbps / HBM_PEAK_GBPS, 4),
            "hbm_frac_of_measured_peak": round(call_gbps / peaks["hbm_read_gbps"], 4) if peaks else None,
            "mfma_tflops": round(float(rate), 3),
            "mfma_datapath": mk,
            "mfma_util": mfma_util,
            "device_us_per_call": percentiles(call_us),
            "single_call_latency_us": percentiles(lat_us),
            "router_gflop": round(router_flops / 1e9, 3),
            "experts_touched": float(touched.mean()),
            "routed_pairs": float(pairs.mean()),
        },
        "stages_us": {n: round(float(v * 1e3), 2) for n, v in zip(cm.STAGE_NAMES, mean_stage)},
        "peaks_measured": peaks,
        "cpu_baseline": None,
    }

    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(inp, B, N, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
