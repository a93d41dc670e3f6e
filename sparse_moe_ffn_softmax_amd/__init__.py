"""Python binding of the block-restricted sparse-MoE FFN library for MI355X.

A thin ctypes layer over ``include/clover_moe.h``: the functions here have the
same names as the C entry points and only marshal arguments (shapes into the
C structs, device pointers out of torch tensors).  Every step of the
operation runs in the HIP kernels of ``libclover_moe.so``; there is no
fallback of any kind -- if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libclover_moe.so")

CMOE_OK, CMOE_ERR_NULL, CMOE_ERR_VALUE, CMOE_ERR_UNSUPPORTED = 0, 1, 2, 3
CMOE_ERR_ALIGN, CMOE_ERR_ALIAS, CMOE_ERR_WORKSPACE, CMOE_ERR_HIP = 4, 5, 6, 7
CMOE_F32, CMOE_BF16, CMOE_FP8_E4M3, CMOE_FP4_E2M1 = 0, 1, 2, 3
DTYPE_CODES = {"f32": CMOE_F32, "bf16": CMOE_BF16, "fp8_e4m3": CMOE_FP8_E4M3, "fp4_e2m1": CMOE_FP4_E2M1}
CMOE_LAYOUT_ROWS, CMOE_LAYOUT_PANELS = 0, 1
LAYOUT_CODES = {"rows": CMOE_LAYOUT_ROWS, "panels": CMOE_LAYOUT_PANELS}

EXPORTED = ("clover_moe_workspace_size", "clover_moe_block_forward", "clover_moe_block_forward_ex",
            "clover_moe_block_forward_staged", "clover_moe_block_forward_noalloc", "clover_moe_pack_weights",
            "clover_moe_status_string", "clover_moe_last_error", "clover_moe_plan_info")
NOALLOC_MAX_WORKSPACE = 128 * 1024 * 1024  # CLOVER_MOE_NOALLOC_MAX_WORKSPACE
NUM_STAGES = 5
STAGE_NAMES = ("router", "route_blocks", "expert_up", "expert_down", "combine")


class cmoe_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "num_experts", "inter", "shared_inter", "block_rows", "num_blocks",
                 "act_dtype", "weight_dtype")]


class cmoe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_b", "w13", "w13_scale", "w2", "w2_scale",
                 "shared_w13", "shared_w13_scale", "shared_w2", "shared_w2_scale")] + [
        ("layout", ctypes.c_int32)]


class cmoe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "gates", "coreset_ids", "coreset_size", "expert_counts",
                 "expert_offsets", "perm", "logits", "block_mass")]


class cmoe_options(ctypes.Structure):
    _fields_ = [("expert_budget", ctypes.c_int32), ("live_rows", ctypes.c_void_p),
                ("activation_fp8", ctypes.c_int32)]


class cmoe_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tile_rows", "gate_up", "down", "y_bytes", "kernels")]


CMOE_GEMM_REGISTER, CMOE_GEMM_LDS_TILED, CMOE_GEMM_PERSISTENT, CMOE_GEMM_DOWN_COMBINE = 0, 1, 2, 3
GEMM_KIND_NAMES = {CMOE_GEMM_REGISTER: "register", CMOE_GEMM_LDS_TILED: "lds_tiled",
                   CMOE_GEMM_PERSISTENT: "persistent", CMOE_GEMM_DOWN_COMBINE: "down_combine"}


class ClovermoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libclover_moe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(path)
    L.clover_moe_workspace_size.restype = ctypes.c_int
    L.clover_moe_workspace_size.argtypes = [ctypes.POINTER(cmoe_problem), ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_size_t)]
    L.clover_moe_block_forward.restype = ctypes.c_int
    L.clover_moe_block_forward.argtypes = [
        ctypes.POINTER(cmoe_problem), ctypes.POINTER(cmoe_weights), ctypes.c_void_p, ctypes.c_float,
        ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(cmoe_routing), ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p]
    ex_args = [ctypes.POINTER(cmoe_problem), ctypes.POINTER(cmoe_weights), ctypes.c_void_p, ctypes.c_float,
               ctypes.c_int32, ctypes.POINTER(cmoe_options), ctypes.c_void_p, ctypes.POINTER(cmoe_routing),
               ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.clover_moe_block_forward_ex.restype = ctypes.c_int
    L.clover_moe_block_forward_ex.argtypes = ex_args
    L.clover_moe_block_forward_staged.restype = ctypes.c_int
    L.clover_moe_block_forward_staged.argtypes = ex_args + [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
    L.clover_moe_block_forward_noalloc.restype = ctypes.c_int
    L.clover_moe_block_forward_noalloc.argtypes = [
        ctypes.POINTER(cmoe_problem), ctypes.POINTER(cmoe_weights), ctypes.c_void_p, ctypes.c_float,
        ctypes.c_int32, ctypes.POINTER(cmoe_options), ctypes.c_void_p, ctypes.POINTER(cmoe_routing),
        ctypes.c_void_p]
    L.clover_moe_pack_weights.restype = ctypes.c_int
    L.clover_moe_pack_weights.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.clover_moe_status_string.restype = ctypes.c_char_p
    L.clover_moe_status_string.argtypes = [ctypes.c_int]
    L.clover_moe_last_error.restype = ctypes.c_char_p
    L.clover_moe_last_error.argtypes = []
    L.clover_moe_plan_info.restype = ctypes.c_int
    L.clover_moe_plan_info.argtypes = [ctypes.POINTER(cmoe_problem), ctypes.c_int32, ctypes.POINTER(cmoe_options),
                                       ctypes.POINTER(cmoe_plan_info)]
    _lib = L
    return L


def clover_moe_status_string(status: int) -> str:
    return load_library().clover_moe_status_string(status).decode()


def clover_moe_last_error() -> str:
    return load_library().clover_moe_last_error().decode()


def _check(status: int):
    if status != CMOE_OK:
        raise ClovermoeError(status, clover_moe_last_error() or clover_moe_status_string(status))


def clover_moe_plan_info(problem: cmoe_problem, top_k: int, options=None) -> dict:
    """The grouped-GEMM kernels a call runs (host-only): tile_rows, gate_up and
    down (names from GEMM_KIND_NAMES), y_bytes and kernels per call."""
    info = cmoe_plan_info()
    _check(load_library().clover_moe_plan_info(ctypes.byref(problem), top_k,
                                               ctypes.byref(options) if options is not None else None,
                                               ctypes.byref(info)))
    return {"tile_rows": info.tile_rows, "gate_up": GEMM_KIND_NAMES[info.gate_up],
            "down": GEMM_KIND_NAMES[info.down], "y_bytes": info.y_bytes, "kernels": info.kernels}


def clover_moe_workspace_size(problem: cmoe_problem, top_k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().clover_moe_workspace_size(ctypes.byref(problem), top_k, ctypes.byref(n)))
    return n.value


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def clover_moe_block_forward(problem: cmoe_problem, weights: cmoe_weights, x, mass_threshold: float,
                             top_k: int, out, routing: Optional[cmoe_routing], workspace,
                             workspace_bytes: Optional[int] = None, stream=None,
                             options: Optional[cmoe_options] = None) -> None:
    """Queue one call on `stream` (a torch.cuda.Stream, a raw hipStream_t int,
    or None for torch's current stream).  x, out, workspace: torch tensors or
    raw device pointers.  With `options` the call goes through
    clover_moe_block_forward_ex."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rt = ctypes.byref(routing) if routing is not None else None
    if options is None:
        _check(load_library().clover_moe_block_forward(
            ctypes.byref(problem), ctypes.byref(weights), _ptr(x), ctypes.c_float(mass_threshold),
            top_k, _ptr(out), rt, _ptr(workspace), workspace_bytes, stream))
    else:
        _check(load_library().clover_moe_block_forward_ex(
            ctypes.byref(problem), ctypes.byref(weights), _ptr(x), ctypes.c_float(mass_threshold),
            top_k, ctypes.byref(options), _ptr(out), rt, _ptr(workspace), workspace_bytes, stream))


def clover_moe_block_forward_noalloc(problem: cmoe_problem, weights: cmoe_weights, x,
                                     mass_threshold: float, top_k: int, out,
                                     routing: Optional[cmoe_routing] = None, stream=None,
                                     options: Optional[cmoe_options] = None) -> None:
    """Queue one call without a workspace argument: the library's static
    per-GPU scratch array serves as the workspace (calls must not overlap on
    one GPU)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    rt = ctypes.byref(routing) if routing is not None else None
    opt = ctypes.byref(options) if options is not None else None
    _check(load_library().clover_moe_block_forward_noalloc(
        ctypes.byref(problem), ctypes.byref(weights), _ptr(x), ctypes.c_float(mass_threshold),
        top_k, opt, _ptr(out), rt, stream))


def clover_moe_pack_weights(src, dst, count: int, rows: int, row_bytes: int, gate_up: int,
                            stream=None) -> None:
    """Queue the row-major -> MFMA-panel rearrangement of `count` matrices of
    `rows` x `row_bytes` bytes (src, dst: torch tensors or raw device pointers)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(load_library().clover_moe_pack_weights(_ptr(src), _ptr(dst), count, rows, row_bytes, gate_up, stream))


def pack_matrix_stack(t, gate_up: bool, stream=None):
    """A new device tensor holding the MFMA panels of `t`, a [..., rows, cols]
    stack of row-major matrices in any storage dtype (the last dimension is
    the row's storage elements, e.g. two fp4 codes per byte)."""
    import torch
    rows = t.shape[-2]
    row_bytes = t.shape[-1] * t.element_size()
    dst = torch.empty_like(t)
    clover_moe_pack_weights(t, dst, t.numel() // (t.shape[-1] * rows), rows, row_bytes, int(gate_up), stream)
    return dst


def clover_moe_block_forward_staged(problem: cmoe_problem, weights: cmoe_weights, x,
                                    mass_threshold: float, top_k: int, out,
                                    routing: Optional[cmoe_routing], workspace, stage_events,
                                    workspace_bytes: Optional[int] = None, stream=None,
                                    options: Optional[cmoe_options] = None) -> None:
    """As clover_moe_block_forward, recording the NUM_STAGES + 1 raw hipEvent_t
    handles in `stage_events` (ints) around the stages."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    ev = (ctypes.c_void_p * len(stage_events))(*stage_events)
    rt = ctypes.byref(routing) if routing is not None else None
    opt = ctypes.byref(options) if options is not None else None
    _check(load_library().clover_moe_block_forward_staged(
        ctypes.byref(problem), ctypes.byref(weights), _ptr(x), ctypes.c_float(mass_threshold),
        top_k, opt, _ptr(out), rt, _ptr(workspace), workspace_bytes, stream, ev, len(stage_events)))


# ---------------------------------------------------------------------------
# conveniences (still marshalling only)
# ---------------------------------------------------------------------------

def make_problem(hidden, num_experts, inter, shared_inter, block_rows, num_blocks,
                 act_dtype="bf16", weight_dtype="bf16") -> cmoe_problem:
    return cmoe_problem(hidden, num_experts, inter, shared_inter, block_rows, num_blocks,
                        DTYPE_CODES[act_dtype], DTYPE_CODES[weight_dtype])


def make_weights(router_w, w13, w2, router_b=None, w13_scale=None, w2_scale=None,
                 shared_w13=None, shared_w13_scale=None, shared_w2=None,
                 shared_w2_scale=None, layout="rows") -> cmoe_weights:
    return cmoe_weights(_ptr(router_w), _ptr(router_b), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                        _ptr(w2_scale), _ptr(shared_w13), _ptr(shared_w13_scale), _ptr(shared_w2),
                        _ptr(shared_w2_scale), LAYOUT_CODES[layout])


def make_options(expert_budget: int = 0, live_rows=None, activation_fp8: int = 0) -> cmoe_options:
    """live_rows: a [N] uint8 device tensor (1 = live) or None; activation_fp8:
    1 = MXFP8 activations into the fp8-weight expert GEMMs (W8A8)."""
    return cmoe_options(int(expert_budget), _ptr(live_rows), int(activation_fp8))


def make_routing(**tensors) -> cmoe_routing:
    return cmoe_routing(*[_ptr(tensors.get(n)) for n, _ in cmoe_routing._fields_])


@dataclass
class DeviceProblem:
    """Device copies of one call's inputs plus the structs that describe them."""
    problem: cmoe_problem
    weights: cmoe_weights
    tensors: dict
    rows: int
    hidden: int


def upload(inp, device="cuda", layout="rows") -> DeviceProblem:
    """Copy a host ``workloads.MoEInputs`` (storage-format numpy arrays) to the
    device, keeping the raw bytes, and describe it with the C structs.  With
    layout="panels" the four expert matrices are packed on the device
    (clover_moe_pack_weights) and only the panels are kept."""
    import numpy as np
    import torch

    wl = inp.wl

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        elif a.dtype == np.uint8:
            t = torch.from_numpy(a).view(torch.float8_e4m3fn)
        else:
            t = torch.from_numpy(a)
        return t.to(device)

    names = ("x", "router_w", "router_b", "w13", "w13_scale", "w2", "w2_scale", "shared_w13",
             "shared_w13_scale", "shared_w2", "shared_w2_scale")
    ts = {n: dev(getattr(inp, n)) for n in names}
    if layout == "panels":
        for n, gate_up in (("w13", True), ("w2", False), ("shared_w13", True), ("shared_w2", False)):
            if ts[n] is not None:
                ts[n] = pack_matrix_stack(ts[n], gate_up)
    elif layout != "rows":
        raise ValueError(f"layout={layout!r}")
    live = getattr(inp, "live_rows", None)
    ts["live_rows"] = None if live is None else torch.from_numpy(np.ascontiguousarray(live, np.uint8)).to(device)
    prob = make_problem(wl.hidden, wl.num_experts, wl.inter, wl.shared_inter, wl.block_rows,
                        wl.num_blocks, wl.act_dtype, wl.weight_dtype)
    w = make_weights(ts["router_w"], ts["w13"], ts["w2"], ts["router_b"], ts["w13_scale"],
                     ts["w2_scale"], ts["shared_w13"], ts["shared_w13_scale"], ts["shared_w2"],
                     ts["shared_w2_scale"], layout)
    return DeviceProblem(prob, w, ts, wl.rows, wl.hidden)


def alloc_workspace(problem: cmoe_problem, top_k: int, device="cuda"):
    import torch
    n = clover_moe_workspace_size(problem, top_k)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def alloc_routing(problem: cmoe_problem, top_k: int, device="cuda", names=None):
    """Device tensors for the optional routing outputs (all, or those named),
    plus the struct."""
    import torch
    N = problem.block_rows * problem.num_blocks
    E, B = problem.num_experts, problem.num_blocks
    i32, f32 = torch.int32, torch.float32
    t = {
        "topk_idx": torch.empty((N, top_k), dtype=i32, device=device),
        "gates": torch.empty((N, top_k), dtype=f32, device=device),
        "coreset_ids": torch.empty((B, E), dtype=i32, device=device),
        "coreset_size": torch.empty((B,), dtype=i32, device=device),
        "expert_counts": torch.empty((E,), dtype=i32, device=device),
        "expert_offsets": torch.empty((E + 1,), dtype=i32, device=device),
        "perm": torch.empty((N * top_k,), dtype=i32, device=device),
        "logits": torch.empty((N, E), dtype=f32, device=device),
        "block_mass": torch.empty((B, E), dtype=torch.float64, device=device),
    }
    if names is not None:
        t = {k: v for k, v in t.items() if k in names}
    return t, make_routing(**t)
