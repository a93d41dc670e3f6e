"""ctypes wrapper of the CPU oracle (oracle/clover_moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library; inputs come from :mod:`workloads`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "clover_moe_oracle.c")
_LIB = os.path.join(_HERE, "libclover_moe_oracle.so")

ORC_F32, ORC_BF16, ORC_FP8, ORC_FP4 = 0, 1, 2, 3
_DT = {"f32": ORC_F32, "bf16": ORC_BF16, "fp8_e4m3": ORC_FP8, "fp4_e2m1": ORC_FP4}


def build() -> str:
    """Compile the oracle with gcc (plain C11, OpenMP, no fp contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("hidden", "num_experts", "inter", "shared_inter", "block_rows", "num_blocks",
                 "act_dtype", "weight_dtype")]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_b", "w13", "w13_scale", "w2", "w2_scale",
                 "shared_w13", "shared_w13_scale", "shared_w2", "shared_w2_scale")]


class _Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "gates", "coreset_ids", "coreset_size", "expert_counts",
                 "expert_offsets", "perm", "logits", "block_mass")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.orc_exp.restype = ctypes.c_double
        L.orc_exp.argtypes = [ctypes.c_double]
        L.orc_exp_constants.argtypes = [ctypes.c_void_p]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_to_double.restype = ctypes.c_double
        L.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_double.restype = ctypes.c_double
        L.orc_e2m1_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_double.restype = ctypes.c_double
        L.orc_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.orc_router_logits.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int]
        L.orc_softmax.argtypes = [ctypes.c_void_p] * 4
        L.orc_block_mass.argtypes = [ctypes.c_void_p] * 4
        L.orc_coreset.restype = ctypes.c_int
        L.orc_coreset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
        L.orc_row_topk.restype = ctypes.c_int
        L.orc_row_topk.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_expert_ffn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6
        L.orc_forward.restype = ctypes.c_int
        L.orc_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_int]
        L.orc_forward_ex.restype = ctypes.c_int
        L.orc_forward_ex.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.orc_forward_ex_act8.restype = ctypes.c_int
        L.orc_forward_ex_act8.argtypes = L.orc_forward_ex.argtypes
        L.orc_round_bf16.restype = ctypes.c_double
        L.orc_round_bf16.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_mx8_scale_exp.restype = ctypes.c_int
        L.orc_mx8_scale_exp.argtypes = [ctypes.c_double]
        L.orc_mx8_round.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.orc_expert_ffn_mx8.argtypes = L.orc_expert_ffn.argtypes
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _problem(inp) -> _Problem:
    wl = inp.wl
    return _Problem(wl.hidden, wl.num_experts, wl.inter, wl.shared_inter, wl.block_rows,
                    wl.num_blocks, _DT[wl.act_dtype], _DT[wl.weight_dtype])


def _weights(inp) -> _Weights:
    return _Weights(_ptr(inp.router_w), _ptr(inp.router_b), _ptr(inp.w13), _ptr(inp.w13_scale),
                    _ptr(inp.w2), _ptr(inp.w2_scale), _ptr(inp.shared_w13),
                    _ptr(inp.shared_w13_scale), _ptr(inp.shared_w2), _ptr(inp.shared_w2_scale))


# --------------------------------------------------------------------------
# scalar pieces
# --------------------------------------------------------------------------

def exp(d: float) -> float:
    return lib().orc_exp(float(d))


def exp_many(d: np.ndarray) -> np.ndarray:
    f = lib().orc_exp
    return np.array([f(float(v)) for v in np.asarray(d, dtype=np.float64).ravel()]).reshape(np.shape(d))


def exp_constants() -> np.ndarray:
    out = np.zeros(17, dtype=np.float64)
    lib().orc_exp_constants(_ptr(out))
    return out


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(int(bits))


def e4m3_to_double(code: int) -> float:
    return lib().orc_e4m3_to_double(int(code))


def e2m1_to_double(code: int) -> float:
    return lib().orc_e2m1_to_double(int(code))


def e8m0_to_double(s: int) -> float:
    return lib().orc_e8m0_to_double(int(s))


# fp8 activations (the library's opt-in W8A8 mode, see clover_moe_oracle.h)

def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def mx8_scale_exp(amax: float) -> int:
    return int(lib().orc_mx8_scale_exp(float(amax)))


def mx8_round(v: np.ndarray) -> np.ndarray:
    """Rows of 32-element groups rounded to MXFP8 and back (fp64)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.size % 32 == 0
    out = np.empty_like(v)
    lib().orc_mx8_round(_ptr(v), v.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------

def router_logits(inp, threads: int = 0) -> np.ndarray:
    wl = inp.wl
    out = np.zeros((wl.rows, wl.num_experts), dtype=np.float32)
    p = _problem(inp)
    lib().orc_router_logits(ctypes.byref(p), _ptr(inp.x), _ptr(inp.router_w), _ptr(inp.router_b),
                            _ptr(out), threads)
    return out


def softmax(inp, logits: np.ndarray):
    """Returns (u, p): softmax numerators exp(l - max) and probabilities, fp64."""
    wl = inp.wl
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    u = np.zeros((wl.rows, wl.num_experts), dtype=np.float64)
    pr = np.zeros_like(u)
    p = _problem(inp)
    lib().orc_softmax(ctypes.byref(p), _ptr(logits), _ptr(u), _ptr(pr))
    return u, pr


def block_mass(inp, prob: np.ndarray, live: Optional[np.ndarray] = None) -> np.ndarray:
    wl = inp.wl
    prob = np.ascontiguousarray(prob, dtype=np.float64)
    if live is not None:
        live = np.ascontiguousarray(live, dtype=np.uint8)
    mass = np.zeros((wl.num_blocks, wl.num_experts), dtype=np.float64)
    p = _problem(inp)
    lib().orc_block_mass(ctypes.byref(p), _ptr(prob), _ptr(live), _ptr(mass))
    return mass


def coreset(mass_row: np.ndarray, tau: float):
    """(ids sorted by mass desc / id asc, coreset size)."""
    mass_row = np.ascontiguousarray(mass_row, dtype=np.float64)
    ids = np.zeros(mass_row.shape[0], dtype=np.int32)
    m = lib().orc_coreset(_ptr(mass_row), mass_row.shape[0], ctypes.c_float(tau), _ptr(ids))
    return ids, m


def row_topk(logits_row, u_row, in_set, top_k: int):
    logits_row = np.ascontiguousarray(logits_row, dtype=np.float32)
    u_row = np.ascontiguousarray(u_row, dtype=np.float64)
    in_set = np.ascontiguousarray(in_set, dtype=np.uint8)
    idx = np.zeros(top_k, dtype=np.int32)
    g = np.zeros(top_k, dtype=np.float32)
    k_eff = lib().orc_row_topk(_ptr(logits_row), _ptr(u_row), _ptr(in_set), logits_row.shape[0],
                               top_k, _ptr(idx), _ptr(g))
    return idx, g, k_eff


def expert_ffn(hidden: int, inter: int, wdtype: str, w13, w13_scale, w2, w2_scale,
               xrow: np.ndarray, act_fp8: bool = False) -> np.ndarray:
    """One expert on one row; with act_fp8, xrow must already be MXFP8-rounded
    (mx8_round) and h is rounded to bf16 and MXFP8 inside."""
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    xrow = np.ascontiguousarray(xrow, dtype=np.float64)
    y = np.zeros(hidden, dtype=np.float64)
    fn = lib().orc_expert_ffn_mx8 if act_fp8 else lib().orc_expert_ffn
    fn(hidden, inter, _DT[wdtype], _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(xrow), _ptr(y))
    return y


def forward(inp, tau: Optional[float] = None, top_k: Optional[int] = None,
            rows: Optional[np.ndarray] = None, threads: int = 0, ffn: bool = True,
            expert_budget: Optional[int] = None, live_rows: Optional[np.ndarray] = None,
            act_fp8: bool = False) -> dict:
    """Whole call.  ``rows``: row indices whose FFN output is computed (None =
    all).  ``expert_budget`` and ``live_rows`` default to the workload's
    (``inp.wl.expert_budget``, ``inp.live_rows``).  ``act_fp8``: MXFP8
    activations into the expert GEMMs (fp8 weights only).  Returns a dict with
    'out' (fp64 [N,H], NaN for rows not computed and for resolved rows) and
    every routing array."""
    wl = inp.wl
    tau = wl.mass_threshold if tau is None else tau
    K = wl.top_k if top_k is None else top_k
    budget = wl.expert_budget if expert_budget is None else expert_budget
    live = inp.live_rows if live_rows is None else live_rows
    if live is not None:
        live = np.ascontiguousarray(live, dtype=np.uint8)
    N, E, B, H = wl.rows, wl.num_experts, wl.num_blocks, wl.hidden
    res = {
        "topk_idx": np.zeros((N, K), np.int32), "gates": np.zeros((N, K), np.float32),
        "coreset_ids": np.zeros((B, E), np.int32), "coreset_size": np.zeros(B, np.int32),
        "expert_counts": np.zeros(E, np.int32), "expert_offsets": np.zeros(E + 1, np.int32),
        "perm": np.zeros(N * K, np.int32), "logits": np.zeros((N, E), np.float32),
        "block_mass": np.zeros((B, E), np.float64),
    }
    rt = _Routing(*[_ptr(res[n]) for n in ("topk_idx", "gates", "coreset_ids", "coreset_size",
                                           "expert_counts", "expert_offsets", "perm", "logits",
                                           "block_mass")])
    out = None
    mask = None
    if ffn:
        out = np.full((N, H), np.nan, dtype=np.float64)
        if rows is not None:
            mask = np.zeros(N, dtype=np.uint8)
            mask[np.asarray(rows)] = 1
    p = _problem(inp)
    w = _weights(inp)
    fn = lib().orc_forward_ex_act8 if act_fp8 else lib().orc_forward_ex
    rc = fn(ctypes.byref(p), ctypes.byref(w), _ptr(inp.x), ctypes.c_float(tau), K, int(budget), _ptr(live),
            _ptr(out), ctypes.byref(rt), _ptr(mask), threads)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    res["out"] = out
    res["top_k"] = K
    res["tau"] = tau
    return res
