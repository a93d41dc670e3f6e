"""Build of the HIP library libclover_moe.so for gfx950 (hipcc, in-tree), and
of libclover_moe_peaks.so, the benchmark's achievable-peak probes (not part of
the library's C ABI).

Every HIP source is compiled with fp contraction off (the routing steps rely
on the exact operation sequence written in the source) and with packed fp32
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libclover_moe.so")
SOURCES = ["api.cpp", "router.hip", "route_block.hip", "permute_blocks.hip", "expert_gemm.hip",
           "expert_tiled.hip", "expert_many.hip", "quant.hip", "combine.hip", "pack.hip"]
PEAKS_LIB = os.path.join(PKG, "libclover_moe_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
          "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out:
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build() -> str:
    """Compile every source, link libclover_moe.so and libclover_moe_peaks.so;
    returns the path of the former."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
