"""Build the gfx950 MoE library (libmoe_mi355x.so) in-tree with hipcc, and the
small calibration library (libmoe_calibrate.so: MFMA-loop and streaming-read
kernels the benchmark reports beside the nominal peaks).

Usage: python -m mixture_experts_layer_31_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB = os.path.join(PKG, LIB_NAME)

SOURCES = ["moe_api.hip", "router.hip", "index.hip", "rows.hip", "gemm_bf16.hip", "gemm_f32.hip",
           "backward.hip", "gemm_kmajor.hip", "noalloc.hip"]
CALIB_SOURCE = "calibrate.hip"
CALIB_LIB = os.path.join(PKG, "libmoe_calibrate.so")

# packed fp32 VALU ops are disabled: the compiler would otherwise form them from
# plain float code, and this build keeps every fp32 operation scalar
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Always rebuilds."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
                    "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max(1, min(len(SOURCES) + 1, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, SOURCES + [CALIB_SOURCE]))
    calib_obj = objs.pop()
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = CALIB_LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, calib_obj])
    os.replace(tmp, CALIB_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
