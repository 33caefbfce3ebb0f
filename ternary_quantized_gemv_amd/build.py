"""Builds libbq.so (HIP for gfx950) in-tree with hipcc.

python ternary_quantized_gemv_amd/build.py   (runs without importing the package)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbq.so")
SOURCES = [os.path.join(CSRC, f) for f in ("bq_sweep.hip", "bq_cols.hip", "bq_group.hip", "bq_quantize.hip", "bq_floor.hip",
                                            "bq_api.cpp",
                                            "bq_pack.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("bq_layout.h", "bq_types.h", "bq_device.h", "bq_split.h", "bq_launch.h")] + [os.path.join(ROOT, "include", "bq.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # the dot-product order is spelled out with explicit fma; nothing else may fuse
    "-ffp-contract=off",
    # packed fp32 instructions stay off (scalar fp32 VALU only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


def asm(out: str, source: str = "bq_sweep.hip") -> str:
    """Device assembly of the kernels of one source file (for inspection)."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           "-o", out, os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
