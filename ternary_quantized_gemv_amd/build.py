"""Builds libbq.so (HIP for gfx950) in-tree with hipcc.

python ternary_quantized_gemv_amd/build.py   (runs without importing the package)

Each source compiles to an object of its own under _build/ (in parallel),
then one hipcc line links the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbq.so")
SOURCES = [os.path.join(CSRC, f) for f in ("bq_sweep.hip", "bq_cols.hip", "bq_mfma.hip", "bq_group.hip", "bq_quantize.hip",
                                            "bq_floor.hip", "bq_api.cpp", "bq_pack.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("bq_layout.h", "bq_types.h", "bq_device.h", "bq_split.h",
                                            "bq_launch.h")] + [os.path.join(ROOT, "include", "bq.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _quiet(text: str) -> str:
    return "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and "unused during compilation" not in l)


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    # .cpp sources hold host code only; they go through hipcc as C++ all the same
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", "-o", obj + ".tmp", src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({r.returncode}):\n{_quiet(r.stdout + r.stderr)}")
    os.replace(obj + ".tmp", obj)
    return obj, _quiet(r.stdout + r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 8)) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for obj, out in results:
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{_quiet(r.stdout + r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


def asm(out: str, source: str = "bq_sweep.hip") -> str:
    """Device assembly of the kernels of one source file (for inspection)."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           "-o", out, os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
