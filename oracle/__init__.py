"""CPU oracle for the Q1_0 / Q2_0 quantized matrix-vector product.

TEST INFRASTRUCTURE ONLY: the product library never imports this package.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  The arithmetic lives in ``oracle.c`` (plain scalar C);
this module only marshals numpy arrays through ctypes.

Every function here follows the bankML documentation pages, cited in
``oracle.c`` next to the code that implements each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
FLOOR_SRC = os.path.join(HERE, "host_floor.c")
FLOOR_LIB = os.path.join(HERE, "libhostfloor.so")

Q1_0 = 1
Q2_0 = 2
QK = {Q1_0: 128, Q2_0: 64}
BLOCK_BYTES = 18


GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile ``oracle.c`` (or a variant of it) with plain gcc, no fast-math;
    the default build also compiles the host memory-floor probe."""
    subprocess.run(["gcc", *GCC_FLAGS, "-o", out, src, "-lm", "-lpthread"], check=True)
    if src == SRC:
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-o", FLOOR_LIB, FLOOR_SRC,
                        "-lpthread"], check=True)
    return out


class Oracle:
    """ctypes front end of one build of ``oracle.c`` (the default build, or a
    variant the tests compile with a planted mistake)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        for f in (lib.oracle_quantize_q8, lib.oracle_quantize_q8_f16):
            f.restype = ctypes.c_int64
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        for name in ("oracle_q1_0_row", "oracle_q2_0_row"):
            f = getattr(lib, name)
            f.restype = ctypes.c_float
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_int32]
        lib.oracle_matvec.restype = ctypes.c_int
        lib.oracle_matvec.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_int]
        lib.oracle_cover_rows.restype = ctypes.c_int
        lib.oracle_cover_rows.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        self.lib = lib

    def f16_to_f32(self, bits) -> np.ndarray:
        """Exact widening of f16 bit patterns (uint16) to float32, element by element."""
        b = np.asarray(bits, dtype=np.uint16).ravel()
        out = np.empty(b.shape, dtype=np.float32)
        f = self.lib.oracle_f16_to_f32
        for i, v in enumerate(b.tolist()):
            out[i] = f(v)
        return out

    def f32_to_f16(self, values) -> np.ndarray:
        """f16 bit patterns (uint16) of f32 values, nearest with ties to even."""
        v = np.asarray(values, dtype=np.float32).ravel()
        return np.array([self.lib.oracle_f32_to_f16(float(x)) for x in v], dtype=np.uint16)

    def quantize_q8(self, x: np.ndarray, qa: int, f16_scale: bool = False):
        """Per-block int8 quantization: returns (q int8[n], d f32[n/qa], clamped count).
        f16_scale: the scales are rounded to f16 values first (reading R6)."""
        x = np.ascontiguousarray(x, dtype=np.float32).ravel()
        n = x.size
        if qa <= 0 or n % qa:
            raise ValueError("length must be a multiple of qa")
        q = np.empty(n, dtype=np.int8)
        d = np.empty(n // qa, dtype=np.float32)
        fn = self.lib.oracle_quantize_q8_f16 if f16_scale else self.lib.oracle_quantize_q8
        clamped = fn(_ptr(x), n, qa, _ptr(q), _ptr(d))
        return q, d, int(clamped)

    def row(self, fmt: int, blocks: np.ndarray, q: np.ndarray, d: np.ndarray, qa: int) -> np.float32:
        """One output element: one row of canonical blocks dotted with (q, d)."""
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, BLOCK_BYTES)
        q = np.ascontiguousarray(q, dtype=np.int8)
        d = np.ascontiguousarray(d, dtype=np.float32)
        nb = blocks.shape[0]
        if q.size < nb * QK[fmt] or d.size * qa < nb * QK[fmt]:
            raise ValueError("activation shorter than the row")
        f = self.lib.oracle_q1_0_row if fmt == Q1_0 else self.lib.oracle_q2_0_row
        return np.float32(f(_ptr(blocks), nb, _ptr(q), _ptr(d), qa))

    def matvec(self, fmt: int, canon: np.ndarray, rows: int, cols: int, q: np.ndarray,
               d: np.ndarray, qa: int, ncols: int = 1, threads: int = 1) -> np.ndarray:
        """All rows for all activation columns: float32 [ncols, rows].

        ``canon`` is uint8 [rows, cols/QK, 18]; ``q`` is int8 [ncols, cols] and
        ``d`` float32 [ncols, cols/qa]."""
        canon = np.ascontiguousarray(canon, dtype=np.uint8)
        q = np.ascontiguousarray(q, dtype=np.int8).reshape(ncols, -1)
        d = np.ascontiguousarray(d, dtype=np.float32).reshape(ncols, -1)
        if canon.size != rows * (cols // QK[fmt]) * BLOCK_BYTES:
            raise ValueError("canonical block array has the wrong size")
        if q.shape[1] < cols or d.shape[1] * qa < cols:
            raise ValueError("activation shorter than cols")
        y = np.empty((ncols, rows), dtype=np.float32)
        rc = self.lib.oracle_matvec(fmt, _ptr(canon), rows, cols, _ptr(q), _ptr(d), qa, ncols,
                                    q.shape[1], d.shape[1], _ptr(y), threads)
        if rc != 0:
            raise ValueError("oracle_matvec rejected its arguments")
        return y

    def cover_rows(self, rows: int, threads: int) -> np.ndarray:
        """How many times the row scheduler visits each row (must be exactly once)."""
        counts = np.zeros(max(rows, 1), dtype=np.int32)
        self.lib.oracle_cover_rows(rows, threads, _ptr(counts))
        return counts[:rows]


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default


def f16_to_f32(bits):
    return default().f16_to_f32(bits)


def quantize_q8(x, qa, f16_scale=False):
    return default().quantize_q8(x, qa, f16_scale)


def f32_to_f16(values):
    return default().f32_to_f16(values)


def row(fmt, blocks, q, d, qa):
    return default().row(fmt, blocks, q, d, qa)


def matvec(fmt, canon, rows, cols, q, d, qa, ncols=1, threads=1):
    return default().matvec(fmt, canon, rows, cols, q, d, qa, ncols, threads)


def cover_rows(rows, threads):
    return default().cover_rows(rows, threads)


def host_read_floor(nbytes: int, thread_counts, reps: int = 3) -> list:
    """The host's streaming-read bandwidth (GB/s, median of reps passes) over
    a buffer of nbytes, for each thread count (host_floor.c).  A measurement
    aid of the benchmark's CPU leg, not part of the oracle's arithmetic."""
    if not os.path.exists(FLOOR_LIB) or os.path.getmtime(FLOOR_LIB) < os.path.getmtime(FLOOR_SRC):
        build()
    lib = ctypes.CDLL(FLOOR_LIB)
    lib.host_read_floor.restype = ctypes.c_int
    lib.host_read_floor.argtypes = [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    tc = np.ascontiguousarray(thread_counts, dtype=np.int32)
    out = np.zeros(tc.size, dtype=np.float64)
    rc = lib.host_read_floor(int(nbytes), _ptr(tc), int(tc.size), int(reps), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"host_read_floor failed ({rc})")
    return [float(v) for v in out]
