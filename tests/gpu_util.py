"""Staging helpers for the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, bring results back as numpy."""
from __future__ import annotations

import sys

import numpy as np

import synth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def assert_parity(y_gpu, y_ref, what):
    """The parity bar: every element bit-identical (float32 bit patterns,
    so -0 differs from +0 and a NaN differs from every number).  The scaled
    error max|gpu - oracle| / max|oracle| is logged beside it."""
    y_gpu = np.asarray(y_gpu, np.float32)
    y_ref = np.asarray(y_ref, np.float32)
    assert y_gpu.shape == y_ref.shape, (what, y_gpu.shape, y_ref.shape)
    bad = np.flatnonzero(y_gpu.view(np.uint32) != y_ref.view(np.uint32))
    scale = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    scale = scale or 1.0
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref))) / scale if y_ref.size else 0.0
    log(f"{what}: {y_ref.size} outputs, {bad.size} differ, scaled error {err:.3g}")
    assert bad.size == 0, (what, bad[:8], y_gpu.ravel()[bad[:4]], y_ref.ravel()[bad[:4]])


def torch():
    import torch as t
    return t


def paired_walk_shapes(fmt: int):
    """Products whose rows span several table chunks (32 blocks: 4096 columns
    of Q1_0, 2048 of Q2_0), ahead of 1024 one-tile products.  A sweep
    dispatches its heaviest work items first and cuts only the last 1024
    back to one tile per wavefront, so the one-tile products take that cut
    and the items of the products in front keep two tiles per wavefront,
    each chunk's table serving both:
      a: 16 tiles (the last one 40 rows), 3 full chunks and a partial one --
         every wavefront two tiles;
      b: 11 tiles, a full chunk and 2 blocks -- three wavefronts two tiles,
         five one;
      c: 40 tiles, two full chunks -- items of 16, 16 and 8 tiles;
      d: 15 tiles of one chunk (the single-chunk walk beside them)."""
    qk = 128 if fmt == 1 else 64
    heavy = [("a", 1000, 100 * qk), ("b", 700, 34 * qk), ("c", 2560, 64 * qk), ("d", 900, 32 * qk)]
    return heavy + [(f"t{i}", 1 + i % 64, 128) for i in range(1024)]


def dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def bqmod():
    import ternary_quantized_gemv_amd as bq
    return bq


def stage_act(q: np.ndarray, d: np.ndarray, qa: int):
    """q int8 [ncols, n], d float32 [ncols, n/qa] -> bq.Act on the device."""
    bq = bqmod()
    q = np.atleast_2d(q)
    d = np.atleast_2d(d)
    ncols, n = q.shape
    return bq.Act(dev(q), dev(d), n, qa, ncols)


def quantize_gpu(x: np.ndarray, qa: int):
    t, bq = torch(), bqmod()
    xd = dev(x.astype(np.float32))
    q = t.empty(x.size, dtype=t.int8, device="cuda")
    d = t.empty(x.size // qa, dtype=t.float32, device="cuda")
    bq.bq_quantize_act_q8(xd, qa, q, d)
    t.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy()


def matvec_gpu(fmt: int, canon: np.ndarray, rows: int, cols: int, q: np.ndarray, d: np.ndarray, qa: int):
    t, bq = torch(), bqmod()
    w = bq.Weights.upload(fmt, canon, rows, cols)
    a = stage_act(q, d, qa)
    y = t.full((a.ncols * rows,), float("nan"), dtype=t.float32, device="cuda")
    (bq.bq_q1_0_matvec if fmt == 1 else bq.bq_q2_0_matvec)(w, a, y)
    t.cuda.synchronize()
    return y.cpu().numpy().reshape(a.ncols, rows)


class SweepWorkload:
    """Seeded products (the 253 of one decode token, or any list of shapes)
    staged on the GPU, one float32 N(0, 1) activation vector per product."""

    def __init__(self, fmt: int, shapes, seed: int, qa: int = 128, f16_scale: bool = False):
        from ternary_quantized_gemv_amd.staging import StagedSweep
        shapes = list(shapes)
        canon = [synth.blocks(fmt, r, c, seed, i) for i, (_, r, c) in enumerate(shapes)]
        x = [synth.activation(c, seed, 1000 + i) for i, (_, _, c) in enumerate(shapes)]
        self.s = StagedSweep(fmt, canon, shapes, x, qa, f16_scale=f16_scale)
        s = self.s
        self.fmt, self.shapes, self.qa, self.f16_scale = fmt, shapes, qa, f16_scale
        self.canon, self.weights, self.entries = s.canon, s.weights, s.entries
        self.koff, self.yoff, self.x = s.koff, s.yoff, s.x
        self.q, self.d, self.y = s.q, s.d, s.y
        self.rows_total = s.rows_total

    def run(self, stream=None):
        self.s.run(stream)

    def close(self):
        self.s.close()
