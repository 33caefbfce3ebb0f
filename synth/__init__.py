"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it only draws random numbers
and lays them out in the canonical block format, so that the CPU oracle and the
HIP path can be fed the very same bytes.

Canonical block (18 bytes): f16 scale (little-endian bit pattern), then 16 payload
bytes.  Q1_0 payload: 128 sign bits, weight k in bit (k & 7) of byte (k >> 3).
Q2_0 payload: 64 two-bit codes, weight k in bits 2(k&3)..2(k&3)+1 of byte (k >> 2),
codes drawn from {0, 1, 2} (weights -1, 0, +1) with probability 1/3 each.

Distributions follow the workloads the pages describe: sign bits uniform, block
scales |N(0, 0.02)| rounded to f16 (numpy's round-to-nearest-even conversion),
activations N(0, 1) in float32.  Every array is a pure function of
(seed, stream...), drawn from numpy's PCG64 through a SeedSequence, so any
matrix of a workload can be regenerated on its own.
"""
from __future__ import annotations

import numpy as np

Q1_0 = 1
Q2_0 = 2
QK = {Q1_0: 128, Q2_0: 64}
BLOCK_BYTES = 18

# Qwen3-8B-shaped decode step: 36 layers of seven projections, then the LM head
# (253 matrix-vector products).  (name, rows, cols)
LAYER_SHAPES = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 12288, 4096),
    ("up", 12288, 4096),
    ("down", 4096, 12288),
)
N_LAYERS = 36
LM_HEAD = ("lm_head", 151936, 4096)


def decode_sweep_shapes(n_layers: int = N_LAYERS, lm_head: bool = True):
    """[(name, rows, cols)] of one decode token's 253 products, layer by layer."""
    out = []
    for layer in range(n_layers):
        for name, r, c in LAYER_SHAPES:
            out.append((f"l{layer}.{name}", r, c))
    if lm_head:
        out.append(LM_HEAD)
    return out


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def scales_f16(g: np.random.Generator, n: int, sigma: float = 0.02) -> np.ndarray:
    """f16 bit patterns (uint16) of |N(0, sigma)|."""
    return np.abs(g.standard_normal(n) * sigma).astype(np.float16).view(np.uint16)


def _assemble(scales: np.ndarray, payload: np.ndarray, rows: int, nb: int) -> np.ndarray:
    out = np.empty((rows, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = scales.reshape(rows, nb).astype("<u2").view(np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = payload.reshape(rows, nb, 16)
    return out


def q1_0_blocks(rows: int, cols: int, seed: int, *stream: int, sigma: float = 0.02) -> np.ndarray:
    """Canonical Q1_0 weights: uint8 [rows, cols/128, 18]."""
    if cols % 128:
        raise ValueError("Q1_0 needs cols % 128 == 0")
    nb = cols // 128
    g = rng(seed, 1, *stream)
    sc = scales_f16(g, rows * nb, sigma)
    bits = g.integers(0, 256, size=rows * nb * 16, dtype=np.uint8)
    return _assemble(sc, bits, rows, nb)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Four 2-bit codes per byte, first code in the low bits (canonical Q2_0 payload)."""
    c = codes.reshape(-1, 4).astype(np.uint8)
    return (c[:, 0] | (c[:, 1] << 2) | (c[:, 2] << 4) | (c[:, 3] << 6)).astype(np.uint8)


def _code_bytes() -> np.ndarray:
    """The 81 payload bytes whose four 2-bit codes all lie in {0, 1, 2}."""
    c = np.array([(i % 3, i // 3 % 3, i // 9 % 3, i // 27) for i in range(81)], dtype=np.uint8)
    return pack_codes(c.ravel())


def q2_0_blocks(rows: int, cols: int, seed: int, *stream: int, sigma: float = 0.02) -> np.ndarray:
    """Canonical Q2_0 weights: uint8 [rows, cols/64, 18].  Each payload byte's
    four codes are drawn together: a uniform 16-bit draw u picks combination
    (81 * u) >> 16 of the 81, so each code is 0, 1 or 2 with probability 1/3
    (to within 81/65536 relative)."""
    if cols % 64:
        raise ValueError("Q2_0 needs cols % 64 == 0")
    nb = cols // 64
    g = rng(seed, 2, *stream)
    sc = scales_f16(g, rows * nb, sigma)
    table = _code_bytes()
    total = rows * nb * 16
    payload = np.empty(total, dtype=np.uint8)
    step = 1 << 24  # drawn in slices to bound host memory
    for s in range(0, total, step):
        e = min(s + step, total)
        u = g.integers(0, 65536, size=e - s, dtype=np.uint32)
        payload[s:e] = table[(u * 81) >> 16]
    return _assemble(sc, payload, rows, nb)


def q2_0_blocks_all_codes(rows: int, cols: int, seed: int, *stream: int, sigma: float = 0.02) -> np.ndarray:
    """Canonical Q2_0 weights whose payload bytes are uniform over all 256
    values, so the unused code 3 appears with probability 1/4 (a test regime
    for its defined decoding, not a workload): uint8 [rows, cols/64, 18]."""
    if cols % 64:
        raise ValueError("Q2_0 needs cols % 64 == 0")
    nb = cols // 64
    g = rng(seed, 7, *stream)
    sc = scales_f16(g, rows * nb, sigma)
    payload = g.integers(0, 256, size=rows * nb * 16, dtype=np.uint8)
    return _assemble(sc, payload, rows, nb)


def blocks(fmt: int, rows: int, cols: int, seed: int, *stream: int, **kw) -> np.ndarray:
    return (q1_0_blocks if fmt == Q1_0 else q2_0_blocks)(rows, cols, seed, *stream, **kw)


def activation(n: int, seed: int, *stream: int) -> np.ndarray:
    """float32 N(0, 1) activation vector."""
    return rng(seed, 3, *stream).standard_normal(n, dtype=np.float32)


def raw_q8(n: int, qa: int, seed: int, *stream: int, force_min: bool = True):
    """Hand-made int8 activations (the pages' test regime): quants uniform over
    [-128, 127], a -128 planted in every 16th lane group, and f16-valued block
    scales.  Returns (q int8[n], d float32[n/qa])."""
    g = rng(seed, 4, *stream)
    q = g.integers(-128, 128, size=n, dtype=np.int16).astype(np.int8)
    if force_min:
        q[::64] = -128
    d = scales_f16(g, n // qa, sigma=0.05).view(np.float16).astype(np.float32)
    return q, d


def layer_shaped(fmt: int, rows: int, cols: int, seed: int, *stream: int):
    """A "layer-shaped" regime: block scales spread over many binades and
    activations whose magnitude changes from block to block, so that the
    products are inexact in float32.  Returns (canonical blocks, x float32[cols])."""
    g = rng(seed, 5, *stream)
    w = blocks(fmt, rows, cols, seed, 6, *stream)
    nb = cols // QK[fmt]
    e = g.integers(-14, 8, size=(rows, nb))
    sc = (np.abs(g.standard_normal((rows, nb))) * np.exp2(e)).astype(np.float16).view(np.uint16)
    w[:, :, 0:2] = sc.astype("<u2").view(np.uint8).reshape(rows, nb, 2)
    x = g.standard_normal(cols).astype(np.float32)
    x *= np.exp2(g.integers(-20, 12, size=cols // 32)).repeat(32).astype(np.float32)
    return w, x
