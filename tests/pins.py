"""Checks that tie the CPU oracle to facts fixed outside it.

Each check takes an ``oracle.Oracle`` and raises AssertionError on a mismatch.
They are run against the real oracle (``test_oracle_pins.py``) and against
copies of it with a planted mistake (``test_oracle_mutants.py``), which must
each fail at least one of them.

What pins what:
  witnesses      hand-derived exact outputs (tests/golden/witnesses.json): the
                 rounded first product, the fused inner and outer steps, the
                 final tree, the lane grouping, the int8 wrap, the Q2_0 code map
  f16            every one of the 65,536 f16 patterns against numpy's widening
  f16 narrowing  f32 -> f16 against numpy's narrowing (nearest, ties to even):
                 every f16 value, every midpoint between neighbours, both
                 sides of each midpoint, random values over all exponents
  quantizer_f16  f16-scale flavour: d is the f16 nearest to amax/127 (exact
                 rationals), quants nearest to x/d, ties away, the clamp at
                 subnormal scales, zero blocks, d = 0 when amax/127 narrows to 0
  f16_merge      with f16-valued scales one per block, d1*s is exact, so the
                 sub-blocks of a block can be taken in any order without
                 changing a bit (and with f32 scales they cannot)
  quantizer      ties, amax -> 127, zero blocks, the correctly rounded scale,
                 nearest-integer property checked in exact rationals, 2x scaling
  exact_q1/q2    power-of-two scales make every float step exact, so the output
                 must equal the integer dot product, decoded here by another route
                 (numpy.unpackbits / base-4 digits)
  bound          random realistic inputs: |y - exact| <= gamma_(nb+7) * sum|terms|
                 with the exact value from math.fsum of exact float64 products
  invariants     negating all weights negates y; rows, threads, row order and
                 activation columns change nothing else; a zero block scale is
                 the same as dropping the block
"""
from __future__ import annotations

import json
import math
import os
import struct
from fractions import Fraction

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
Q1_0, Q2_0 = 1, 2
QK = {Q1_0: 128, Q2_0: 64}


def f32_from_hex(h: str) -> np.float32:
    return np.float32(struct.unpack("<f", bytes.fromhex(h))[0])


def load_witnesses():
    with open(os.path.join(HERE, "golden", "witnesses.json")) as f:
        ws = json.load(f)
    out = []
    for w in ws:
        blocks = np.array(w["blocks"], dtype=np.uint8).reshape(1, -1, 18)
        q = np.array(w["q"], dtype=np.int8)
        d = np.array([f32_from_hex(h) for h in w["d"]], dtype=np.float32)
        out.append(dict(w, blocks=blocks, q=q, d=d, expected=f32_from_hex(w["expected"])))
    return out


def same_bits(a, b) -> bool:
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ witnesses
def check_witnesses(o):
    for w in load_witnesses():
        y = o.matvec(w["fmt"], w["blocks"], 1, w["cols"], w["q"], w["d"], w["qa"])
        assert same_bits(y[0, 0], w["expected"]), (w["name"], float(y[0, 0]), float(w["expected"]))


# ------------------------------------------------------------------------ f16
def check_f16(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_grid_values():
    """Every finite f16 value, as f32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16).astype(np.float32)
    return v[np.isfinite(v)]


def check_f16_narrowing(o):
    fin = _f16_grid_values()
    pos = np.unique(fin[fin >= 0])                       # 0 .. 65504, ascending
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)  # exact in f32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1].astype(np.float64) + pos[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    down = np.nextafter(mids, np.float32(-np.inf))
    g = np.random.default_rng(5)
    rnd = (g.uniform(1, 2, 20000) * 2.0 ** g.integers(-30, 17, 20000)).astype(np.float32)
    tail = np.array([65504, 65519, 65519.996, 65520, 65536, 1e9, np.inf, 2.0 ** -25, 2.0 ** -26,
                     np.float32(2.0 ** -25) * np.float32(1.0000001)], np.float32)
    v = np.concatenate([fin, mids, up, down, rnd, -rnd, tail, -tail])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = o.f32_to_f16(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:5]]
    nan = o.f32_to_f16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


# ------------------------------------------------------------------ quantizer
def check_quantizer_ties(o):
    x = np.zeros(128, np.float32)
    x[:8] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -127.0, 126.5]
    q, d, clamped = o.quantize_q8(x, 128)
    assert d[0] == np.float32(1.0) and clamped == 0
    assert q[:8].tolist() == [127, 3, -3, 1, -1, 2, -127, 127]
    assert not q[8:].any()
    # amax = 127 * 41 gives d = 41 exactly; 20.5 / 41 is exactly 1/2, so the
    # quant is 1 (away from zero).  Multiplying by RN(1/41) instead would give
    # 0.49999997 and the quant 0.
    x = np.zeros(32, np.float32)
    x[:3] = [5207.0, 20.5, -20.5]
    q, d, _ = o.quantize_q8(x, 32)
    assert d[0] == np.float32(41.0) and q[:3].tolist() == [127, 1, -1]


def check_quantizer_zero_block(o):
    x = np.zeros(256, np.float32)
    x[128:] = 1.0
    q, d, _ = o.quantize_q8(x, 128)
    assert d[0] == 0.0 and not q[:128].any()
    assert d[1] == np.float32(1.0) / np.float32(127.0) and (q[128:] == 127).all()


def _correctly_rounded_div(a: np.float32, b: float, got: np.float32) -> bool:
    exact = Fraction(float(a)) / Fraction(b)
    err = abs(Fraction(float(got)) - exact)
    for nb in (np.nextafter(got, np.float32(np.inf)), np.nextafter(got, np.float32(-np.inf))):
        if abs(Fraction(float(nb)) - exact) < err:
            return False
    return True


def check_quantizer_properties(o, qa: int = 32, seed: int = 7):
    x = np.concatenate([synth.activation(1024, seed, 0),
                        synth.layer_shaped(Q1_0, 1, 1024, seed, 1)[1]])
    q, d, clamped = o.quantize_q8(x, qa)
    assert clamped == 0
    assert q.min() >= -127 and q.max() <= 127
    for b in range(x.size // qa):
        xb = x[b * qa:(b + 1) * qa]
        amax = np.abs(xb).max()
        assert _correctly_rounded_div(amax, 127.0, d[b]), b
        i = int(np.argmax(np.abs(xb)))
        assert abs(int(q[b * qa + i])) == 127
        db = Fraction(float(d[b]))
        for k in range(qa):
            r = Fraction(float(xb[k])) / db
            dist = abs(r - int(q[b * qa + k]))
            # one f32 rounding of x/d sits between the rational and the final rounding
            assert dist <= Fraction(1, 2) + Fraction(1, 1 << 17), (b, k)
            if dist > Fraction(1, 2) - Fraction(1, 1 << 17):
                # a (near) tie must go away from zero
                assert abs(int(q[b * qa + k])) >= abs(r), (b, k)


def check_quantizer_scaling(o, seed: int = 8):
    x = synth.activation(4096, seed)
    q1, d1, _ = o.quantize_q8(x, 128)
    q2, d2, _ = o.quantize_q8(x * np.float32(2.0), 128)
    assert np.array_equal(q1, q2) and same_bits(d2, d1 * np.float32(2.0))


# ------------------------------------------------------ exact special cases
def _pow2_inputs(fmt, rows, cols, qa, seed, all_codes=False):
    g = synth.rng(seed, 9)
    w = synth.q2_0_blocks_all_codes(rows, cols, seed, 10) if all_codes else synth.blocks(fmt, rows, cols, seed, 10)
    nb = cols // QK[fmt]
    e0 = g.integers(-1, 3, size=(rows, nb))
    w[:, :, 0:2] = np.exp2(e0).astype(np.float16).view(np.uint16).astype("<u2").view(np.uint8).reshape(rows, nb, 2)
    q = g.integers(-128, 128, size=cols).astype(np.int8)
    q[::37] = -128
    d = np.exp2(g.integers(-2, 1, size=cols // qa)).astype(np.float32)
    return w, q, d, e0


def _q1_products(w, q):
    rows, nb, _ = w.shape
    bits = np.unpackbits(w[:, :, 2:], axis=-1, bitorder="little").reshape(rows, nb * 128).astype(np.int64)
    qq = q.astype(np.int64)[None, :]
    neg = np.where(qq == -128, -128, -qq)
    return np.where(bits == 1, qq, neg)


def _q2_products(w, q):
    rows, nb, _ = w.shape
    by = w[:, :, 2:].astype(np.int64)
    codes = np.stack([by % 4, (by // 4) % 4, (by // 16) % 4, by // 64], axis=-1).reshape(rows, nb * 64)
    return (codes - 1) * q.astype(np.int64)[None, :]


def _exact_sum(fmt, w, q, d, qa, e0):
    prods = _q1_products(w, q) if fmt == Q1_0 else _q2_products(w, q)
    rows, nb, _ = w.shape
    scale = np.exp2(e0.astype(np.float64)).repeat(QK[fmt], axis=1) * d.astype(np.float64).repeat(qa)[None, :]
    return [math.fsum((prods[r] * scale[r]).tolist()) for r in range(rows)]


def check_exact(o, fmt, rows=64, cols=512, qa=32, seed=11, all_codes=False):
    """Power-of-two scales make every step exact, so y is the integer dot
    product decoded another way (numpy.unpackbits / base-4 digits).  With
    all_codes (Q2_0) a quarter of the codes are the unused code 3, which must
    decode as c - 1 = +2 like the others."""
    w, q, d, e0 = _pow2_inputs(fmt, rows, cols, qa, seed, all_codes)
    if all_codes:
        by = w[:, :, 2:]
        n3 = sum(int(np.count_nonzero(((by >> (2 * i)) & 3) == 3)) for i in range(4))
        assert n3 > rows * cols // 8, n3
    y = o.matvec(fmt, w, rows, cols, q, d, qa)[0]
    exact = _exact_sum(fmt, w, q, d, qa, e0)
    assert all(abs(v) < 2.0**20 for v in exact)
    assert np.array_equal(y.astype(np.float64), np.array(exact)), (fmt, rows, cols)


# -------------------------------------------------------------- error bound
def check_bound(o, fmt, rows=48, cols=1024, qa=128, seed=12, layer=False):
    if layer:
        w, x = synth.layer_shaped(fmt, rows, cols, seed)
    else:
        w = synth.blocks(fmt, rows, cols, seed)
        x = synth.activation(cols, seed)
    q, d, _ = o.quantize_q8(x, qa)
    y = o.matvec(fmt, w, rows, cols, q, d, qa)[0]
    nb = cols // QK[fmt]
    prods = _q1_products(w, q) if fmt == Q1_0 else _q2_products(w, q)
    d0 = w[:, :, 0:2].copy().view("<u2").reshape(rows, nb).view(np.float16).astype(np.float64)
    scale = d0.repeat(QK[fmt], axis=1) * d.astype(np.float64).repeat(qa)[None, :]
    u = 2.0**-24
    n = nb + 7
    gamma = n * u / (1 - n * u)
    for r in range(rows):
        terms = (prods[r] * scale[r]).tolist()  # each product is exact in float64
        exact = math.fsum(terms)
        bound = gamma * math.fsum(abs(t) for t in terms)
        assert abs(float(y[r]) - exact) <= bound, (fmt, r, float(y[r]), exact, bound)


# --------------------------------------------------------------- invariants
def check_negation(o, fmt, rows=40, cols=768, qa=128, seed=13):
    w = synth.blocks(fmt, rows, cols, seed)
    q, d, _ = o.quantize_q8(synth.activation(cols, seed), qa)  # never -128
    y = o.matvec(fmt, w, rows, cols, q, d, qa)[0]
    wn = w.copy()
    if fmt == Q1_0:
        wn[:, :, 2:] ^= 0xFF
    else:
        by = wn[:, :, 2:].astype(np.int64)
        digits = [(by >> (2 * i)) & 3 for i in range(4)]
        wn[:, :, 2:] = sum(((2 - c) << (2 * i)) for i, c in enumerate(digits)).astype(np.uint8)
    yn = o.matvec(fmt, wn, rows, cols, q, d, qa)[0]
    assert np.array_equal(yn, -y)


def check_rows_threads_order(o, fmt, rows=203, cols=512, qa=32, seed=14):
    w = synth.blocks(fmt, rows, cols, seed)
    q, d = synth.raw_q8(cols, qa, seed)
    ref = o.matvec(fmt, w, rows, cols, q, d, qa, threads=1)[0]
    for t in (2, 3, 5):
        assert same_bits(o.matvec(fmt, w, rows, cols, q, d, qa, threads=t)[0], ref)
    sub = o.matvec(fmt, w[17:90], 73, cols, q, d, qa)[0]
    assert same_bits(sub, ref[17:90])
    perm = synth.rng(seed, 15).permutation(rows)
    assert same_bits(o.matvec(fmt, w[perm], rows, cols, q, d, qa, threads=3)[0], ref[perm])
    for r in (0, 101, rows - 1):
        assert same_bits(o.row(fmt, w[r], q, d, qa), ref[r])


def check_columns(o, fmt, rows=33, cols=256, qa=128, seed=16):
    w = synth.blocks(fmt, rows, cols, seed)
    qs, ds = [], []
    for c in range(3):
        q, d, _ = o.quantize_q8(synth.activation(cols, seed, c), qa)
        qs.append(q)
        ds.append(d)
    y = o.matvec(fmt, w, rows, cols, np.stack(qs), np.stack(ds), qa, ncols=3)
    for c in range(3):
        assert same_bits(y[c], o.matvec(fmt, w, rows, cols, qs[c], ds[c], qa)[0])


def check_zero_scale_is_dropped_block(o, fmt, rows=21, cols=640, qa=32, seed=17):
    w = synth.blocks(fmt, rows, cols, seed)
    q, d = synth.raw_q8(cols, qa, seed)
    k = QK[fmt]
    b = 2
    wz = w.copy()
    wz[:, b, 0:2] = 0
    y = o.matvec(fmt, wz, rows, cols, q, d, qa)[0]
    keep = [i for i in range(cols // k) if i != b]
    qk = np.concatenate([q[:b * k], q[(b + 1) * k:]])
    dk = np.concatenate([d[:b * k // qa], d[(b + 1) * k // qa:]])
    y2 = o.matvec(fmt, np.ascontiguousarray(w[:, keep]), rows, cols - k, qk, dk, qa)[0]
    assert same_bits(y, y2)


def check_scaling(o, fmt, rows=30, cols=512, qa=128, seed=18):
    w = synth.blocks(fmt, rows, cols, seed)
    x = synth.activation(cols, seed)
    q, d, _ = o.quantize_q8(x, qa)
    q2, d2, _ = o.quantize_q8(x * np.float32(2.0), qa)
    assert same_bits(o.matvec(fmt, w, rows, cols, q2, d2, qa)[0],
                     o.matvec(fmt, w, rows, cols, q, d, qa)[0] * np.float32(2.0))


def _f16_neighbours(d: float):
    """The f16 values just below and above (or equal to) the positive value d."""
    fin = np.unique(_f16_grid_values())
    i = np.searchsorted(fin, d)
    return [float(fin[j]) for j in (i - 1, i, i + 1) if 0 <= j < fin.size]


def check_quantizer_f16(o, seed: int = 11):
    # ties and exact scales carry over: amax = 127 gives d = 1, an f16 value
    x = np.zeros(128, np.float32)
    x[:6] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5]
    q, d, c = o.quantize_q8(x, 128, f16_scale=True)
    assert d[0] == 1.0 and c == 0 and q[:6].tolist() == [127, 3, -3, 1, -1, 2]
    # realistic blocks, a tiny block (subnormal f16 scale, clamp binds) and a zero block
    x = np.concatenate([synth.activation(2048, seed, 0), synth.layer_shaped(Q1_0, 1, 1024, seed, 1)[1],
                        synth.activation(32, seed, 2) * np.float32(1e-6), np.zeros(32, np.float32),
                        np.full(32, 1e-9, np.float32)])
    qa = 32
    q, d, clamped = o.quantize_q8(x, qa, f16_scale=True)
    assert q.min() >= -127 and q.max() <= 127
    for b in range(x.size // qa):
        xb = x[b * qa:(b + 1) * qa]
        amax = Fraction(float(np.abs(xb).max()))
        # d is an f16 value, and the nearest one to the correctly rounded amax / 127
        assert o.f32_to_f16(d[b:b + 1]).view(np.float16).astype(np.float32)[0] == d[b]
        d32 = np.float32(np.abs(xb).max()) / np.float32(127.0)
        assert _correctly_rounded_div(np.abs(xb).max(), 127.0, d32)
        near = min(_f16_neighbours(float(d32)), key=lambda v: (abs(Fraction(v) - Fraction(float(d32)))))
        assert abs(Fraction(float(d[b])) - Fraction(float(d32))) == abs(Fraction(near) - Fraction(float(d32))), b
        if d[b] == 0:
            assert not q[b * qa:(b + 1) * qa].any()
            continue
        db = Fraction(float(d[b]))
        for k in range(qa):
            r = Fraction(float(xb[k])) / db
            if abs(r) > 127 + Fraction(1, 2):
                assert abs(int(q[b * qa + k])) == 127 and (int(q[b * qa + k]) > 0) == (r > 0), (b, k)
                continue
            dist = abs(r - int(q[b * qa + k]))
            assert dist <= Fraction(1, 2) + Fraction(1, 1 << 17), (b, k)
    assert clamped > 0          # the 1e-6 block: d is an f16 subnormal, too coarse for 127 steps
    assert d[-1] == 0.0 and d[-2] == 0.0   # 1e-9 / 127 narrows to 0; the zero block


def _permute_sub_blocks(w: np.ndarray, x: np.ndarray, perm):
    """Q1_0 rows (canonical blocks) and an activation with the four 32-weight
    sub-blocks of every block taken in the order perm."""
    w2 = w.copy()
    pay = w[:, :, 2:].reshape(w.shape[0], w.shape[1], 4, 4)   # sub-block j = payload bytes 4j..4j+3
    w2[:, :, 2:] = pay[:, :, perm, :].reshape(w.shape[0], w.shape[1], 16)
    xb = x.reshape(-1, 4, 32)[:, perm, :].reshape(-1)
    return w2, xb


def check_f16_merge(o, seed: int = 12):
    rows, nb = 64, 16
    cols = nb * 128
    w = synth.q1_0_blocks(rows, cols, seed, 0)
    x = synth.activation(cols, seed, 1)
    perm = [2, 0, 3, 1]
    w2, x2 = _permute_sub_blocks(w, x, perm)
    # f16-valued scales, one per 128 values: every partial sum d1*(s0+..+sj) is exact
    q, d, _ = o.quantize_q8(x, 128, f16_scale=True)
    q2, d2, _ = o.quantize_q8(x2, 128, f16_scale=True)
    assert same_bits(d, d2)
    assert same_bits(o.matvec(Q1_0, w, rows, cols, q, d, 128), o.matvec(Q1_0, w2, rows, cols, q2, d2, 128))
    # with f32 scales the inner chain rounds, and the order shows in some rows
    q, d, _ = o.quantize_q8(x, 128)
    q2, d2, _ = o.quantize_q8(x2, 128)
    assert not same_bits(o.matvec(Q1_0, w, rows, cols, q, d, 128), o.matvec(Q1_0, w2, rows, cols, q2, d2, 128))


def check_cover(o):
    for t in (1, 2, 3, 5):
        for rows in (0, 1, 15, 16, 17, 100, 1000):
            for _ in range(20):
                c = o.cover_rows(rows, t)
                assert c.size == rows and (c == 1).all(), (t, rows)


ALL_CHECKS = [
    ("witnesses", check_witnesses),
    ("f16", check_f16),
    ("quantizer_ties", check_quantizer_ties),
    ("quantizer_zero_block", check_quantizer_zero_block),
    ("quantizer_properties", check_quantizer_properties),
    ("quantizer_scaling", check_quantizer_scaling),
    ("f16_narrowing", check_f16_narrowing),
    ("quantizer_f16", check_quantizer_f16),
    ("f16_merge", check_f16_merge),
    ("exact_q1", lambda o: check_exact(o, Q1_0)),
    ("exact_q2", lambda o: check_exact(o, Q2_0)),
    ("exact_q1_qa128", lambda o: check_exact(o, Q1_0, rows=64, cols=128, qa=128)),
    ("exact_q2_code3", lambda o: check_exact(o, Q2_0, rows=64, cols=512, qa=64, seed=19, all_codes=True)),
    ("bound_q1", lambda o: check_bound(o, Q1_0)),
    ("bound_q2", lambda o: check_bound(o, Q2_0)),
    ("bound_q1_layer", lambda o: check_bound(o, Q1_0, layer=True, qa=32)),
    ("bound_q2_layer", lambda o: check_bound(o, Q2_0, layer=True, qa=32)),
    ("negation_q1", lambda o: check_negation(o, Q1_0)),
    ("negation_q2", lambda o: check_negation(o, Q2_0)),
    ("rows_threads_order_q1", lambda o: check_rows_threads_order(o, Q1_0)),
    ("rows_threads_order_q2", lambda o: check_rows_threads_order(o, Q2_0)),
    ("columns_q1", lambda o: check_columns(o, Q1_0)),
    ("columns_q2", lambda o: check_columns(o, Q2_0)),
    ("zero_scale_q1", lambda o: check_zero_scale_is_dropped_block(o, Q1_0)),
    ("zero_scale_q2", lambda o: check_zero_scale_is_dropped_block(o, Q2_0)),
    ("scaling_q1", lambda o: check_scaling(o, Q1_0)),
    ("scaling_q2", lambda o: check_scaling(o, Q2_0)),
    ("cover", check_cover),
]
