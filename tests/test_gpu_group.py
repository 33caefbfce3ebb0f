"""bq_group_matvec: the products of one decode group computed from an f32
activation that the kernel quantizes itself.  Every output must equal the
oracle's quantize_q8 followed by its matvec, bit for bit: ragged rows, one to
four products, one to several table chunks and a short last chunk, every qa,
activations with zero blocks, exact ties, values within a few ulps of a
rounding boundary (where the kernels' reciprocal shortcut must hand over to
the exact division) and subnormal scales, and each
workgroup shape: a quarter tile (groups of at most 64 tiles), half a tile
(up to 128), one tile (up to 256) or two tiles in turn (up to 512) per
sixteen-wavefront workgroup, and
one row per lane with eight tiles per workgroup (more), with odd tile
counts."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bqmod, dev, log, torch
from pins import same_bits

pytestmark = pytest.mark.gpu

THREADS = 16


def near_ties(cols, qa, seed):
    """Blocks whose values sit within a few ulps of (k + 1/2) * d, with d not a
    power of two: x / d lands next to, or on, a rounding boundary."""
    g = np.random.default_rng(seed)
    x = np.empty(cols, np.float32)
    for b in range(cols // qa):
        dt = np.float32(g.uniform(0.01, 3.0))
        k = g.integers(-127, 127, qa)
        v = ((k + 0.5) * np.float64(dt)).astype(np.float32)
        for _ in range(3):  # up to three ulps either way
            step = g.integers(-1, 2, qa)
            v = np.where(step > 0, np.nextafter(v, np.float32(np.inf)),
                         np.where(step < 0, np.nextafter(v, np.float32(-np.inf)), v)).astype(np.float32)
        v[0] = np.float32(127) * dt * (1 if k[0] >= 0 else -1)  # the block maximum: d = fl(amax / 127)
        x[b * qa:(b + 1) * qa] = v
    return x


def group_input(fmt, cols, qa, regime, seed):
    if regime == "layer":
        return synth.layer_shaped(fmt, 1, cols, seed, qa)[1].astype(np.float32)
    if regime == "nearties":
        return near_ties(cols, qa, seed)
    x = synth.activation(cols, seed, qa)
    if regime == "special":
        nblk = cols // qa
        picks = [
            lambda s: s.__setitem__(slice(None), 0.0),                                      # all-zero block
            lambda s: s.__setitem__(slice(0, 6), [127.0, 2.5, -2.5, 0.5, -0.5, 1.5]),      # d = 1: ties
            lambda s: s.__setitem__(slice(0, 3), [5207.0, 20.5, -20.5]),                    # d = 41: x/d = k + 1/2
            lambda s: s.__imul__(np.float32(1e-40)),                                        # subnormal scale
            lambda s: s.__setitem__(slice(None), -3.0),                                     # constant block
        ]
        for i in range(nblk):
            blk = x[i * qa:(i + 1) * qa]
            if i % 2 == 1 or nblk == 1:
                picks[(i // 2) % len(picks)](blk)
    return x


# fmt, rows of each product, blocks per row, qa, regime
CASES = [
    (1, [1], 1, 128, "normal"),
    (1, [300, 64], 33, 32, "nearties"),
    (2, [129, 1000], 40, 128, "nearties"),
    (1, [9000], 32, 64, "nearties"),          # two tiles per wide workgroup
    (1, [1, 63, 65, 130], 3, 32, "special"),
    (1, [300, 64], 96, 128, "normal"),        # three table chunks
    (1, [200], 40, 64, "special"),            # a short last chunk (32 + 8 blocks)
    (1, [4096, 1024, 1024], 32, 128, "layer"),
    (2, [1, 63, 65, 130], 3, 32, "special"),
    (2, [300, 64], 64, 128, "normal"),        # two table chunks
    (2, [129], 37, 64, "layer"),              # 32 + 5 blocks
    (2, [12288, 12288], 64, 128, "normal"),   # 384 tiles
    (1, [8000, 300], 40, 64, "special"),      # 130 tiles: one per workgroup, 32 + 8 blocks
    (2, [9000], 37, 32, "normal"),            # 141 tiles, 32 + 5 blocks
    (1, [20000], 3, 64, "special"),           # 313 tiles: two tiles per wide workgroup
    (1, [20000, 16000, 700, 5], 2, 128, "normal"),  # 575 tiles: one row per lane, partial workgroups
    (2, [40000, 3], 4, 64, "special"),              # 626 tiles
    (1, [40000, 100], 40, 128, "normal"),           # 627 tiles, 32 + 8 blocks
    (2, [33000], 70, 64, "nearties"),               # 516 tiles, three chunks
    (2, [7000, 1100, 300], 70, 32, "special"),      # 133 tiles, three chunks, odd tile counts
    # more than 2048 tiles: fewer busy wavefronts per row-tile workgroup, the rest only build tables
    (1, [100000, 40001, 3], 8, 128, "nearties"),     # 2190 tiles: five per workgroup, ragged last workgroups
    (2, [131072, 2000], 40, 64, "special"),         # 2080 tiles: five per workgroup, 32 + 8 blocks
]


@pytest.mark.parametrize("fmt,rows,nb,qa,regime", CASES)
def test_group_against_oracle(fmt, rows, nb, qa, regime):
    t, bq = torch(), bqmod()
    cols = nb * bq.BLOCK_LEN[fmt]
    seed = 500 + 7 * fmt + nb
    log(f"group fmt={fmt} rows={rows} cols={cols} qa={qa} {regime}")
    canon = [synth.blocks(fmt, r, cols, seed, i) for i, r in enumerate(rows)]
    x = group_input(fmt, cols, qa, regime, seed)
    ws = [bq.Weights.upload(fmt, c, r, cols) for c, r in zip(canon, rows)]
    ys = [t.full((r,), float("nan"), dtype=t.float32, device="cuda") for r in rows]
    bq.bq_group_matvec(ws, dev(x), qa, ys)
    t.cuda.synchronize()
    q, d, clamped = oracle.quantize_q8(x, qa)
    assert clamped == 0
    for i, (c, r) in enumerate(zip(canon, rows)):
        ref = oracle.matvec(fmt, c, r, cols, q, d, qa, threads=THREADS)[0]
        got = ys[i].cpu().numpy()
        assert same_bits(got, ref), f"product {i}: {np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))} differ"


def test_group_rejects_bad_arguments():
    t, bq = torch(), bqmod()
    w1 = bq.Weights.upload(1, synth.blocks(1, 64, 256, 1, 0), 64, 256)
    w2 = bq.Weights.upload(2, synth.blocks(2, 64, 256, 1, 1), 64, 256)
    w3 = bq.Weights.upload(1, synth.blocks(1, 64, 384, 1, 2), 64, 384)
    x = t.zeros(256, device="cuda")
    y = [t.zeros(64, device="cuda") for _ in range(5)]
    for ws, qa, ys, what in [([w1, w2], 128, y[:2], "format"), ([w1, w3], 128, y[:2], "cols"),
                             ([w1] * 5, 128, y, "count"), ([w1], 48, y[:1], "qa")]:
        with pytest.raises(bq.BQError) as e:
            bq.bq_group_matvec(ws, x, qa, ys)
        assert e.value.code == bq.BQ_EARG and what in str(e.value), what
    with pytest.raises(bq.BQError) as e:
        bq.bq_group_matvec([w1], x[1:], 128, y[:1])
    assert e.value.code in (bq.BQ_EARG, bq.BQ_EALIGN)
