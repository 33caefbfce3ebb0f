"""The small batch with its lane-group sums on the matrix cores
(bq_set_batch_path(BQ_BATCH_MFMA)): every output bit-identical to the oracle.

Cases cover both formats, the three workgroup shapes of the kernel (eight
columns with both slice halves in one wavefront on matrices of more than
1024 row tiles, in two below; four columns with whole sub-blocks for 2-4
columns), one and two column groups (a ragged count pads the last group),
every qa, the -128 regimes (Q1_0's int8 wrap goes through the MFMA
accumulator input), rows not a multiple of 32, and block counts that leave a
partial 4-block chunk.  The table kernels are covered by test_gpu_parity.py,
which forces them."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, bqmod, log, matvec_gpu

pytestmark = pytest.mark.gpu

Q1, Q2 = 1, 2
THREADS = 8


@pytest.fixture
def mfma_path():
    bq = bqmod()
    prev = bq.bq_set_batch_path(bq.BQ_BATCH_MFMA)
    try:
        yield
    finally:
        bq.bq_set_batch_path(prev)


def _inputs(fmt, rows, cols, ncols, qa, regime, seed):
    """Weights and ncols columns.  "quant": the quantizer's output; "raw": raw
    int8 quants with -128 planted; "mixed": -128 only in the last column."""
    w = synth.blocks(fmt, rows, cols, seed, rows, ncols)
    if regime in ("raw", "mixed"):
        qs, ds = zip(*[synth.raw_q8(cols, qa, 11 * c + seed, force_min=regime == "raw") for c in range(ncols)])
        if regime == "mixed":
            qs = [q.copy() for q in qs]
            qs[-1][7] = -128
            qs[-1][cols - 2] = -128
    else:
        qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, seed, c), qa)[:2] for c in range(ncols)])
    return w, np.stack(qs), np.stack(ds)


CASES = [
    # up to 1024 row tiles: each slice half in its own wavefront
    (Q1, 4096, 4096, 8, 128, "quant"),
    (Q1, 4100, 1152, 16, 32, "raw"),       # ragged rows, 9 blocks (a chunk of 1)
    (Q1, 12288, 640, 12, 64, "mixed"),     # two column groups, the second of four
    (Q1, 1000, 128, 9, 128, "raw"),        # one block per row; a group of one column
    (Q2, 4096, 4096, 16, 128, "quant"),
    (Q2, 3001, 320, 8, 64, "raw"),         # 5 blocks
    (Q2, 40001, 576, 11, 32, "quant"),     # 626 ragged tiles
    # more than 1024 row tiles: both slice halves in one wavefront
    (Q1, 65600, 640, 8, 128, "quant"),
    (Q1, 66000, 1152, 16, 64, "raw"),
    (Q1, 65601, 384, 13, 32, "mixed"),
    (Q2, 65600, 448, 8, 32, "raw"),
    (Q2, 65700, 4096, 16, 128, "quant"),
    (Q2, 70000, 320, 10, 64, "raw"),
    # 2-4 columns: four columns per workgroup, whole sub-blocks
    (Q1, 65600, 640, 4, 128, "quant"),
    (Q1, 65601, 384, 2, 64, "mixed"),
    (Q1, 4100, 1152, 3, 32, "raw"),        # few tiles, ragged rows, 9 blocks
    (Q2, 65600, 448, 4, 32, "raw"),
    (Q2, 70000, 320, 3, 64, "quant"),
    (Q2, 3001, 256, 2, 128, "raw"),
]


@pytest.mark.parametrize("fmt,rows,cols,ncols,qa,regime", CASES,
                         ids=[f"q{f}-{r}x{c}-n{n}-qa{a}-{g}" for f, r, c, n, a, g in CASES])
def test_mfma_parity(mfma_path, fmt, rows, cols, ncols, qa, regime):
    name = f"mfma fmt={fmt} {rows}x{cols} N={ncols} qa={qa} {regime}"
    log(name)
    w, q, d = _inputs(fmt, rows, cols, ncols, qa, regime, 61)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


@pytest.mark.parametrize("fmt,rows", [(Q1, 12288), (Q1, 151936), (Q2, 12288)])
def test_mfma_full_size(mfma_path, fmt, rows):
    """The small-batch workloads at their full sizes (qa 128, quantizer output)."""
    cols, qa = 4096, 128
    w = synth.blocks(fmt, rows, cols, 51, rows)
    for ncols in (4, 8, 16):
        name = f"mfma full fmt={fmt} {rows}x{cols} N={ncols}"
        log(name)
        qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, 51, c), qa)[:2] for c in range(ncols)])
        q, d = np.stack(qs), np.stack(ds)
        y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
        assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


def test_mfma_q2_code3(mfma_path):
    """Q2_0 code 3 (+2) through the matrix cores."""
    rows, cols, ncols, qa = 5000, 640, 10, 64
    w = synth.q2_0_blocks_all_codes(rows, cols, 93, rows, ncols)
    qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, 93, c), qa)[:2] for c in range(ncols)])
    q, d = np.stack(qs), np.stack(ds)
    y_ref = oracle.matvec(Q2, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(Q2, w, rows, cols, q, d, qa), y_ref, "mfma Q2_0 code 3")


@pytest.mark.parametrize("fmt,rows,ncols,cols", [(Q1, 20000, 16, 1024), (Q1, 70000, 8, 1024), (Q1, 70000, 6, 1024),
                                                  (Q1, 70000, 3, 1024), (Q2, 20000, 12, 1024), (Q2, 70000, 16, 1024),
                                                  (Q2, 70000, 4, 1024), (Q2, 70000, 5, 1024),
                                                  # Q2_0 rows of one full 32-block chunk
                                                  (Q2, 70000, 6, 2048), (Q2, 20000, 5, 2048)])
def test_batch_paths_agree(fmt, rows, ncols, cols):
    """Both small-batch paths and the automatic choice give the same bits,
    and the same as the oracle."""
    bq = bqmod()
    qa = 128
    w, q, d = _inputs(fmt, rows, cols, ncols, qa, "quant", 67)
    ys = []
    for path in (bq.BQ_BATCH_TABLES, bq.BQ_BATCH_MFMA, bq.BQ_BATCH_AUTO):
        prev = bq.bq_set_batch_path(path)
        try:
            ys.append(matvec_gpu(fmt, w, rows, cols, q, d, qa))
        finally:
            bq.bq_set_batch_path(prev)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(ys[0], y_ref, "tables")
    assert_parity(ys[1], y_ref, "mfma")
    assert_parity(ys[2], y_ref, "auto")


@pytest.mark.parametrize("fmt,rows,ncols", [(Q1, 20000, 6), (Q1, 70000, 6), (Q2, 20000, 5), (Q2, 70000, 9)])
def test_batch_zero_activations(fmt, rows, ncols):
    """Zero quants: an all-zero column (scale 0) and columns with zero
    blocks, on every small-batch path.  Zero table entries and zero lane-group
    sums must come out as +0, as the oracle's integer sums do, so that every
    output bit (the sign of a zero included) matches."""
    bq = bqmod()
    cols, qa = 1024, 64
    w = synth.blocks(fmt, rows, cols, 73, rows, ncols)
    xs = [synth.activation(cols, 73, c) for c in range(ncols)]
    xs[1][:] = 0.0                      # the whole column
    xs[2][: cols // 2] = 0.0            # the first half of the blocks
    xs[-1][qa: 3 * qa] = 0.0            # two blocks inside
    qs, ds = zip(*[oracle.quantize_q8(x, qa)[:2] for x in xs])
    q, d = np.stack(qs), np.stack(ds)
    assert not q[1].any() and not d[1].any()
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    for path, name in ((bq.BQ_BATCH_TABLES, "tables"), (bq.BQ_BATCH_MFMA, "mfma"), (bq.BQ_BATCH_AUTO, "auto")):
        prev = bq.bq_set_batch_path(path)
        try:
            y = matvec_gpu(fmt, w, rows, cols, q, d, qa)
        finally:
            bq.bq_set_batch_path(prev)
        assert_parity(y, y_ref, f"zero activations {name} fmt={fmt} {rows}x{cols} N={ncols}")


@pytest.mark.parametrize("fmt,rows,ncols", [(Q1, 70000, 8), (Q2, 70000, 4), (Q2, 12288, 16)])
def test_mfma_graph_replay(mfma_path, fmt, rows, ncols):
    """A matrix-core product captured in a graph: every replay, with eager
    work and synchronisation between replays, gives the eager bits (and the
    oracle's)."""
    import torch as t
    from gpu_util import stage_act
    bq = bqmod()
    cols, qa = 1024, 128
    w, q, d = _inputs(fmt, rows, cols, ncols, qa, "quant", 71)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    wd = bq.Weights.upload(fmt, w, rows, cols)
    a = stage_act(q, d, qa)
    y = t.full((ncols * rows,), float("nan"), dtype=t.float32, device="cuda")
    f = bq.bq_q1_0_matvec if fmt == Q1 else bq.bq_q2_0_matvec
    f(wd, a, y)
    t.cuda.synchronize()
    assert_parity(y.cpu().numpy().reshape(ncols, rows), y_ref, "mfma eager")
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        f(wd, a, y)  # warm-up on the capture stream
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        f(wd, a, y)
    for rep in range(3):
        y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert_parity(y.cpu().numpy().reshape(ncols, rows), y_ref, f"mfma graph replay {rep}")
        f(wd, a, y)  # eager work between replays
        t.cuda.synchronize()
