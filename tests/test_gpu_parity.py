"""The HIP path (through the C ABI) against the CPU oracle, element by element.

The bar is bit-exact equality for every output element: the order of every
rounding is fixed (bankML "gpu/ -- the video-card component", section
"kernels.rs -- the Q1_0 kernels"), so exactly one result is correct.  The
scaled error max|gpu - oracle| / max|oracle| is reported beside it.  Several
columns run on the table kernels here (bq_set_batch_path(BQ_BATCH_TABLES));
the matrix-core path has its own cases in test_gpu_mfma.py.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import SweepWorkload, assert_parity, log, matvec_gpu, paired_walk_shapes, quantize_gpu, torch
from pins import load_witnesses, same_bits

pytestmark = pytest.mark.gpu

Q1, Q2 = 1, 2
QK = {Q1: 128, Q2: 64}
THREADS = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import ternary_quantized_gemv_amd as bq  # fails loudly if libbq.so is missing
    prev = bq.bq_set_batch_path(bq.BQ_BATCH_TABLES)
    try:
        yield
    finally:
        bq.bq_set_batch_path(prev)


# --------------------------------------------------------------- witnesses
@pytest.mark.parametrize("w", load_witnesses(), ids=lambda w: w["name"])
def test_witness_gpu(w):
    log("witness", w["name"])
    y = matvec_gpu(w["fmt"], w["blocks"], 1, w["cols"], w["q"], w["d"], w["qa"])
    assert same_bits(y[0, 0], w["expected"]), (float(y[0, 0]), float(w["expected"]))


# ---------------------------------------------------------------- quantizer
@pytest.mark.parametrize("qa", [32, 64, 128])
@pytest.mark.parametrize("regime", ["normal", "layer", "special"])
def test_quantizer_parity(qa, regime):
    log("quantizer", qa, regime)
    n = 12288 + 384
    if regime == "normal":
        x = synth.activation(n, 21, qa)
    elif regime == "layer":
        x = synth.layer_shaped(Q1, 1, n, 22, qa)[1]
    else:
        x = synth.activation(n, 23, qa)
        x[:qa] = 0.0                                     # an all-zero block
        x[qa:2 * qa] = 0.0
        x[qa:qa + 6] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5]  # d = 1: exact ties
        x[2 * qa:2 * qa + 3] = [5207.0, 20.5, -20.5]       # d = 41: x/d = 1/2 exactly
        x[3 * qa:4 * qa] *= np.float32(1e-30)              # tiny scale
        x[5 * qa:6 * qa] *= np.float32(1e-40)              # subnormal values and scale
        x[4 * qa:5 * qa] = -3.0                            # constant block
    q_ref, d_ref, clamped = oracle.quantize_q8(x, qa)
    assert clamped == 0
    q, d = quantize_gpu(x, qa)
    assert np.array_equal(q, q_ref)
    assert same_bits(d, d_ref)


# ------------------------------------------------------- small-shape matvec
SHAPES = [(1, 1), (64, 4), (100, 33), (513, 8), (1000, 64), (130, 70)]  # (rows, blocks per row)


def _cases():
    out = []
    for fmt in (Q1, Q2):
        for rows, nb in SHAPES:
            cols = nb * QK[fmt]
            for qa in (32, 64, 128):
                if cols % qa:
                    continue
                for regime in ("quant", "raw", "layer"):
                    out.append((fmt, rows, cols, qa, regime))
    return out


def _inputs(fmt, rows, cols, qa, regime, seed):
    if regime == "layer":
        w, x = synth.layer_shaped(fmt, rows, cols, seed)
        q, d, _ = oracle.quantize_q8(x, qa)
    elif regime == "raw":
        w = synth.blocks(fmt, rows, cols, seed)
        q, d = synth.raw_q8(cols, qa, seed)
    else:
        w = synth.blocks(fmt, rows, cols, seed)
        q, d, _ = oracle.quantize_q8(synth.activation(cols, seed), qa)
    return w, q, d


@pytest.mark.parametrize("fmt,rows,cols,qa,regime", _cases())
def test_matvec_parity_small(fmt, rows, cols, qa, regime):
    name = f"matvec fmt={fmt} {rows}x{cols} qa={qa} {regime}"
    log(name)
    w, q, d = _inputs(fmt, rows, cols, qa, regime, seed=rows * 7 + cols)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


@pytest.mark.parametrize("fmt", [Q1, Q2])
@pytest.mark.parametrize("ncols", [2, 4, 16])
def test_matvec_columns(fmt, ncols):
    rows, cols, qa = 200, 33 * 128, 128
    log(f"columns fmt={fmt} ncols={ncols}")
    w = synth.blocks(fmt, rows, cols, 31)
    qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, 31, c), qa)[:2] for c in range(ncols)])
    q, d = np.stack(qs), np.stack(ds)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, f"columns fmt={fmt} ncols={ncols}")


# Several columns on the wide shapes, chosen for the tiles of all columns
# together: quarter (2 x 30 tiles), half (3 x 32), one tile (5 x 47), two
# tiles in turn (4 x 65, 4 x 128 = 512), then the split walk (3 x 200).
WIDE_COLS = [
    (Q1, 1900, 4096, 2, 128, "quant"), (Q2, 2000, 2048, 3, 64, "raw"), (Q1, 3000, 4096, 5, 32, "mixed"),
    (Q2, 4100, 2048, 4, 128, "quant"), (Q1, 8192, 1024, 4, 64, "raw"), (Q2, 12800, 1024, 3, 128, "quant"),
]


@pytest.mark.parametrize("fmt,rows,cols,ncols,qa,regime", WIDE_COLS,
                         ids=[f"q{f}-{r}x{c}-n{n}-qa{a}-{g}" for f, r, c, n, a, g in WIDE_COLS])
def test_columns_wide_shapes(fmt, rows, cols, ncols, qa, regime):
    name = f"wide columns fmt={fmt} {rows}x{cols} N={ncols} qa={qa} {regime}"
    log(name)
    w, q, d = _batch_inputs(fmt, rows, cols, ncols, qa, regime)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


def _batch_cases():
    out = []
    for fmt in (Q1, Q2):
        for rows, nb in ((100, 33), (72, 17), (64, 8), (129, 9)):
            for ncols in (2, 3, 5, 8, 16):
                for qa, regime in ((128, "quant"), (32, "raw"), (64, "raw"), (64, "mixed")):
                    if (nb * QK[fmt]) % qa == 0:
                        out.append((fmt, rows, nb * QK[fmt], ncols, qa, regime))
    return out


def _batch_inputs(fmt, rows, cols, ncols, qa, regime):
    """Seeded weights and ncols activation columns.  "quant": the quantizer's
    output; "raw": raw int8 quants with q = -128 planted (the wrap of int8
    negation in Q1_0); "mixed": -128 only near both ends of the last column."""
    w = synth.blocks(fmt, rows, cols, rows + ncols)
    if regime in ("raw", "mixed"):
        qs, ds = zip(*[synth.raw_q8(cols, qa, 7 * c + rows, force_min=regime == "raw") for c in range(ncols)])
        if regime == "mixed":
            qs = [q.copy() for q in qs]
            qs[-1][5] = -128
            qs[-1][cols - 3] = -128
    else:
        qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, rows, c), qa)[:2] for c in range(ncols)])
    return w, np.stack(qs), np.stack(ds)


@pytest.mark.parametrize("fmt,rows,cols,ncols,qa,regime", _batch_cases())
def test_small_batch_parity(fmt, rows, cols, ncols, qa, regime):
    """Several activation columns against one small matrix (the wide shapes,
    one grid row per column)."""
    name = f"batch fmt={fmt} {rows}x{cols} N={ncols} qa={qa} {regime}"
    log(name)
    w, q, d = _batch_inputs(fmt, rows, cols, ncols, qa, regime)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


# Tall matrices (more than 1024 row tiles): four or more columns run four per
# workgroup from interleaved tables (including a last group of 1-3 columns),
# fewer on the one-row-per-lane kernel; ragged row counts, ragged last chunks
# (blocks not a multiple of 4), every qa and the -128 regimes.
TALL = [
    (Q1, 65600, 640, 5, 128, "quant"), (Q1, 65600, 640, 16, 32, "raw"), (Q1, 65601, 384, 8, 64, "mixed"),
    (Q1, 65536 + 64 * 7 + 3, 4096, 9, 128, "quant"), (Q1, 65600, 640, 3, 32, "raw"), (Q1, 65600, 256, 1, 64, "raw"),
    (Q1, 65600, 1152, 4, 32, "raw"), (Q1, 65600, 128, 6, 128, "mixed"),
    (Q2, 65600, 320, 5, 64, "raw"), (Q2, 65600, 448, 16, 32, "quant"), (Q2, 65700, 4096, 12, 128, "quant"),
    (Q2, 65601, 192, 13, 64, "mixed"), (Q2, 65600, 320, 2, 32, "raw"), (Q2, 65600, 576, 4, 64, "raw"),
]


@pytest.mark.parametrize("fmt,rows,cols,ncols,qa,regime", TALL,
                         ids=[f"q{f}-{r}x{c}-n{n}-qa{a}-{g}" for f, r, c, n, a, g in TALL])
def test_small_batch_tall(fmt, rows, cols, ncols, qa, regime):
    name = f"tall batch fmt={fmt} {rows}x{cols} N={ncols} qa={qa} {regime}"
    log(name)
    w, q, d = _batch_inputs(fmt, rows, cols, ncols, qa, regime)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


# Several columns on matrices of up to 1024 row tiles past the wide shapes:
# the split-columns kernel, four columns per workgroup from interleaved
# tables, eight wavefronts per tile (one tile per workgroup) or four (two,
# three or four tiles), the shape chosen so the workgroups fit one round of
# the GPU (else two tiles per workgroup), with 16-block table chunks where
# the workgroups fit one round and rows are longer than 8 blocks, else
# 8-block ones.  Cases: each shape and format, rows ragged, rows of 5 / 8 /
# 9 / 10 / 24 / 32 / 34 / 96 blocks (partial and several chunks of either
# length), a last group of one to three columns, every qa, the -128
# regimes, 1024 tiles.
SPLITCOLS = [
    (Q1, 12800, 1152, 3, 128, "quant"),   # 200 tiles: eight per tile; 9 blocks (8 + 1)
    (Q2, 12801, 576, 3, 64, "raw"),       # 201 ragged tiles, eight per tile
    (Q1, 19200, 4096, 2, 32, "raw"),      # 300 tiles: four per tile, two tiles per workgroup
    (Q2, 19250, 2176, 5, 128, "quant"),   # 301 tiles, five columns: four per tile, three tiles; 34 blocks
    (Q1, 44800, 1024, 2, 64, "mixed"),    # 700 tiles: four per tile, three tiles
    (Q1, 4096, 12288, 16, 128, "raw"),    # 64 tiles, sixteen columns: eight per tile; 96 blocks
    (Q2, 8192, 4096, 8, 64, "quant"),     # 128 tiles, eight columns: eight per tile
    (Q1, 65536, 640, 6, 32, "quant"),     # 1024 tiles, six columns: no shape fits one round, two tiles
    (Q2, 65536, 512, 3, 64, "raw"),       # 1024 tiles: four per tile, four tiles
    (Q2, 6400, 2048, 7, 32, "mixed"),     # 100 tiles, seven columns (a group of three)
    # chunk lengths: 1024 tiles x 2 column groups fit no round (two tiles per workgroup, 8-block
    # chunks: 8 + 2 blocks); 192 workgroups with 16-block chunks, 24 blocks (16 + 8)
    (Q1, 65536, 1280, 6, 64, "raw"),
    (Q2, 12288, 1536, 4, 128, "quant"),
]


@pytest.mark.parametrize("fmt,rows,cols,ncols,qa,regime", SPLITCOLS,
                         ids=[f"q{f}-{r}x{c}-n{n}-qa{a}-{g}" for f, r, c, n, a, g in SPLITCOLS])
def test_small_batch_split_columns(fmt, rows, cols, ncols, qa, regime):
    name = f"split columns fmt={fmt} {rows}x{cols} N={ncols} qa={qa} {regime}"
    log(name)
    w, q, d = _batch_inputs(fmt, rows, cols, ncols, qa, regime)
    y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


# ------------------------------------------------- full-size single products
FULL = [
    (Q1, 4096, 4096), (Q1, 12288, 4096), (Q1, 4096, 12288), (Q1, 151936, 4096),
    (Q2, 4096, 4096), (Q2, 1024, 4096), (Q2, 12288, 4096), (Q2, 4096, 12288),
    # 100, 313 and 700 tiles: half a tile and two tiles per wide workgroup; the four-wavefront split
    (Q1, 6400, 2048), (Q2, 6390, 4096), (Q1, 20000, 4096), (Q2, 20000, 2048), (Q1, 44800, 1024),
    # one row per lane with fewer than eight tiles per workgroup: 2374 tiles (five per workgroup),
    # 2051 ragged tiles (five, the last workgroup one), 2188 tiles of two table chunks each
    (Q2, 151936, 4096), (Q1, 131201, 1024), (Q2, 140001, 4096),
    # Q2_0 rows of one full 32-block chunk: the four-wavefront split (700 tiles), two tiles per wide
    # workgroup (438 tiles), one row per lane (1094 tiles)
    (Q2, 44800, 2048), (Q2, 28000, 2048), (Q2, 70000, 2048),
    # three half tiles per workgroup in turn over two table chunks (the units' two ab buffers
    # across a chunk boundary)
    (Q1, 20000, 8192),
]


@pytest.mark.parametrize("fmt,rows,cols", FULL, ids=[f"q{f}-{r}x{c}" for f, r, c in FULL])
def test_matvec_full_size(fmt, rows, cols):
    name = f"full fmt={fmt} {rows}x{cols}"
    log(name)
    w = synth.blocks(fmt, rows, cols, 41, rows, cols)
    x = synth.activation(cols, 41, rows)
    q_ref, d_ref, _ = oracle.quantize_q8(x, 128)
    q, d = quantize_gpu(x, 128)
    assert np.array_equal(q, q_ref) and same_bits(d, d_ref)
    y_ref = oracle.matvec(fmt, w, rows, cols, q_ref, d_ref, 128, threads=THREADS)
    assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, 128), y_ref, name)


@pytest.mark.parametrize("fmt,rows", [(Q1, 12288), (Q1, 151936), (Q2, 12288)])
def test_small_batch_full_size(fmt, rows):
    cols, qa = 4096, 128
    w = synth.blocks(fmt, rows, cols, 51, rows)
    for ncols in (1, 4, 8, 16):
        name = f"small batch fmt={fmt} {rows}x{cols} N={ncols}"
        log(name)
        qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, 51, c), qa)[:2] for c in range(ncols)])
        q, d = np.stack(qs), np.stack(ds)
        y_ref = oracle.matvec(fmt, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
        assert_parity(matvec_gpu(fmt, w, rows, cols, q, d, qa), y_ref, name)


# -------------------------------------- Q2_0 code 3: its defined decoding
# Code 3 never occurs in ternary weights; the layout contract decodes it as
# c - 1 = +2 on both sides.  Payload bytes uniform over all 256 values (a
# quarter of the codes are 3), through every kernel path.
CODE3 = [
    (1024, 4096, 1, 128),    # 16 tiles: wide kernel, quarter tiles
    (2000, 2048, 3, 64),     # 96 tiles over three columns: half tiles, one grid row per column
    (44800, 1024, 1, 128),   # 700 tiles: four wavefronts per tile
    (131201, 1024, 1, 32),   # 2051 tiles: one row per lane
    (65600, 320, 5, 64),     # tall, five columns: interleaved four-column tables
]


@pytest.mark.parametrize("rows,cols,ncols,qa", CODE3, ids=[f"{r}x{c}-n{n}-qa{a}" for r, c, n, a in CODE3])
def test_q2_code3_parity(rows, cols, ncols, qa):
    name = f"Q2_0 code 3 {rows}x{cols} N={ncols} qa={qa}"
    log(name)
    w = synth.q2_0_blocks_all_codes(rows, cols, 91, rows, ncols)
    qs, ds = zip(*[oracle.quantize_q8(synth.activation(cols, 91, c), qa)[:2] for c in range(ncols)])
    q, d = np.stack(qs), np.stack(ds)
    y_ref = oracle.matvec(Q2, w, rows, cols, q, d, qa, ncols=ncols, threads=THREADS)
    assert_parity(matvec_gpu(Q2, w, rows, cols, q, d, qa), y_ref, name)


def test_q2_code3_sweeps_and_group():
    """Code 3 through the token sweep (two launches and one launch) and a
    fused decode group."""
    import ternary_quantized_gemv_amd as bq
    from ternary_quantized_gemv_amd.staging import StagedSweep
    t = torch()
    shapes = [("a", 100, 33 * 64), ("b", 700, 4096), ("c", 130, 96 * 64), ("d", 64, 64)]
    canon = [synth.q2_0_blocks_all_codes(r, c, 92, i) for i, (_, r, c) in enumerate(shapes)]
    x = [synth.activation(c, 92, 100 + i) for i, (_, _, c) in enumerate(shapes)]
    sw = StagedSweep(Q2, canon, shapes, x, 64)
    try:
        q_ref, d_ref, _ = oracle.quantize_q8(sw.x, 64)
        refs = []
        for i, (_, rows, cols) in enumerate(shapes):
            k0, k1 = int(sw.koff[i]), int(sw.koff[i + 1])
            refs.append(oracle.matvec(Q2, canon[i], rows, cols, q_ref[k0:k1], d_ref[k0 // 64:k1 // 64], 64,
                                      threads=THREADS)[0])
        for how in ("two launches", "one launch"):
            sw.y.fill_(float("nan"))
            sw.run() if how == "two launches" else sw.sweep_fused()
            t.cuda.synchronize()
            y = sw.y.cpu().numpy()
            for i, (nm, _, _) in enumerate(shapes):
                assert_parity(y[int(sw.yoff[i]):int(sw.yoff[i + 1])], refs[i], f"code 3 sweep, {how}, {nm}")
        ys = [t.empty(shapes[i][1], dtype=t.float32, device="cuda") for i in (1,)]
        bq.bq_group_matvec([sw.weights[1]], sw.xd[int(sw.koff[1]):int(sw.koff[2])], 64, ys)
        t.cuda.synchronize()
        assert_parity(ys[0].cpu().numpy(), refs[1], "code 3 decode group")
    finally:
        sw.close()


# ------------------------------------------------------------ token sweeps
def _check_sweep(fmt, shapes, seed, qa=128, f16_scale=False):
    t = torch()
    log(f"sweep fmt={fmt} qa={qa} f16_scale={f16_scale}: staging {len(shapes)} products")
    wl = SweepWorkload(fmt, shapes, seed, qa, f16_scale)
    try:
        wl.run()
        t.cuda.synchronize()
        y = wl.y.cpu().numpy()
        q_gpu, d_gpu = wl.q.cpu().numpy(), wl.d.cpu().numpy()
        q_ref, d_ref, _ = oracle.quantize_q8(wl.x, wl.qa, f16_scale)
        assert np.array_equal(q_gpu, q_ref) and same_bits(d_gpu, d_ref)
        bad = 0
        for i, (name, rows, cols) in enumerate(shapes):
            k0 = wl.koff[i]
            y_ref = oracle.matvec(fmt, wl.canon[i], rows, cols, q_ref[k0:k0 + cols],
                                  d_ref[k0 // wl.qa:(k0 + cols) // wl.qa], wl.qa, threads=THREADS)[0]
            yi = y[wl.yoff[i]:wl.yoff[i + 1]]
            nbad = int(np.count_nonzero(yi.view(np.uint32) != y_ref.view(np.uint32)))
            if nbad:
                log(f"  {name}: {nbad} of {rows} rows differ")
            bad += nbad
        log(f"sweep fmt={fmt}: {wl.rows_total} outputs checked, {bad} differ")
        assert bad == 0
        # the sweep and the single-product call agree bit for bit, and repeat runs are identical
        for i in sorted({0, min(6, len(shapes) - 1), len(shapes) - 1}):
            a = wl.entries[i][1]
            yi = t.empty(shapes[i][1], dtype=t.float32, device="cuda")
            import ternary_quantized_gemv_amd as bq
            (bq.bq_q1_0_matvec if fmt == Q1 else bq.bq_q2_0_matvec)(wl.weights[i], a, yi)
            t.cuda.synchronize()
            assert same_bits(yi.cpu().numpy(), y[wl.yoff[i]:wl.yoff[i + 1]])
        wl.run()
        t.cuda.synchronize()
        assert same_bits(wl.y.cpu().numpy(), y)
    finally:
        wl.close()


def test_sweep_q1_0_decode_token():
    _check_sweep(Q1, synth.decode_sweep_shapes(), seed=61)


def test_sweep_q2_0_decode_token():
    _check_sweep(Q2, synth.decode_sweep_shapes(), seed=62)


def test_sweep_ragged_mix():
    shapes = [("a", 1, 128), ("b", 100, 33 * 128), ("c", 65, 4096), ("d", 700, 12288), ("e", 64, 256)]
    _check_sweep(Q1, shapes, seed=63)


@pytest.mark.parametrize("fmt,qa,f16", [(Q1, 128, False), (Q1, 32, False), (Q2, 128, False), (Q2, 32, False),
                                         (Q1, 32, True), (Q2, 32, True)])
def test_sweep_paired_walk(fmt, qa, f16):
    """Work items of two tiles per wavefront over several chunks
    (gpu_util.paired_walk_shapes), every output against the oracle; also
    with the q8_0 activation flavour (qa 32, f16-valued scales)."""
    _check_sweep(fmt, paired_walk_shapes(fmt), seed=65 + fmt + int(f16), qa=qa, f16_scale=f16)


def test_sweep_ragged_mix_q2():
    """Q2_0 rows of one full 32-block chunk over 18 and 79 tiles (the
    single-chunk walk, several tiles per wavefront), a full chunk and a
    partial one, three full chunks and a partial one, and a row shorter than
    a chunk."""
    shapes = [("a", 1100, 2048), ("b", 700, 33 * 64), ("c", 1000, 100 * 64), ("d", 64, 64), ("e", 5000, 2048)]
    _check_sweep(Q2, shapes, seed=64, qa=64)


def test_gpu_errors_are_reported():
    import ternary_quantized_gemv_amd as bq
    t = torch()
    x = t.zeros(256, device="cuda")
    with pytest.raises(bq.BQError) as e:
        bq.bq_quantize_act_q8(x, 48, t.zeros(256, dtype=t.int8, device="cuda"), t.zeros(8, device="cuda"))
    assert e.value.code == bq.BQ_EARG and "bq_quantize_act_q8" in str(e.value)


def test_binding_refuses_short_or_wrong_tensors():
    """The binding checks every tensor it turns into a pointer (device, dtype,
    contiguity, enough elements) and raises BQError before any launch, so a
    short output cannot become an out-of-bounds write on the GPU."""
    import ternary_quantized_gemv_amd as bq
    t = torch()
    rows, cols = 256, 4096
    w = bq.Weights.upload(Q1, synth.blocks(Q1, rows, cols, 3), rows, cols)
    q = t.zeros(cols, dtype=t.int8, device="cuda")
    d = t.ones(cols // 128, dtype=t.float32, device="cuda")
    a = bq.Act(q, d, cols, 128, 1)
    x = t.zeros(cols, dtype=t.float32, device="cuda")
    sentinel = t.full((rows + 64,), 7.0, dtype=t.float32, device="cuda")
    bad_calls = [
        ("short y", lambda: bq.bq_q1_0_matvec(w, a, sentinel[:rows - 1])),
        ("f64 y", lambda: bq.bq_q1_0_matvec(w, a, t.zeros(rows, dtype=t.float64, device="cuda"))),
        ("host y", lambda: bq.bq_q1_0_matvec(w, a, t.zeros(rows))),
        ("strided y", lambda: bq.bq_q1_0_matvec(w, a, sentinel[::2])),
        ("short q", lambda: bq.Act(q[:cols - 16], d, cols, 128, 1)),
        ("f32 q", lambda: bq.Act(x, d, cols, 128, 1)),
        ("short d", lambda: bq.Act(q, d[:-1], cols, 128, 1)),
        ("two columns of one", lambda: bq.Act(q, d, cols, 128, 2)),
        ("quantizer short q", lambda: bq.bq_quantize_act_q8(x, 128, q[:100], d)),
        ("quantizer short d", lambda: bq.bq_quantize_act_q8(x, 128, q, d[:3])),
        ("quantizer int x", lambda: bq.bq_quantize_act_q8(q, 128, q, d)),
        ("short weights", lambda: bq.Weights(Q1, rows, cols, w.bits[:-16], w.scales)),
        ("group short y", lambda: bq.bq_group_matvec([w], x, 128, [sentinel[:10]])),
        ("sweep short y", lambda: bq.bq_sweep_create([(w, a, sentinel[:rows - 1])])),
        ("sweep_x short x", lambda: bq.bq_sweep_create_x([(w, x[:cols - 4], sentinel[:rows])], 128)),
    ]
    for what, call in bad_calls:
        with pytest.raises(bq.BQError):
            call()
        log(f"refused: {what}")
    t.cuda.synchronize()
    assert bool((sentinel == 7.0).all()), "a refused call wrote to the output"
