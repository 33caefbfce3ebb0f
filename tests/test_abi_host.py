"""Host-side checks of libbq that need no GPU: the library loads, exports every
symbol the header declares, packs and unpacks losslessly, lays blocks out as
documented, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
import ternary_quantized_gemv_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "bq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = header_functions()
    assert set(names) == set(bq.EXPORTS), names
    lib = ctypes.CDLL(bq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    assert bq.bq_abi_version() == bq.BQ_ABI_VERSION == 8


@pytest.mark.parametrize("fmt", [bq.BQ_Q1_0, bq.BQ_Q2_0])
@pytest.mark.parametrize("rows,nb", [(1, 1), (63, 3), (64, 8), (65, 9), (200, 33)])
def test_pack_roundtrip(fmt, rows, nb):
    cols = nb * bq.BLOCK_LEN[fmt]
    w = synth.blocks(fmt, rows, cols, 3, rows, nb)
    bits, scales = bq.bq_pack(fmt, w, rows, cols)
    nbits, nsc = bq.bq_packed_bytes(fmt, rows, cols)
    tiles = -(-rows // 64)
    gaps = 7 * ((tiles - 1) // 8) if fmt == bq.BQ_Q2_0 else 0  # Q2_0: 7 blocks after every eight tiles
    assert bits.nbytes == nbits == (tiles * nb + gaps) * 64 * 16
    assert scales.nbytes == nsc == tiles * 64 * (-(-nb // 8)) * 16
    assert np.array_equal(bq.bq_unpack(fmt, bits, scales, rows, cols), w)


def test_pack_layout():
    """Payload word j of (row r, block b) sits at [tile][b][lane][j], rotated
    left by 2; the scale at [tile][b/8][lane][b%8]; padding is zero."""
    rows, nb = 70, 10
    w = synth.q1_0_blocks(rows, nb * 128, 4)
    bits, scales = bq.bq_pack(1, w, rows, nb * 128)
    words = bits.view("<u4").reshape(2, nb, 64, 4)
    sc = scales.reshape(2, 2, 64, 8)
    for r in (0, 5, 63, 64, 69):
        t, lane = divmod(r, 64)
        for b in (0, 7, 8, 9):
            canon = w[r, b, 2:].copy().view("<u4")
            rot = ((canon.astype(np.uint64) << 2) | (canon.astype(np.uint64) >> 30)) & 0xFFFFFFFF
            assert np.array_equal(words[t, b, lane], rot.astype(np.uint32))
            assert int(sc[t, b // 8, lane, b % 8]) == int(w[r, b, 0]) | (int(w[r, b, 1]) << 8)
    assert not words[1, :, 6:].any() and not sc[1, :, 6:].any()  # padded rows
    assert not sc[:, 1, :, 2:].any()  # padded blocks 10..15


@pytest.mark.parametrize("fmt", [bq.BQ_Q1_0, bq.BQ_Q2_0])
def test_pack_layout_tile_groups(fmt):
    """Tile t's block b starts at block t * nb + b of the payload plane, plus,
    for Q2_0, a gap of 7 zero blocks after every eight tiles (t * nb + 7 *
    (t // 8) + b); blocks stay in row order.  18 tiles (three groups), rows
    of two full 32-block chunks and a partial one."""
    rows, nb = 64 * 17 + 5, 70
    cols = nb * bq.BLOCK_LEN[fmt]
    w = synth.blocks(fmt, rows, cols, 5)
    bits, scales = bq.bq_pack(fmt, w, rows, cols)
    gap = 7 if fmt == bq.BQ_Q2_0 else 0
    blocks = bits.view("<u4").reshape(-1, 64, 4)
    assert len(blocks) == 18 * nb + 2 * gap
    for r in (0, 63, 64 * 8, 64 * 8 + 7, 64 * 16 + 3, rows - 1):
        t, lane = divmod(r, 64)
        for b in (0, 5, 24, 31, 32, 40, 63, 64, 69):
            canon = w[r, b, 2:].copy().view("<u4").astype(np.uint64)
            expect = (((canon << 2) | (canon >> 30)) & 0xFFFFFFFF).astype(np.uint32)
            assert np.array_equal(blocks[t * nb + gap * (t // 8) + b, lane], expect), (r, b)
    for g in (1, 2):  # the gaps are zero
        assert not blocks[g * 8 * nb + (g - 1) * gap:g * 8 * nb + g * gap].any()
    assert np.array_equal(bq.bq_unpack(fmt, bits, scales, rows, cols), w)


@pytest.mark.parametrize("call,args,code", [
    ("bq_packed_bytes", (3, 4, 128), bq.BQ_EARG),
    ("bq_packed_bytes", (1, 0, 128), bq.BQ_EARG),
    ("bq_packed_bytes", (1, 4, 100), bq.BQ_EARG),
    ("bq_packed_bytes", (2, 4, 96), bq.BQ_EARG),
])
def test_host_argument_errors(call, args, code):
    with pytest.raises(bq.BQError) as e:
        getattr(bq, call)(*args)
    assert e.value.code == code and call in str(e.value)


def _c(fn, *args):
    return fn(*args)


def test_gpu_entry_points_validate_before_launch():
    """Bad arguments are refused on the host, so these calls touch no GPU."""
    lib = bq.lib
    x = ctypes.c_void_p(0x1000)
    assert lib.bq_quantize_act_q8(x, 256, 33, x, x, None) == bq.BQ_EARG
    assert "qa" in bq.bq_last_error()
    assert lib.bq_quantize_act_q8(x, 100, 32, x, x, None) == bq.BQ_EARG
    assert lib.bq_quantize_act_q8(None, 256, 32, x, x, None) == bq.BQ_EARG
    assert lib.bq_quantize_act_q8(ctypes.c_void_p(0x1004), 256, 32, x, x, None) == bq.BQ_EALIGN
    assert lib.bq_quantize_act_q8(x, 0, 32, x, x, None) == bq.BQ_OK  # empty input: nothing to do
    assert lib.bq_quantize_act_q8_f16(x, 256, 33, x, x, None) == bq.BQ_EARG
    assert "bq_quantize_act_q8_f16" in bq.bq_last_error() and "qa" in bq.bq_last_error()
    assert lib.bq_quantize_act_q8_f16(x, 100, 32, x, x, None) == bq.BQ_EARG
    assert lib.bq_quantize_act_q8_f16(x, 256, 32, None, x, None) == bq.BQ_EARG
    assert lib.bq_quantize_act_q8_f16(ctypes.c_void_p(0x1008), 256, 32, x, x, None) == bq.BQ_EALIGN
    assert lib.bq_quantize_act_q8_f16(x, 0, 32, x, x, None) == bq.BQ_OK

    w = bq.bq_weights(1, 0, 64, 256, 0x1000, 0x2000)
    a = bq.bq_act(0x3000, 0x4000, 256, 128, 1, 256, 2)
    ok = lambda: (ctypes.byref(w), ctypes.byref(a))
    assert lib.bq_q2_0_matvec(*ok(), 0x5000, None) == bq.BQ_EARG  # Q1_0 weights to the Q2_0 call
    assert "format" in bq.bq_last_error()
    assert lib.bq_q1_0_matvec(None, ctypes.byref(a), 0x5000, None) == bq.BQ_EARG
    assert lib.bq_q1_0_matvec(*ok(), None, None) == bq.BQ_EARG
    for field, val, code in [("cols", 200, bq.BQ_EARG), ("rows", 0, bq.BQ_EARG), ("bits", 0x1008, bq.BQ_EALIGN),
                             ("reserved", 1, bq.BQ_EARG)]:
        old = getattr(w, field)
        setattr(w, field, val)
        assert lib.bq_q1_0_matvec(*ok(), 0x5000, None) == code, field
        setattr(w, field, old)
    for field, val, code in [("n", 128, bq.BQ_EARG), ("qa", 16, bq.BQ_EARG), ("ncols", 0, bq.BQ_EARG),
                             ("ncols", 17, bq.BQ_EARG), ("q", 0x3004, bq.BQ_EALIGN), ("d", 0x4002, bq.BQ_EALIGN)]:
        old = getattr(a, field)
        setattr(a, field, val)
        assert lib.bq_q1_0_matvec(*ok(), 0x5000, None) == code, field
        setattr(a, field, old)
    assert lib.bq_q1_0_matvec(*ok(), 0x5002, None) == bq.BQ_EALIGN

    plan = ctypes.c_void_p()
    assert lib.bq_sweep_create(None, 0, ctypes.byref(plan)) == bq.BQ_EARG and not plan.value
    arr = (bq.bq_gemv * 2)()
    arr[0].w, arr[0].a, arr[0].y = w, a, 0x5000
    arr[1].w, arr[1].a, arr[1].y = w, a, 0x6000
    arr[1].a.qa = 32
    assert lib.bq_sweep_create(arr, 2, ctypes.byref(plan)) == bq.BQ_EARG
    assert "entry 1" in bq.bq_last_error()
    arr[1].a.qa = 128
    arr[1].a.ncols = 2
    assert lib.bq_sweep_create(arr, 2, ctypes.byref(plan)) == bq.BQ_EARG
    assert lib.bq_token_sweep(None, None) == bq.BQ_EARG
    lib.bq_sweep_destroy(None)


def test_group_validates_before_launch():
    """bq_group_matvec refuses bad groups on the host (no GPU is touched)."""
    lib = bq.lib
    W = bq.bq_weights * 5
    P = ctypes.c_void_p * 5
    w = W(*[bq.bq_weights(1, 0, 64, 256, 0x1000 * (i + 1), 0x9000) for i in range(5)])
    y = P(*[0x20000 + 0x100 * i for i in range(5)])
    x = ctypes.c_void_p(0x40000)
    assert lib.bq_group_matvec(w, 0, x, 128, y, None) == bq.BQ_EARG
    assert lib.bq_group_matvec(w, 5, x, 128, y, None) == bq.BQ_EARG and "count" in bq.bq_last_error()
    assert lib.bq_group_matvec(None, 1, x, 128, y, None) == bq.BQ_EARG
    assert lib.bq_group_matvec(w, 1, None, 128, y, None) == bq.BQ_EARG
    assert lib.bq_group_matvec(w, 1, ctypes.c_void_p(0x40004), 128, y, None) == bq.BQ_EALIGN
    assert lib.bq_group_matvec(w, 1, x, 96, y, None) == bq.BQ_EARG and "qa" in bq.bq_last_error()
    w[1].fmt = 2
    assert lib.bq_group_matvec(w, 2, x, 128, y, None) == bq.BQ_EARG and "product 1" in bq.bq_last_error()
    w[1].fmt, w[2].cols = 1, 384
    assert lib.bq_group_matvec(w, 3, x, 128, y, None) == bq.BQ_EARG and "cols" in bq.bq_last_error()
    w[2].cols = 256
    y[3] = 0
    assert lib.bq_group_matvec(w, 4, x, 128, y, None) == bq.BQ_EARG and "product 3" in bq.bq_last_error()
    y[3] = 0x20002
    assert lib.bq_group_matvec(w, 4, x, 128, y, None) == bq.BQ_EALIGN
    w[0].fmt = 3
    assert lib.bq_group_matvec(w, 1, x, 128, y, None) == bq.BQ_EARG


def test_sweep_create_x_validates_before_launch():
    """bq_sweep_create_x refuses bad entries on the host (no GPU is touched)."""
    lib = bq.lib
    plan = ctypes.c_void_p()
    arr = (bq.bq_gemv_x * 2)()
    for i in range(2):
        arr[i].w = bq.bq_weights(1, 0, 64, 256, 0x1000 * (i + 1), 0x9000)
        arr[i].x, arr[i].y = 0x40000 + 0x1000 * i, 0x60000 + 0x1000 * i
    assert lib.bq_sweep_create_x(arr, 2, 128, None) == bq.BQ_EARG
    assert lib.bq_sweep_create_x(None, 1, 128, ctypes.byref(plan)) == bq.BQ_EARG and not plan.value
    assert lib.bq_sweep_create_x(arr, 0, 128, ctypes.byref(plan)) == bq.BQ_EARG
    assert lib.bq_sweep_create_x(arr, 2, 96, ctypes.byref(plan)) == bq.BQ_EARG and "qa" in bq.bq_last_error()
    arr[1].w.fmt = 2
    assert lib.bq_sweep_create_x(arr, 2, 128, ctypes.byref(plan)) == bq.BQ_EARG and "entry 1" in bq.bq_last_error()
    arr[0].w.fmt, arr[1].w.cols = 2, 192  # Q2_0 rows of three 64-weight blocks: not a multiple of qa 128
    assert lib.bq_sweep_create_x(arr, 2, 128, ctypes.byref(plan)) == bq.BQ_EARG and "qa" in bq.bq_last_error()
    arr[0].w.fmt = arr[1].w.fmt = 1
    arr[1].w.cols = 256
    arr[1].x = 0
    assert lib.bq_sweep_create_x(arr, 2, 128, ctypes.byref(plan)) == bq.BQ_EARG
    arr[1].x = 0x41004
    assert lib.bq_sweep_create_x(arr, 2, 128, ctypes.byref(plan)) == bq.BQ_EALIGN
    arr[1].x, arr[1].y = 0x41000, 0x61002
    assert lib.bq_sweep_create_x(arr, 2, 128, ctypes.byref(plan)) == bq.BQ_EALIGN
    assert "bq_sweep_create_x" in bq.bq_last_error() and not plan.value


def test_read_floor_validates_before_launch():
    """bq_read_floor refuses bad buffers on the host (no GPU is touched)."""
    lib = bq.lib
    p, sink = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    assert lib.bq_read_floor(None, 1024, sink, None) == bq.BQ_EARG
    assert lib.bq_read_floor(p, 1024, None, None) == bq.BQ_EARG
    assert lib.bq_read_floor(p, 0, sink, None) == bq.BQ_EARG and "bytes" in bq.bq_last_error()
    assert lib.bq_read_floor(p, 1000, sink, None) == bq.BQ_EARG
    assert lib.bq_read_floor(ctypes.c_void_p(0x10008), 1024, sink, None) == bq.BQ_EALIGN
    assert lib.bq_read_floor(p, 1024, ctypes.c_void_p(0x20002), None) == bq.BQ_EALIGN
    assert "bq_read_floor" in bq.bq_last_error()


def test_host_tensors_are_refused():
    torch = pytest.importorskip("torch")
    x = torch.zeros(256)
    with pytest.raises(bq.BQError):
        bq.bq_quantize_act_q8(x, 128, torch.zeros(256, dtype=torch.int8), torch.zeros(2))


def test_size_limits():
    """Shapes the kernels cannot address are refused before anything runs:
    rows and cols below 2^31, and a 64-row tile's payload (nb x 1 KiB) within
    the 2^31 - 16 bytes one buffer resource spans."""
    lim = {bq.BQ_Q1_0: 2097151, bq.BQ_Q2_0: 2097151}  # blocks per row
    for fmt, qk in ((bq.BQ_Q1_0, 128), (bq.BQ_Q2_0, 64)):
        b, s = bq.bq_packed_bytes(fmt, 64, lim[fmt] * qk)
        assert b == lim[fmt] * 1024 <= 0x7FFFFFF0
        with pytest.raises(bq.BQError) as e:
            bq.bq_packed_bytes(fmt, 64, (lim[fmt] + 1) * qk)
        assert e.value.code == bq.BQ_EARG and "payload" in str(e.value)
    bq.bq_packed_bytes(bq.BQ_Q1_0, (1 << 31) - 1, 128)
    for rows, cols in (((1 << 31), 128), (64, 1 << 31)):
        with pytest.raises(bq.BQError) as e:
            bq.bq_packed_bytes(bq.BQ_Q1_0, rows, cols)
        assert e.value.code == bq.BQ_EARG and "2^31" in str(e.value)

    lib = bq.lib
    big = (lim[bq.BQ_Q1_0] + 1) * 128
    w = bq.bq_weights(1, 0, 64, big, 0x1000, 0x2000)
    a = bq.bq_act(0x3000, 0x4000, big, 128, 1, big, big // 128)
    assert lib.bq_q1_0_matvec(ctypes.byref(w), ctypes.byref(a), 0x5000, None) == bq.BQ_EARG
    assert "payload" in bq.bq_last_error()
    w.rows = 1 << 31
    w.cols = 256
    assert lib.bq_q1_0_matvec(ctypes.byref(w), ctypes.byref(a), 0x5000, None) == bq.BQ_EARG
    w.rows, w.cols = 64, big
    y = (ctypes.c_void_p * 1)(0x5000)
    assert lib.bq_group_matvec(ctypes.byref(w), 1, ctypes.c_void_p(0x6000), 128, y, None) == bq.BQ_EARG
    assert "payload" in bq.bq_last_error()
    arr = (bq.bq_gemv * 1)()
    arr[0].w, arr[0].a, arr[0].y = w, a, 0x5000
    plan = ctypes.c_void_p()
    assert lib.bq_sweep_create(arr, 1, ctypes.byref(plan)) == bq.BQ_EARG and not plan.value
    assert "payload" in bq.bq_last_error()


def test_noalloc_sweep_validates_before_launch():
    """The no-allocation sweep refuses bad lists on the host, before it looks
    up its scratch or touches the GPU."""
    lib = bq.lib
    w = bq.bq_weights(1, 0, 64, 256, 0x1000, 0x2000)
    a = bq.bq_act(0x3000, 0x4000, 256, 128, 1, 256, 2)
    assert lib.bq_token_sweep_noalloc(None, 1, None) == bq.BQ_EARG
    arr = (bq.bq_gemv * 2)()
    assert lib.bq_token_sweep_noalloc(arr, 0, None) == bq.BQ_EARG
    assert lib.bq_token_sweep_noalloc(arr, 1025, None) == bq.BQ_EARG and "1024" in bq.bq_last_error()
    arr[0].w, arr[0].a, arr[0].y = w, a, 0x5000
    arr[1].w, arr[1].a, arr[1].y = w, a, 0x6000
    arr[1].a.qa = 32
    assert lib.bq_token_sweep_noalloc(arr, 2, None) == bq.BQ_EARG and "entry 1" in bq.bq_last_error()
    arr[1].a.qa = 128
    arr[1].y = 0x6002
    assert lib.bq_token_sweep_noalloc(arr, 2, None) == bq.BQ_EALIGN
    # more work items than the scratch holds: 400 products of 151,936 rows (2,374 tiles each)
    big = (bq.bq_gemv * 400)()
    for i in range(400):
        big[i].w = bq.bq_weights(1, 0, 151936, 4096, 0x1000, 0x2000)
        big[i].a = bq.bq_act(0x3000, 0x4000, 4096, 128, 1, 4096, 32)
        big[i].y = 0x5000
    assert lib.bq_token_sweep_noalloc(big, 400, None) == bq.BQ_EARG and "16384" in bq.bq_last_error()


def test_batch_path_knob():
    """bq_set_batch_path returns the previous setting and refuses unknown paths."""
    prev = bq.bq_set_batch_path(bq.BQ_BATCH_TABLES)
    try:
        assert bq.bq_set_batch_path(bq.BQ_BATCH_MFMA) == bq.BQ_BATCH_TABLES
        with pytest.raises(bq.BQError, match="path 5 unknown"):
            bq.bq_set_batch_path(5)
        assert bq.bq_set_batch_path(bq.BQ_BATCH_AUTO) == bq.BQ_BATCH_MFMA
    finally:
        bq.bq_set_batch_path(prev)
