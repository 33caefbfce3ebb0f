"""Python binding of libbq (include/bq.h): 1-bit (Q1_0) and ternary (Q2_0)
quantized matrix-vector products on MI355X.

The functions keep the C names and only marshal arguments: torch tensors on a
ROCm device become device pointers, numpy arrays become host pointers, and a
nonzero return code becomes a ``BQError`` carrying ``bq_last_error()``.  Every
step of the computation runs in the HIP kernels of ``libbq.so``; importing
this package fails if the library has not been built
(``python ternary_quantized_gemv_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbq.so")

BQ_Q1_0 = 1
BQ_Q2_0 = 2
BQ_OK, BQ_EARG, BQ_EALIGN, BQ_EHIP, BQ_ENOMEM = 0, 1, 2, 3, 4
BQ_FLOOR_SINK_WORDS = 8192
BQ_ABI_VERSION = 8  # include/bq.h
BQ_BATCH_AUTO, BQ_BATCH_TABLES, BQ_BATCH_MFMA = 0, 1, 2
BLOCK_LEN = {BQ_Q1_0: 128, BQ_Q2_0: 64}
BLOCK_BYTES = 18

EXPORTS = (
    "bq_abi_version", "bq_last_error", "bq_packed_bytes", "bq_pack", "bq_unpack",
    "bq_quantize_act_q8", "bq_quantize_act_q8_f16", "bq_q1_0_matvec", "bq_q2_0_matvec", "bq_group_matvec",
    "bq_sweep_create", "bq_sweep_create_x", "bq_token_sweep", "bq_sweep_destroy", "bq_read_floor",
    "bq_token_sweep_noalloc", "bq_set_batch_path",
)


class BQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[bq error {code}] {msg}")
        self.code = code


class bq_weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("bits", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class bq_act(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("qa", ctypes.c_int32), ("ncols", ctypes.c_int32), ("ld_q", ctypes.c_int64),
                ("ld_d", ctypes.c_int64)]


class bq_gemv(ctypes.Structure):
    _fields_ = [("w", bq_weights), ("a", bq_act), ("y", ctypes.c_void_p)]


class bq_gemv_x(ctypes.Structure):
    _fields_ = [("w", bq_weights), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


def _hip_runtimes() -> set:
    """Paths of every HIP runtime library mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python ternary_quantized_gemv_amd/build.py`")
    # torch ships its own HIP runtime (same soname).  Loading torch first lets
    # libbq bind to that already-loaded copy, so device pointers and streams
    # from torch are valid in libbq's calls.  Two runtimes in one process would
    # each see the device separately, so that case is refused below.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(runtimes)}); import torch before anything "
                          "that links libamdhip64 so that libbq shares torch's runtime")
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.bq_abi_version.restype = ctypes.c_int
    lib.bq_abi_version.argtypes = []
    if lib.bq_abi_version() != BQ_ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.bq_abi_version()}, this binding {BQ_ABI_VERSION}: "
                          "rebuild it with `python ternary_quantized_gemv_amd/build.py`")
    lib.bq_last_error.restype = ctypes.c_char_p
    lib.bq_last_error.argtypes = []
    lib.bq_packed_bytes.restype = ctypes.c_int
    lib.bq_packed_bytes.argtypes = [i32, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.bq_pack.restype = ctypes.c_int
    lib.bq_pack.argtypes = [i32, vp, i64, i64, vp, vp]
    lib.bq_unpack.restype = ctypes.c_int
    lib.bq_unpack.argtypes = [i32, vp, vp, i64, i64, vp]
    lib.bq_quantize_act_q8.restype = ctypes.c_int
    lib.bq_quantize_act_q8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.bq_quantize_act_q8_f16.restype = ctypes.c_int
    lib.bq_quantize_act_q8_f16.argtypes = [vp, i64, i32, vp, vp, vp]
    for f in (lib.bq_q1_0_matvec, lib.bq_q2_0_matvec):
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(bq_weights), ctypes.POINTER(bq_act), vp, vp]
    lib.bq_sweep_create.restype = ctypes.c_int
    lib.bq_group_matvec.restype = ctypes.c_int
    lib.bq_group_matvec.argtypes = [ctypes.POINTER(bq_weights), i32, vp, i32, ctypes.POINTER(vp), vp]
    lib.bq_sweep_create.argtypes = [ctypes.POINTER(bq_gemv), i32, ctypes.POINTER(vp)]
    lib.bq_sweep_create_x.restype = ctypes.c_int
    lib.bq_sweep_create_x.argtypes = [ctypes.POINTER(bq_gemv_x), i32, i32, ctypes.POINTER(vp)]
    lib.bq_token_sweep.restype = ctypes.c_int
    lib.bq_token_sweep.argtypes = [vp, vp]
    lib.bq_sweep_destroy.restype = None
    lib.bq_sweep_destroy.argtypes = [vp]
    lib.bq_token_sweep_noalloc.restype = ctypes.c_int
    lib.bq_token_sweep_noalloc.argtypes = [ctypes.POINTER(bq_gemv), i32, vp]
    lib.bq_read_floor.restype = ctypes.c_int
    lib.bq_read_floor.argtypes = [vp, i64, vp, vp]
    lib.bq_set_batch_path.restype = ctypes.c_int
    lib.bq_set_batch_path.argtypes = [ctypes.c_int]
    return lib


lib = _load()


def _check(rc: int):
    if rc != BQ_OK:
        raise BQError(rc, lib.bq_last_error().decode())


def _dev(t, what: str) -> int:
    """Device pointer of a torch tensor on a GPU (refuses host tensors)."""
    if t is None:
        return 0
    if not getattr(t, "is_cuda", False):
        raise BQError(BQ_EARG, f"{what} must be a tensor on a ROCm device")
    return t.data_ptr()


def _need(t, what: str, dtype, numel: int, fn: str) -> None:
    """Refuses (BQError, before anything is launched) a tensor that is not on
    a ROCm device, not of dtype, not contiguous, or holds fewer than numel
    elements: the library takes bare pointers and would read or write past
    its end."""
    if t is None or not getattr(t, "is_cuda", False):
        raise BQError(BQ_EARG, f"{fn}: {what} must be a tensor on a ROCm device")
    if t.dtype != dtype:
        raise BQError(BQ_EARG, f"{fn}: {what} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise BQError(BQ_EARG, f"{fn}: {what} must be contiguous")
    if t.numel() < numel:
        raise BQError(BQ_EARG, f"{fn}: {what} holds {t.numel()} elements, needs {numel}")


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ----------------------------------------------------------------- host calls
def bq_abi_version() -> int:
    return lib.bq_abi_version()


def bq_last_error() -> str:
    return lib.bq_last_error().decode()


def bq_packed_bytes(fmt: int, rows: int, cols: int) -> tuple[int, int]:
    b, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.bq_packed_bytes(fmt, rows, cols, ctypes.byref(b), ctypes.byref(s)))
    return b.value, s.value


def bq_pack(fmt: int, canon: np.ndarray, rows: int, cols: int) -> tuple[np.ndarray, np.ndarray]:
    """Canonical blocks (uint8, rows x cols/QK x 18) -> (payload plane uint8, scale plane uint16)."""
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    if canon.size != rows * (cols // BLOCK_LEN.get(fmt, 1)) * BLOCK_BYTES:
        raise BQError(BQ_EARG, "bq_pack: canonical array has the wrong size")
    nb, ns = bq_packed_bytes(fmt, rows, cols)
    bits = np.empty(nb, dtype=np.uint8)
    scales = np.empty(ns // 2, dtype=np.uint16)
    _check(lib.bq_pack(fmt, canon.ctypes.data, rows, cols, bits.ctypes.data, scales.ctypes.data))
    return bits, scales


def bq_unpack(fmt: int, bits: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    nb, ns = bq_packed_bytes(fmt, rows, cols)
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if bits.nbytes != nb or scales.nbytes != ns:
        raise BQError(BQ_EARG, "bq_unpack: plane sizes do not match")
    out = np.empty((rows, cols // BLOCK_LEN[fmt], BLOCK_BYTES), dtype=np.uint8)
    _check(lib.bq_unpack(fmt, bits.ctypes.data, scales.ctypes.data, rows, cols, out.ctypes.data))
    return out


# ------------------------------------------------------------------ GPU calls
def _quantize_args(fn: str, x, qa: int, q, d) -> int:
    import torch
    _need(x, "x", torch.float32, 0, fn)
    n = x.numel()
    _need(q, "q", torch.int8, n, fn)
    _need(d, "d", torch.float32, n // qa if qa > 0 else 0, fn)
    return n


def bq_quantize_act_q8(x, qa: int, q, d, stream=None) -> None:
    """x: float32 device tensor (n); q: int8 device tensor (n); d: float32 device tensor (n/qa)."""
    n = _quantize_args("bq_quantize_act_q8", x, qa, q, d)
    _check(lib.bq_quantize_act_q8(_dev(x, "x"), n, qa, _dev(q, "q"), _dev(d, "d"), _stream(stream)))


def bq_quantize_act_q8_f16(x, qa: int, q, d, stream=None) -> None:
    """As bq_quantize_act_q8, with the scales narrowed to f16 values."""
    n = _quantize_args("bq_quantize_act_q8_f16", x, qa, q, d)
    _check(lib.bq_quantize_act_q8_f16(_dev(x, "x"), n, qa, _dev(q, "q"), _dev(d, "d"), _stream(stream)))


def bq_read_floor(buf, sink, stream=None) -> None:
    """Streaming read of every byte of the device tensor buf (the read
    bandwidth floor); sink is a device tensor of BQ_FLOOR_SINK_WORDS int32
    whose XOR equals the XOR of buf's 32-bit words."""
    if sink.numel() * sink.element_size() < 4 * BQ_FLOOR_SINK_WORDS:
        raise ValueError(f"bq_read_floor: sink holds fewer than {BQ_FLOOR_SINK_WORDS} words")
    _check(lib.bq_read_floor(_dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"),
                             _stream(stream)))


class Weights:
    """A packed matrix resident on the GPU (the two planes of bq_pack)."""

    def __init__(self, fmt: int, rows: int, cols: int, bits, scales):
        import torch
        nb, ns = bq_packed_bytes(fmt, rows, cols)
        _need(bits, "weights.bits", torch.uint8, nb, "Weights")
        _need(scales, "weights.scales", torch.int16, ns // 2, "Weights")
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.bits, self.scales = bits, scales

    @classmethod
    def upload(cls, fmt: int, canon: np.ndarray, rows: int, cols: int, device="cuda"):
        import torch
        bits, scales = bq_pack(fmt, canon, rows, cols)
        return cls(fmt, rows, cols, torch.from_numpy(bits).to(device),
                   torch.from_numpy(scales.view(np.int16)).to(device))

    def c(self) -> bq_weights:
        return bq_weights(self.fmt, 0, self.rows, self.cols, _dev(self.bits, "weights.bits"),
                          _dev(self.scales, "weights.scales"))


class Act:
    """ncols quantized activation columns on the GPU: q int8 [ncols, ld_q], d f32 [ncols, ld_d]."""

    def __init__(self, q, d, n: int, qa: int, ncols: int = 1):
        import torch
        for t, what, dt in ((q, "act.q", torch.int8), (d, "act.d", torch.float32)):
            if not getattr(t, "is_cuda", False) or t.dtype != dt:
                raise BQError(BQ_EARG, f"Act: {what} must be a {dt} tensor on a ROCm device")
            if t.dim() not in (1, 2) or t.stride(-1) != 1 or (t.dim() == 2 and t.shape[0] < ncols):
                raise BQError(BQ_EARG, f"Act: {what} must be 1-D, or 2-D [>= ncols, ...] with unit stride")
        self.q, self.d, self.n, self.qa, self.ncols = q, d, n, qa, ncols
        # the library reads column c at q + c ld_q (n values) and d + c ld_d (n / qa values)
        ld_q, ld_d = self._ld()
        for t, ld, need, what in ((q, ld_q, n, "act.q"), (d, ld_d, n // qa if qa > 0 else 0, "act.d")):
            short = t.shape[1] < need if t.dim() == 2 else t.numel() < (ncols - 1) * ld + need
            if short:
                raise BQError(BQ_EARG, f"Act: {what} holds fewer values than {ncols} column(s) of {need} need")

    def _ld(self):
        ld_q = self.q.stride(0) if self.q.dim() == 2 else self.n
        ld_d = self.d.stride(0) if self.d.dim() == 2 else (self.n // self.qa if self.qa > 0 else 0)
        return ld_q, ld_d

    def c(self) -> bq_act:
        ld_q, ld_d = self._ld()
        return bq_act(_dev(self.q, "act.q"), _dev(self.d, "act.d"), self.n, self.qa, self.ncols, ld_q, ld_d)


def _matvec(fn, w: Weights, a: Act, y, stream):
    import torch
    _need(y, "y", torch.float32, a.ncols * w.rows, fn.__name__)
    wc, ac = w.c(), a.c()
    _check(fn(ctypes.byref(wc), ctypes.byref(ac), _dev(y, "y"), _stream(stream)))


def bq_q1_0_matvec(w: Weights, a: Act, y, stream=None) -> None:
    _matvec(lib.bq_q1_0_matvec, w, a, y, stream)


def bq_q2_0_matvec(w: Weights, a: Act, y, stream=None) -> None:
    _matvec(lib.bq_q2_0_matvec, w, a, y, stream)


def bq_set_batch_path(path: int) -> int:
    """Kernels for 2..16 activation columns: BQ_BATCH_AUTO, BQ_BATCH_TABLES or
    BQ_BATCH_MFMA (process-wide); returns the previous setting."""
    prev = lib.bq_set_batch_path(int(path))
    if prev < 0:
        raise BQError(BQ_EARG, lib.bq_last_error().decode())
    return prev


class GroupCall:
    """The marshalled arguments of one bq_group_matvec call (weights, the f32
    activation x, qa, one output per product), kept so that the call can be
    issued repeatedly without rebuilding them."""

    def __init__(self, weights, x, qa: int, ys):
        n = len(weights)
        if len(ys) != n:
            raise BQError(BQ_EARG, "bq_group_matvec: one output per product")
        if n and x.numel() != weights[0].cols:
            raise BQError(BQ_EARG, "bq_group_matvec: x length differs from the weights' cols")
        import torch
        _need(x, "x", torch.float32, 0, "bq_group_matvec")
        for w, y in zip(weights, ys):
            _need(y, "y", torch.float32, w.rows, "bq_group_matvec")
        self.w = (bq_weights * n)(*[w.c() for w in weights])
        self.y = (ctypes.c_void_p * n)(*[_dev(y, "y") for y in ys])
        self.n, self.x, self.qa = n, _dev(x, "x"), qa
        self._keep = (list(weights), x, list(ys))

    def launch(self, stream=None) -> None:
        _check(lib.bq_group_matvec(self.w, self.n, self.x, self.qa, self.y, _stream(stream)))


def bq_group_matvec(weights, x, qa: int, ys, stream=None) -> None:
    """weights: [Weights] sharing format and cols; x: float32 device tensor
    (cols); ys: float32 device tensors, one per product (rows)."""
    GroupCall(weights, x, qa, ys).launch(stream)


class Sweep:
    """A bq_sweep plan; keeps the tensors it points at alive until destroyed."""

    def __init__(self, handle: int, keep):
        self.handle = handle
        self._keep = keep

    def destroy(self):
        if self.handle:
            lib.bq_sweep_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _gemv_list(entries, fn: str):
    import torch
    arr = (bq_gemv * len(entries))()
    for i, (w, a, y) in enumerate(entries):
        _need(y, f"entry {i} y", torch.float32, w.rows, fn)
        arr[i].w = w.c()
        arr[i].a = a.c()
        arr[i].y = _dev(y, "y")
    return arr


def bq_sweep_create(entries) -> Sweep:
    """entries: [(Weights, Act, y tensor)]."""
    arr = _gemv_list(entries, "bq_sweep_create")
    h = ctypes.c_void_p()
    _check(lib.bq_sweep_create(arr, len(entries), ctypes.byref(h)))
    return Sweep(h.value, list(entries))


def bq_sweep_create_x(entries, qa: int) -> Sweep:
    """entries: [(Weights, x f32 tensor of length cols, y tensor)]; the launch
    quantizes each x in blocks of qa."""
    import torch
    arr = (bq_gemv_x * len(entries))()
    for i, (w, x, y) in enumerate(entries):
        _need(x, f"entry {i} x", torch.float32, w.cols, "bq_sweep_create_x")
        _need(y, f"entry {i} y", torch.float32, w.rows, "bq_sweep_create_x")
        arr[i].w = w.c()
        arr[i].x = _dev(x, "x")
        arr[i].y = _dev(y, "y")
    h = ctypes.c_void_p()
    _check(lib.bq_sweep_create_x(arr, len(entries), qa, ctypes.byref(h)))
    return Sweep(h.value, list(entries))


def bq_token_sweep(plan: Sweep, stream=None) -> None:
    _check(lib.bq_token_sweep(plan.handle, _stream(stream)))


def bq_sweep_destroy(plan: Sweep) -> None:
    plan.destroy()


def bq_token_sweep_noalloc(entries, stream=None) -> None:
    """entries: [(Weights, Act, y tensor)], as bq_sweep_create; planned and
    launched in one call that allocates no memory (the library's fixed
    scratch holds the plan)."""
    arr = _gemv_list(entries, "bq_token_sweep_noalloc")
    _check(lib.bq_token_sweep_noalloc(arr, len(entries), _stream(stream)))
