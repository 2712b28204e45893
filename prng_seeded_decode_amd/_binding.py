"""ctypes binding of libseedlm.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; PyTorch is used only
for device memory (tensors) and streams.  Loading fails loudly when the built
library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libseedlm.so")

OK = 0
E_INVALID = -1
E_UNSUPPORTED = -2
E_NOMEM = -3
E_DEVICE = -4
E_SCRATCH_LIMIT = -5
NOALLOC_SCRATCH_BYTES = 64 << 20
F32 = 0
F16 = 1
MAX_BATCH = 16
VARIANT_AUTO = 0
VARIANT_LUT = 1
VARIANT_TABLE = 2
VARIANT_SIMPLE = 3
VARIANT_MFMA = 4
VARIANT_DIRECT = 5

EXPORTED = (
    "seedlm_pack_host",
    "seedlm_pack",
    "seedlm_gemv",
    "seedlm_gemv_variant",
    "seedlm_gemv_many",
    "seedlm_gemv_many_begin",
    "seedlm_gemv_many_end",
    "seedlm_gemv_many_noalloc",
    "seedlm_gemv_scratch_bytes",
    "seedlm_scratch_release",
    "seedlm_decode",
    "seedlm_destroy",
    "seedlm_info",
    "seedlm_export",
    "seedlm_status_string",
    "seedlm_bench_time_next_call",
    "seedlm_fp16_gemv",
    "seedlm_stream_read",
    "seedlm_gemm",
    "seedlm_gemm_scratch_bytes",
    "seedlm_gemm_decoded",
    "seedlm_gemm_decoded_bytes",
    "seedlm_encoder_create",
    "seedlm_encoder_destroy",
    "seedlm_encode",
)


class SeedLMError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


class _Info(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("C", ctypes.c_int32),
        ("P", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("blocks_per_row", ctypes.c_int64),
        ("stored_blocks_per_row", ctypes.c_int64),
        ("compressed_bytes", ctypes.c_int64),
        ("Q", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libseedlm.so (once).  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m prng_seeded_decode_amd.build`"
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.seedlm_pack_host.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, vp, ctypes.POINTER(sz)]
    L.seedlm_pack.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, ctypes.POINTER(vp)]
    L.seedlm_gemv.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    L.seedlm_gemv_variant.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    L.seedlm_gemv_many.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    L.seedlm_gemv_many_begin.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    L.seedlm_gemv_many_end.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    L.seedlm_gemv_many_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    L.seedlm_gemv_scratch_bytes.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.seedlm_scratch_release.argtypes = []
    L.seedlm_decode.argtypes = [vp, vp, vp]
    L.seedlm_destroy.argtypes = [vp]
    L.seedlm_info.argtypes = [vp, ctypes.POINTER(_Info)]
    L.seedlm_export.argtypes = [vp, vp, ctypes.POINTER(sz)]
    L.seedlm_status_string.argtypes = [i32]
    L.seedlm_status_string.restype = ctypes.c_char_p
    L.seedlm_bench_time_next_call.argtypes = [vp, vp]
    L.seedlm_fp16_gemv.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    L.seedlm_stream_read.argtypes = [vp, i64, vp, vp]
    L.seedlm_gemm.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    L.seedlm_gemm_scratch_bytes.argtypes = [vp, i64, ctypes.POINTER(sz)]
    L.seedlm_gemm_decoded.argtypes = [vp, vp, vp, i64, i32, i32, vp, ctypes.c_size_t, vp]
    L.seedlm_gemm_decoded_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    L.seedlm_encoder_create.argtypes = [i32, i32, i32, i32, ctypes.POINTER(vp)]
    L.seedlm_encoder_destroy.argtypes = [vp]
    L.seedlm_encode.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp]
    for name in EXPORTED:
        if name != "seedlm_status_string":
            getattr(L, name).restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().seedlm_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise SeedLMError(status, what)


def _records(seeds, coeffs, exps, rows, cols, C, P, K=16):
    nb = -(-cols // C)
    seeds = np.ascontiguousarray(seeds, dtype=np.uint16 if K <= 16 else np.uint32)
    coeffs = np.ascontiguousarray(coeffs, dtype=np.int8)
    exps = np.ascontiguousarray(exps, dtype=np.int8)
    if seeds.shape != (rows, nb) or coeffs.shape != (rows, nb, P) or exps.shape != (rows, nb):
        raise ValueError("record arrays must be seeds[rows][nb], coeffs[rows][nb][P], exps[rows][nb]")
    return seeds, coeffs, exps


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def seedlm_pack_host(seeds, coeffs, exps, rows, cols, C, P, K=16) -> bytes:
    """Packed layout written on the host (no GPU involved)."""
    seeds, coeffs, exps = _records(seeds, coeffs, exps, rows, cols, C, P, K)
    n = ctypes.c_size_t(0)
    _check(lib().seedlm_pack_host(_ptr(seeds), _ptr(coeffs), _ptr(exps), rows, cols, C, P, K,
                                  None, ctypes.byref(n)), "seedlm_pack_host")
    buf = ctypes.create_string_buffer(n.value)
    _check(lib().seedlm_pack_host(_ptr(seeds), _ptr(coeffs), _ptr(exps), rows, cols, C, P, K,
                                  ctypes.cast(buf, ctypes.c_void_p), ctypes.byref(n)),
           "seedlm_pack_host")
    return buf.raw[: n.value]


def pack_host_status(seeds, coeffs, exps, rows, cols, C, P, K=16) -> int:
    """Raw status of seedlm_pack_host on arbitrary arrays (for error-path tests)."""
    seeds = np.ascontiguousarray(seeds, dtype=np.uint16 if K <= 16 else np.uint32)
    coeffs = np.ascontiguousarray(coeffs, dtype=np.int8)
    exps = np.ascontiguousarray(exps, dtype=np.int8)
    n = ctypes.c_size_t(0)
    return lib().seedlm_pack_host(_ptr(seeds), _ptr(coeffs), _ptr(exps), rows, cols, C, P, K,
                                  None, ctypes.byref(n))


def _stream_ptr(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    raise ValueError(f"unsupported dtype {t.dtype}")


class SeedLMMatrix:
    """A packed matrix on the GPU (owns a libseedlm handle)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        info = _Info()
        _check(lib().seedlm_info(self._h, ctypes.byref(info)), "seedlm_info")
        self.rows = info.rows
        self.cols = info.cols
        self.C, self.P, self.K, self.Q = info.C, info.P, info.K, info.Q
        self.blocks_per_row = info.blocks_per_row
        self.stored_blocks_per_row = info.stored_blocks_per_row
        self.compressed_bytes = info.compressed_bytes

    @property
    def handle(self):
        if self._h is None or not self._h.value:
            raise ValueError("matrix has been destroyed")
        return self._h

    def destroy(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(lib().seedlm_destroy(self._h), "seedlm_destroy")
        self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def seedlm_pack(seeds, coeffs, exps, rows, cols, C, P, K=16) -> SeedLMMatrix:
    """Validate, pack and upload records; returns a SeedLMMatrix.  Seeds are
    uint16 for K = 16 and uint32 for K = 20."""
    seeds, coeffs, exps = _records(seeds, coeffs, exps, rows, cols, C, P, K)
    h = ctypes.c_void_p()
    _check(lib().seedlm_pack(_ptr(seeds), _ptr(coeffs), _ptr(exps), rows, cols, C, P, K,
                             ctypes.byref(h)), "seedlm_pack")
    return SeedLMMatrix(h.value)


def seedlm_gemv(m: SeedLMMatrix, x, y, batch=None, stream=None, variant=VARIANT_AUTO):
    """y[batch][rows] = W x[batch][cols] on the GPU (torch CUDA tensors)."""
    if batch is None:
        batch = 1 if x.dim() == 1 else x.shape[0]
    if x.numel() != batch * m.cols or y.numel() != batch * m.rows:
        raise ValueError("x must hold batch*cols and y batch*rows elements")
    if not (x.is_cuda and y.is_cuda and x.is_contiguous() and y.is_contiguous()):
        raise ValueError("x and y must be contiguous device tensors")
    _check(lib().seedlm_gemv_variant(m.handle, ctypes.c_void_p(x.data_ptr()),
                                     ctypes.c_void_p(y.data_ptr()), batch, _dtype_code(x),
                                     _dtype_code(y), variant, _stream_ptr(stream)),
           "seedlm_gemv")
    return y


def _many_args(mats, xs, ys, batch):
    n = len(mats)
    if not (len(xs) == n and len(ys) == n):
        raise ValueError("mats, xs and ys must have the same length")
    for m, x, y in zip(mats, xs, ys):
        if x.numel() != batch * m.cols or y.numel() != batch * m.rows:
            raise ValueError("x must hold batch*cols and y batch*rows elements")
        if not (x.is_cuda and y.is_cuda and x.is_contiguous() and y.is_contiguous()):
            raise ValueError("x and y must be contiguous device tensors")
        if x.dtype != xs[0].dtype or y.dtype != ys[0].dtype:
            raise ValueError("all x (and all y) must share one dtype")
    H = (ctypes.c_void_p * n)(*[m.handle.value for m in mats])
    X = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    Y = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    xdt = _dtype_code(xs[0]) if n else F16
    ydt = _dtype_code(ys[0]) if n else F16
    # the arrays ride along in the cast pointers' _objects, so they stay alive
    return (ctypes.cast(H, ctypes.c_void_p), ctypes.cast(X, ctypes.c_void_p),
            ctypes.cast(Y, ctypes.c_void_p), n, batch, xdt, ydt)


class GemvManyCall:
    """One seedlm_gemv_many call whose arguments are checked and marshalled once,
    for loops that repeat the same call (a serving step, a benchmark): calling
    the object only crosses the C ABI.  It keeps the matrices and tensors alive;
    their contents may change between calls, their storage may not."""

    def __init__(self, mats, xs, ys, batch=1, stream=None):
        self._args = _many_args(mats, xs, ys, batch)
        self._keep = (list(mats), list(xs), list(ys))
        L = lib()
        self._fns = {"all": L.seedlm_gemv_many, "begin": L.seedlm_gemv_many_begin,
                     "end": L.seedlm_gemv_many_end, "noalloc": L.seedlm_gemv_many_noalloc}
        self._stream = None if stream is None else _stream_ptr(stream)

    def __call__(self, stream=None, phase="all"):
        """Run on `stream` (default: the one given at construction, else torch's
        current stream)."""
        sp = _stream_ptr(stream) if stream is not None or self._stream is None else self._stream
        st = self._fns[phase](*self._args, sp)
        if st != OK:
            raise SeedLMError(st, "seedlm_gemv_many")


def seedlm_gemv_many(mats, xs, ys, batch=1, stream=None, phase="all"):
    """ys[i] = W_i xs[i] for several packed matrices, in as few launches as possible.

    phase "begin" / "end" runs only seedlm_gemv_many_begin / _end."""
    fn = {"all": lib().seedlm_gemv_many, "begin": lib().seedlm_gemv_many_begin,
          "end": lib().seedlm_gemv_many_end}[phase]
    _check(fn(*_many_args(mats, xs, ys, batch), _stream_ptr(stream)), "seedlm_gemv_many")
    return ys


def seedlm_gemv_many_noalloc(mats, xs, ys, batch=1, stream=None):
    """seedlm_gemv_many with the partials in the library's fixed device scratch
    (no allocation; calls that overlap on one device race)."""
    _check(lib().seedlm_gemv_many_noalloc(*_many_args(mats, xs, ys, batch), _stream_ptr(stream)),
           "seedlm_gemv_many_noalloc")
    return ys


def seedlm_gemv_scratch_bytes(mats, batch=1, x_dtype=F16, y_dtype=F16) -> int:
    """Scratch bytes a seedlm_gemv_many call over mats needs on its stream."""
    n = len(mats)
    H = (ctypes.c_void_p * n)(*[m.handle.value for m in mats])
    out = ctypes.c_size_t(0)
    _check(lib().seedlm_gemv_scratch_bytes(ctypes.cast(H, ctypes.c_void_p), n, batch, x_dtype,
                                           y_dtype, ctypes.byref(out)),
           "seedlm_gemv_scratch_bytes")
    return out.value


def seedlm_scratch_release():
    """Free the library's per-stream gemv and gemm scratch (synchronises the devices)."""
    _check(lib().seedlm_scratch_release(), "seedlm_scratch_release")


def seedlm_decode(m: SeedLMMatrix, W_out, stream=None):
    """W_out[rows][cols] (fp32 device tensor) = the dense decoded weights."""
    import torch

    if W_out.dtype != torch.float32 or W_out.numel() != m.rows * m.cols:
        raise ValueError("W_out must be a float32 tensor with rows*cols elements")
    if not (W_out.is_cuda and W_out.is_contiguous()):
        raise ValueError("W_out must be a contiguous device tensor")
    _check(lib().seedlm_decode(m.handle, ctypes.c_void_p(W_out.data_ptr()), _stream_ptr(stream)),
           "seedlm_decode")
    return W_out


def seedlm_gemm(m: SeedLMMatrix, X, Y, stream=None):
    """Y[ntok][rows] = X[ntok][cols] W^T (fp16 device tensors), any ntok >= 1."""
    if X.dim() != 2 or X.shape[1] != m.cols or Y.numel() != X.shape[0] * m.rows:
        raise ValueError("X must be [ntok][cols] and Y hold ntok*rows elements")
    if not (X.is_cuda and Y.is_cuda and X.is_contiguous() and Y.is_contiguous()):
        raise ValueError("X and Y must be contiguous device tensors")
    _check(lib().seedlm_gemm(m.handle, ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(Y.data_ptr()),
                             X.shape[0], _dtype_code(X), _dtype_code(Y), _stream_ptr(stream)),
           "seedlm_gemm")
    return Y


def seedlm_gemm_scratch_bytes(m: SeedLMMatrix, ntok: int) -> int:
    """Scratch bytes a seedlm_gemm call on m with ntok activation rows uses on its stream."""
    n = ctypes.c_size_t(0)
    _check(lib().seedlm_gemm_scratch_bytes(m.handle, ntok, ctypes.byref(n)),
           "seedlm_gemm_scratch_bytes")
    return n.value


def seedlm_gemm_decoded_bytes(m: SeedLMMatrix) -> int:
    """Workspace bytes for seedlm_gemm_decoded on m: the decoded matrix (rows * cols * 2,
    rounded up to 256) plus 32 MiB of GEMM scratch."""
    n = ctypes.c_size_t(0)
    _check(lib().seedlm_gemm_decoded_bytes(m.handle, ctypes.byref(n)), "seedlm_gemm_decoded_bytes")
    return n.value


def seedlm_gemm_decoded(m: SeedLMMatrix, X, Y, workspace, stream=None):
    """Y = X W^T through a decoded fp16 copy of W in `workspace` (a device
    tensor of at least rows * cols * 2 bytes; seedlm_gemm_decoded_bytes(m) adds the GEMM's
    scratch) and hipBLASLt."""
    if X.dim() != 2 or X.shape[1] != m.cols or Y.numel() != X.shape[0] * m.rows:
        raise ValueError("X must be [ntok][cols] and Y hold ntok*rows elements")
    if not (X.is_cuda and Y.is_cuda and workspace.is_cuda and X.is_contiguous() and
            Y.is_contiguous() and workspace.is_contiguous()):
        raise ValueError("X, Y and workspace must be contiguous device tensors")
    _check(lib().seedlm_gemm_decoded(m.handle, ctypes.c_void_p(X.data_ptr()),
                                     ctypes.c_void_p(Y.data_ptr()), X.shape[0], _dtype_code(X),
                                     _dtype_code(Y), ctypes.c_void_p(workspace.data_ptr()),
                                     workspace.numel() * workspace.element_size(),
                                     _stream_ptr(stream)), "seedlm_gemm_decoded")
    return Y


def seedlm_export(m: SeedLMMatrix) -> bytes:
    n = ctypes.c_size_t(0)
    _check(lib().seedlm_export(m.handle, None, ctypes.byref(n)), "seedlm_export")
    buf = ctypes.create_string_buffer(n.value)
    _check(lib().seedlm_export(m.handle, ctypes.cast(buf, ctypes.c_void_p), ctypes.byref(n)),
           "seedlm_export")
    return buf.raw[: n.value]


STREAM_READ_SINK = 8192


def seedlm_stream_read(buf, sink, stream=None):
    """Baseline: read the device tensor buf once (plain streaming read) and write
    per-workgroup XOR checksums into sink (device int32[STREAM_READ_SINK])."""
    if not (buf.is_cuda and sink.is_cuda and buf.is_contiguous()):
        raise ValueError("buf and sink must be device tensors, buf contiguous")
    if sink.numel() * sink.element_size() < 4 * STREAM_READ_SINK:
        raise ValueError("sink must hold STREAM_READ_SINK 32-bit words")
    _check(lib().seedlm_stream_read(ctypes.c_void_p(buf.data_ptr()),
                                    buf.numel() * buf.element_size(),
                                    ctypes.c_void_p(sink.data_ptr()), _stream_ptr(stream)),
           "seedlm_stream_read")
    return sink


def seedlm_bench_time_next_call(start, stop):
    """Measurement only: the next gemv call of this thread records torch.cuda.Event
    `start` when its first main kernel starts and `stop` when its last one ends.
    The events must exist already (torch creates an event at its first record)."""
    ptr = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in (start, stop)]
    if any(p is not None and not p.value for p in ptr):
        raise ValueError("record each event once before handing it to the library")
    _check(lib().seedlm_bench_time_next_call(*ptr), "seedlm_bench_time_next_call")


def seedlm_fp16_gemv(W, x, y, batch=None, stream=None):
    """Baseline: y = W x with fp16 W[rows][cols], x[batch][cols], y[batch][rows]."""
    rows, cols = W.shape
    if batch is None:
        batch = 1 if x.dim() == 1 else x.shape[0]
    _check(lib().seedlm_fp16_gemv(ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), rows, cols, batch,
                                  _stream_ptr(stream)), "seedlm_fp16_gemv")
    return y


class SeedLMEncoder:
    """A seed-search encoder for one format on the current device (owns its table)."""

    def __init__(self, C=8, P=3, K=16, Q=4):
        h = ctypes.c_void_p()
        _check(lib().seedlm_encoder_create(C, P, K, Q, ctypes.byref(h)), "seedlm_encoder_create")
        self._h = h
        self.C, self.P, self.K, self.Q = C, P, K, Q

    @property
    def handle(self):
        if self._h is None or not self._h.value:
            raise ValueError("encoder has been destroyed")
        return self._h

    def destroy(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(lib().seedlm_encoder_destroy(self._h), "seedlm_encoder_destroy")
        self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def seedlm_encode(enc: SeedLMEncoder, W, seeds=None, coeffs=None, exps=None, err=None,
                  stream=None):
    """Seed search for every block of W (bf16 device tensor [rows][cols]).

    Returns device tensors seeds [rows][nb] (torch.int16 holding the uint16 bit
    patterns; int32 for K > 16), coeffs [rows][nb][P] int8, exps [rows][nb] int8 and err [rows][nb]
    float32 (the fp32 score of each chosen record).  Preallocated outputs may be
    passed in."""
    import torch

    if W.dtype != torch.bfloat16 or W.dim() != 2 or not (W.is_cuda and W.is_contiguous()):
        raise ValueError("W must be a contiguous 2-D bfloat16 device tensor")
    rows, cols = W.shape
    nb = -(-cols // enc.C)  # a short last block is searched with zeros in its missing slots
    dev = W.device
    if seeds is None:
        seeds = torch.empty((rows, nb), dtype=torch.int16 if enc.K <= 16 else torch.int32,
                            device=dev)
    if coeffs is None:
        coeffs = torch.empty((rows, nb, enc.P), dtype=torch.int8, device=dev)
    if exps is None:
        exps = torch.empty((rows, nb), dtype=torch.int8, device=dev)
    if err is None:
        err = torch.empty((rows, nb), dtype=torch.float32, device=dev)
    for t, n in ((seeds, rows * nb), (coeffs, rows * nb * enc.P), (exps, rows * nb),
                 (err, rows * nb)):
        if t.numel() != n or not (t.is_cuda and t.is_contiguous()):
            raise ValueError("output tensors have the wrong size or are not contiguous")
    _check(lib().seedlm_encode(enc.handle, ctypes.c_void_p(W.data_ptr()), rows, cols,
                               ctypes.c_void_p(seeds.data_ptr()),
                               ctypes.c_void_p(coeffs.data_ptr()),
                               ctypes.c_void_p(exps.data_ptr()),
                               ctypes.c_void_p(err.data_ptr()), _stream_ptr(stream)),
           "seedlm_encode")
    return seeds, coeffs, exps, err
