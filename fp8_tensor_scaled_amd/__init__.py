"""Python binding of libfp8lin.so, the gfx950 FP8 linear layer.

Argument marshalling only: every function below passes device pointers,
sizes and the current HIP stream to the C entry point of the same name
(declared in include/fp8lin.h) and turns a non-OK status into an exception.
All arithmetic runs in the library's HIP kernels; there is no fallback.
torch is used for device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "E4M3", "E5M2", "FMT_MAX", "IN_BF16", "IN_F16", "IN_F32", "Ring", "library_path",
    "fp8_quantize", "fp8_quantize_ex", "fp8_quantize_t", "fp8_quantize2",
    "fp8_scale_ring_finalize", "fp8_mm", "fp8_mm_ex", "fp8_mm_pair", "fp8_colsum",
    "fp8_colsum_workspace", "fp8_quantize_colsum", "fp8_quantize_colsum_noalloc",
    "fp8_quantize_colsum_noalloc_max_bytes",
    "OUT_BF16", "OUT_E4M3", "OUT_E5M2",
    "fp8_linear_fwd", "fp8_linear_bwd", "fp8_linear_fwd_workspace",
    "fp8_linear_bwd_workspace", "fp8_linear_bwd_workspace_codes", "fp8_linear_fwd_x8_offset",
    "fp8_linear_fwd_w8_offset",
    "EXPORTED_SYMBOLS",
]

E4M3 = 0
E5M2 = 1
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp8lin.so")

EXPORTED_SYMBOLS = (
    "fp8_ring_state_floats", "fp8_format_max", "fp8_quantize", "fp8_quantize_ex",
    "fp8_quantize_t", "fp8_quantize2",
    "fp8_scale_ring_finalize",
    "fp8_mm", "fp8_mm_ex", "fp8_mm_pair", "fp8_colsum_workspace", "fp8_colsum",
    "fp8_quantize_colsum", "fp8_quantize_colsum_noalloc_max_bytes",
    "fp8_quantize_colsum_noalloc", "fp8_linear_fwd_workspace",
    "fp8_linear_fwd_x8_offset", "fp8_linear_fwd_w8_offset", "fp8_linear_fwd",
    "fp8_linear_bwd_workspace", "fp8_linear_bwd_workspace_codes", "fp8_linear_bwd",
    "fp8_last_error", "fp8_version",
)


class _RingC(ctypes.Structure):
    _fields_ = [("state", ctypes.c_void_p), ("len", ctypes.c_int32), ("idx", ctypes.c_int32),
                ("initialized", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _MmArgs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("fmt", ctypes.c_int32),
                ("trans_a", ctypes.c_int32), ("trans_b", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("m", ctypes.c_int64), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64),
                ("batch", ctypes.c_int64), ("stride_a", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("scale_a", ctypes.c_void_p),
                ("scale_b", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("out", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m fp8_tensor_scaled_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F, S = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                         ctypes.c_size_t)
    R = ctypes.POINTER(_RingC)
    sig = {
        "fp8_ring_state_floats": (I64, [I32]),
        "fp8_format_max": (F, [I32]),
        "fp8_quantize": (I32, [P, I64, I32, P, P, P, R, I32, P, P]),
        "fp8_quantize_ex": (I32, [P, I32, I64, I32, P, P, P, R, I32, P, P]),
        "fp8_quantize_t": (I32, [P, I64, I64, I32, P, P, P, R, I32, P, P]),
        "fp8_quantize2": (I32, [P, I64, I32, P, P, I32, P, R, I32, P, P]),
        "fp8_scale_ring_finalize": (I32, [R, I32, P, I32, P]),
        "fp8_mm": (I32, [P, P, I32, I32, I32, I64, I64, I64, I64, I64, I64, I64, I64, P, P, P,
                         P, P]),
        "fp8_mm_ex": (I32, [P, P, I32, I32, I32, I64, I64, I64, I64, I64, I64, I64, I64, P, P,
                            P, P, I32, P, P, P]),
        "fp8_mm_pair": (I32, [ctypes.POINTER(_MmArgs), ctypes.POINTER(_MmArgs), P]),
        "fp8_colsum_workspace": (S, [I64, I64]),
        "fp8_colsum": (I32, [P, I64, I64, P, P, S, P]),
        "fp8_quantize_colsum": (I32, [P, I64, I64, I32, P, P, R, I32, P, P, P, S, P]),
        "fp8_quantize_colsum_noalloc_max_bytes": (S, []),
        "fp8_quantize_colsum_noalloc": (I32, [P, I64, I64, I32, P, P, R, I32, P, P, P]),
        "fp8_linear_fwd_workspace": (S, [I64, I64, I64]),
        "fp8_linear_fwd_x8_offset": (S, [I64, I64, I64]),
        "fp8_linear_fwd_w8_offset": (S, [I64, I64, I64]),
        "fp8_linear_fwd": (I32, [P, P, P, I64, I64, I64, I32, I32, I32, R, R, P, S, P, P, I32, P,
                                 P, P]),
        "fp8_linear_bwd_workspace": (S, [I64, I64, I64]),
        "fp8_linear_bwd_workspace_codes": (S, [I64, I64, I64]),
        "fp8_linear_bwd": (I32, [P, P, P, I64, I64, I64, I32, I32, I32, P, R, P, S, P, P, P, P,
                                 P, P, P]),
        "fp8_last_error": (ctypes.c_char_p, []),
        "fp8_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


class _Library:
    """The loaded library, loaded on first use: importing the package (for
    instance to run its build module) never needs a built library, and the
    first call raises if it is missing."""

    _handle = None

    def __getattr__(self, name: str):
        if _Library._handle is None:
            _Library._handle = _load()
        return getattr(_Library._handle, name)


_lib = _Library()


def _check(status: int, what: str) -> None:
    if status == 0:
        return
    msg = _lib.fp8_last_error().decode(errors="replace")
    if status == 1:
        raise ValueError(f"{what}: {msg}")
    raise RuntimeError(f"{what} failed (status {status}): {msg}")


def _ptr(t: torch.Tensor | None):
    """Device pointer of a tensor handed to the library (None -> NULL)."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"tensor of shape {tuple(t.shape)} is on {t.device}, not a GPU")
    return ctypes.c_void_p(t.data_ptr())


# Element sizes of the buffers the C entry points take: bf16 / fp16 bit
# patterns (2 bytes), fp8 codes (1 byte), fp32 steps and amaxes (4 bytes).
_BYTE1 = (torch.uint8, torch.int8, torch.float8_e4m3fn, torch.float8_e5m2)
_BYTE2 = (torch.bfloat16, torch.int16, torch.float16) + (
    (torch.uint16,) if hasattr(torch, "uint16") else ())
_F32 = (torch.float32,)


def _buf(t: torch.Tensor | None, what: str, numel: int, dtypes: tuple,
         nullable: bool = True) -> None:
    """The C side sees only a device pointer: check here that the tensor is
    a dense tensor of one of `dtypes` holding at least `numel` elements, so a
    short or mistyped buffer raises ValueError instead of being read or
    written out of bounds (_ptr then refuses tensors that are not on a
    GPU)."""
    if t is None:
        if nullable:
            return
        raise ValueError(f"{what}: required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of "
                         f"{', '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, needs at least {numel}")


def _ws_bytes(t: torch.Tensor, what: str) -> int:
    """Byte size of a workspace tensor (any dtype, dense, on a GPU)."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{what}: a contiguous GPU tensor is required")
    return t.numel() * t.element_size()


def _extent(rows: int, cols: int, ld: int, batch: int, stride: int) -> int:
    """Elements spanned by `batch` slices of a [rows][cols] matrix with row
    stride ld and batch stride `stride` (0 broadcasts one slice)."""
    if rows <= 0 or cols <= 0 or batch <= 0:
        return 0
    return (batch - 1) * max(int(stride), 0) + (rows - 1) * int(ld) + cols


# torch's raw accessors of the current device and its current stream: the
# public torch.cuda.current_stream() costs about 10 us a call in device
# checks, several times per linear step.
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_RAW_DEVICE = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream=None):
    """HIP stream handle: torch's current stream (of the current device) by
    default, an int handle as given (0 = the null stream), or a
    torch.cuda.Stream."""
    if stream is None:
        if _RAW_STREAM is not None and _RAW_DEVICE is not None:
            return ctypes.c_void_p(_RAW_STREAM(_RAW_DEVICE()))
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Ring:
    """Delayed-scaling state of one operand: the zero-filled device buffer
    [hist len | scale | legacy | amax | done | kernel scratch] (only the first
    len + 4 words, `published()`, mean anything to callers; the scratch is
    zero between calls) and the host-side slot index / initialized flag the
    linear calls maintain."""

    def __init__(self, length: int = 16, device="cuda"):
        n = int(_lib.fp8_ring_state_floats(length))
        if n <= 0:
            raise ValueError(f"bad ring length {length}")
        self.state = torch.zeros(n, dtype=torch.float32, device=device)
        self.c = _RingC(self.state.data_ptr(), length, 0, 0, 0)

    @property
    def len(self) -> int:
        return self.c.len

    def published(self) -> torch.Tensor:
        """View of [hist len | scale | legacy | amax | done]."""
        return self.state[: self.c.len + 4]

    def scratch(self) -> torch.Tensor:
        """View of the kernel scratch after `done` (zero between calls)."""
        return self.state[self.c.len + 4:]

    @property
    def idx(self) -> int:
        return self.c.idx

    @idx.setter
    def idx(self, v: int) -> None:
        self.c.idx = int(v)

    @property
    def initialized(self) -> bool:
        return bool(self.c.initialized)

    @initialized.setter
    def initialized(self, v: bool) -> None:
        self.c.initialized = int(bool(v))

    @property
    def hist(self) -> torch.Tensor:
        return self.state[: self.len]

    @property
    def scale(self) -> torch.Tensor:
        return self.state[self.len: self.len + 1]


def _ring_ref(r: Ring | None):
    return None if r is None else ctypes.byref(r.c)


def fp8_quantize(x: torch.Tensor, fmt: int, scale: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, ring: Ring | None = None, margin: int = 0,
                 scale_used: torch.Tensor | None = None, stream=None,
                 amax_out: torch.Tensor | None = None) -> None:
    """bf16 x -> fp8 codes in ``out`` (uint8, same numel), and / or max |x|
    in ``amax_out`` (float32 [1]); see fp8lin.h."""
    _buf(x, "x", 0, _BYTE2, nullable=False)
    n = x.numel()
    _buf(out, "out", n, _BYTE1)
    _buf(scale, "scale", 1, _F32)
    _buf(scale_used, "scale_used", 1, _F32)
    _buf(amax_out, "amax_out", 1, _F32)
    st = _lib.fp8_quantize(_ptr(x), x.numel(), fmt, _ptr(scale), _ptr(out), _ptr(amax_out),
                           _ring_ref(ring), margin, _ptr(scale_used), _stream(stream))
    _check(st, "fp8_quantize")


def fp8_quantize_t(x: torch.Tensor, rows: int, cols: int, fmt: int, scale: torch.Tensor,
                   out_t: torch.Tensor, out: torch.Tensor | None = None,
                   ring: Ring | None = None, margin: int = 0,
                   scale_used: torch.Tensor | None = None, stream=None) -> None:
    """bf16 x [rows][cols] -> codes transposed in out_t [cols][rows] (and
    row-major in ``out`` when given) from one read of x; see fp8lin.h."""
    n = max(int(rows), 0) * max(int(cols), 0)
    _buf(x, "x", n, _BYTE2, nullable=False)
    _buf(out_t, "out_t", n, _BYTE1, nullable=False)
    _buf(out, "out", n, _BYTE1)
    _buf(scale, "scale", 1, _F32)
    _buf(scale_used, "scale_used", 1, _F32)
    st = _lib.fp8_quantize_t(_ptr(x), rows, cols, fmt, _ptr(scale), _ptr(out), _ptr(out_t),
                             _ring_ref(ring), margin, _ptr(scale_used), _stream(stream))
    _check(st, "fp8_quantize_t")


IN_BF16, IN_F16, IN_F32 = 0, 1, 2
_IN_OF_DTYPE = {torch.bfloat16: IN_BF16, torch.float16: IN_F16, torch.float32: IN_F32}


def fp8_quantize_ex(x: torch.Tensor, fmt: int, scale: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, ring: Ring | None = None, margin: int = 0,
                    scale_used: torch.Tensor | None = None, in_type: int | None = None,
                    stream=None, amax_out: torch.Tensor | None = None) -> None:
    """bf16, fp16 or fp32 x -> fp8 codes; ``in_type`` defaults to x's dtype
    (bfloat16 / float16 / float32; give it for int16 bit views); see
    fp8lin.h."""
    if in_type is None:
        if x.dtype not in _IN_OF_DTYPE:
            raise ValueError(f"fp8_quantize_ex: no input type for dtype {x.dtype}")
        in_type = _IN_OF_DTYPE[x.dtype]
    if in_type not in (IN_BF16, IN_F16, IN_F32):
        raise ValueError(f"fp8_quantize_ex: bad input type {in_type}")
    _buf(x, "x", 0, _F32 if in_type == IN_F32 else _BYTE2, nullable=False)
    n = x.numel()
    _buf(out, "out", n, _BYTE1)
    _buf(scale, "scale", 1, _F32)
    _buf(scale_used, "scale_used", 1, _F32)
    _buf(amax_out, "amax_out", 1, _F32)
    st = _lib.fp8_quantize_ex(_ptr(x), in_type, x.numel(), fmt, _ptr(scale), _ptr(out),
                              _ptr(amax_out), _ring_ref(ring), margin, _ptr(scale_used),
                              _stream(stream))
    _check(st, "fp8_quantize_ex")


def fp8_quantize2(x: torch.Tensor, fmt: int, scale: torch.Tensor, out: torch.Tensor, fmt2: int,
                  out2: torch.Tensor, ring: Ring | None = None, margin: int = 0,
                  scale_used: torch.Tensor | None = None, stream=None) -> None:
    """bf16 x -> fp8 codes of format ``fmt`` in ``out`` and of ``fmt2`` in
    ``out2`` from one read of x (same step); see fp8lin.h."""
    _buf(x, "x", 0, _BYTE2, nullable=False)
    n = x.numel()
    _buf(out, "out", n, _BYTE1, nullable=False)
    _buf(out2, "out2", n, _BYTE1, nullable=False)
    _buf(scale, "scale", 1, _F32)
    _buf(scale_used, "scale_used", 1, _F32)
    st = _lib.fp8_quantize2(_ptr(x), x.numel(), fmt, _ptr(scale), _ptr(out), fmt2, _ptr(out2),
                            _ring_ref(ring), margin, _ptr(scale_used), _stream(stream))
    _check(st, "fp8_quantize2")


def fp8_scale_ring_finalize(ring: Ring, fmt: int, amax: torch.Tensor, margin: int = 0,
                            stream=None) -> None:
    _buf(amax, "amax", 1, _F32, nullable=False)
    st = _lib.fp8_scale_ring_finalize(_ring_ref(ring), fmt, _ptr(amax), margin, _stream(stream))
    _check(st, "fp8_scale_ring_finalize")


def _check_mm(a, b, trans_a, trans_b, m, n, k, lda, ldb, batch, stride_a, stride_b, scale_a,
              scale_b, bias, bias_dtypes, out, out_bytes) -> None:
    """Buffer sizes of one GEMM: A stored [m][k] (or [k][m] when trans_a)
    with row stride lda, B stored [k][n] (or [n][k] when trans_b) with row
    stride ldb, batch slices `stride_*` apart (0 broadcasts), a bias of n
    values and a contiguous [batch][m][n] output."""
    m, n, k, batch = int(m), int(n), int(k), int(batch)
    if min(m, n, k, batch) < 0:
        raise ValueError("fp8_mm: negative size")
    ra, ca = (k, m) if trans_a else (m, k)
    rb, cb = (n, k) if trans_b else (k, n)
    _buf(a, "a", _extent(ra, ca, lda, batch, stride_a), _BYTE1, nullable=False)
    _buf(b, "b", _extent(rb, cb, ldb, batch, stride_b), _BYTE1, nullable=False)
    _buf(scale_a, "scale_a", 1, _F32, nullable=False)
    _buf(scale_b, "scale_b", 1, _F32, nullable=False)
    _buf(bias, "bias", n, bias_dtypes)
    _buf(out, "out", batch * m * n, _BYTE2 if out_bytes == 2 else _BYTE1, nullable=False)


def fp8_mm(a: torch.Tensor, b: torch.Tensor, fmt: int, trans_a: int, trans_b: int, m: int,
           n: int, k: int, lda: int, ldb: int, batch: int, stride_a: int, stride_b: int,
           scale_a: torch.Tensor, scale_b: torch.Tensor, bias: torch.Tensor | None,
           out: torch.Tensor, stream=None) -> None:
    _check_mm(a, b, trans_a, trans_b, m, n, k, lda, ldb, batch, stride_a, stride_b, scale_a,
              scale_b, bias, _BYTE2, out, 2)
    st = _lib.fp8_mm(_ptr(a), _ptr(b), fmt, trans_a, trans_b, m, n, k, lda, ldb, batch,
                     stride_a, stride_b, _ptr(scale_a), _ptr(scale_b), _ptr(bias), _ptr(out),
                     _stream(stream))
    _check(st, "fp8_mm")


# Output types of fp8_mm_ex (fp8_out_t).
OUT_BF16, OUT_E4M3, OUT_E5M2 = 0, 1, 2


def fp8_mm_ex(a: torch.Tensor, b: torch.Tensor, fmt: int, trans_a: int, trans_b: int, m: int,
              n: int, k: int, lda: int, ldb: int, batch: int, stride_a: int, stride_b: int,
              scale_a: torch.Tensor, scale_b: torch.Tensor, bias: torch.Tensor | None,
              bias_scale: torch.Tensor | None, out_type: int, out_scale: torch.Tensor | None,
              out: torch.Tensor, stream=None) -> None:
    """fp8_mm with an fp8 bias (codes of ``fmt`` and their step ``bias_scale``)
    and / or an fp8 output (``out_type`` OUT_E4M3 / OUT_E5M2, step
    ``out_scale``); see fp8lin.h."""
    if out_type not in (OUT_BF16, OUT_E4M3, OUT_E5M2):
        raise ValueError(f"fp8_mm_ex: bad output type {out_type}")
    _check_mm(a, b, trans_a, trans_b, m, n, k, lda, ldb, batch, stride_a, stride_b, scale_a,
              scale_b, bias, _BYTE1 if bias_scale is not None else _BYTE2, out,
              2 if out_type == OUT_BF16 else 1)
    _buf(bias_scale, "bias_scale", 1, _F32)
    _buf(out_scale, "out_scale", 1, _F32)
    st = _lib.fp8_mm_ex(_ptr(a), _ptr(b), fmt, trans_a, trans_b, m, n, k, lda, ldb, batch,
                        stride_a, stride_b, _ptr(scale_a), _ptr(scale_b), _ptr(bias),
                        _ptr(bias_scale), out_type, _ptr(out_scale), _ptr(out),
                        _stream(stream))
    _check(st, "fp8_mm_ex")


def _mm_args(a, b, fmt, trans_a, trans_b, m, n, k, lda, ldb, batch, stride_a, stride_b,
             scale_a, scale_b, bias, out) -> _MmArgs:
    return _MmArgs(_ptr(a), _ptr(b), fmt, trans_a, trans_b, 0, m, n, k, lda, ldb, batch,
                   stride_a, stride_b, _ptr(scale_a), _ptr(scale_b), _ptr(bias), _ptr(out))


def fp8_mm_pair(p0: tuple, p1: tuple, stream=None) -> None:
    """Two independent fp8_mm products from one call; p0, p1 are fp8_mm's
    positional arguments (a, b, fmt, trans_a, trans_b, m, n, k, lda, ldb,
    batch, stride_a, stride_b, scale_a, scale_b, bias, out).  One launch when
    p0 is NN and p1 is TN and both are large; see fp8lin.h."""
    for p in (p0, p1):
        if len(p) != 17:
            raise ValueError("fp8_mm_pair: each problem takes fp8_mm's 17 arguments")
        (a, b, _fmt, ta, tb, m, n, k, lda, ldb, batch, sta, stb, sa, sb, bias, out) = p
        _check_mm(a, b, ta, tb, m, n, k, lda, ldb, batch, sta, stb, sa, sb, bias, _BYTE2, out, 2)
    a0, a1 = _mm_args(*p0), _mm_args(*p1)
    st = _lib.fp8_mm_pair(ctypes.byref(a0), ctypes.byref(a1), _stream(stream))
    _check(st, "fp8_mm_pair")


def fp8_colsum_workspace(m: int, n: int) -> int:
    return int(_lib.fp8_colsum_workspace(m, n))


def fp8_colsum(g: torch.Tensor, m: int, n: int, db: torch.Tensor, workspace: torch.Tensor,
               stream=None) -> None:
    _buf(g, "g", max(int(m), 0) * max(int(n), 0), _BYTE2, nullable=False)
    _buf(db, "db", max(int(n), 0), _BYTE2, nullable=False)
    st = _lib.fp8_colsum(_ptr(g), m, n, _ptr(db), _ptr(workspace),
                         _ws_bytes(workspace, "workspace"), _stream(stream))
    _check(st, "fp8_colsum")


def fp8_quantize_colsum(g: torch.Tensor, m: int, n: int, fmt: int, scale: torch.Tensor,
                        out: torch.Tensor, db: torch.Tensor, workspace: torch.Tensor,
                        ring: Ring | None = None, margin: int = 0,
                        scale_used: torch.Tensor | None = None, stream=None) -> None:
    """Quantize of g [m][n] and its column sum db from one read of g; the
    results equal fp8_quantize + fp8_colsum; see fp8lin.h."""
    mn = max(int(m), 0) * max(int(n), 0)
    _buf(g, "g", mn, _BYTE2, nullable=False)
    _buf(out, "out", mn, _BYTE1)
    _buf(db, "db", max(int(n), 0), _BYTE2, nullable=False)
    _buf(scale, "scale", 1, _F32)
    _buf(scale_used, "scale_used", 1, _F32)
    st = _lib.fp8_quantize_colsum(_ptr(g), m, n, fmt, _ptr(scale), _ptr(out), _ring_ref(ring),
                                  margin, _ptr(scale_used), _ptr(db), _ptr(workspace),
                                  _ws_bytes(workspace, "workspace"), _stream(stream))
    _check(st, "fp8_quantize_colsum")


def fp8_quantize_colsum_noalloc_max_bytes() -> int:
    return int(_lib.fp8_quantize_colsum_noalloc_max_bytes())


def fp8_quantize_colsum_noalloc(g: torch.Tensor, m: int, n: int, fmt: int,
                                scale: torch.Tensor, out: torch.Tensor, db: torch.Tensor,
                                ring: Ring | None = None, margin: int = 0,
                                scale_used: torch.Tensor | None = None, stream=None) -> None:
    """fp8_quantize_colsum with its partials in the library's static scratch
    (no workspace, no allocation); see fp8lin.h."""
    mn = max(int(m), 0) * max(int(n), 0)
    _buf(g, "g", mn, _BYTE2, nullable=False)
    _buf(out, "out", mn, _BYTE1, nullable=False)
    _buf(db, "db", max(int(n), 0), _BYTE2, nullable=False)
    _buf(scale, "scale", 1, _F32, nullable=False)
    _buf(scale_used, "scale_used", 1, _F32)
    st = _lib.fp8_quantize_colsum_noalloc(_ptr(g), m, n, fmt, _ptr(scale), _ptr(out),
                                          _ring_ref(ring), margin, _ptr(scale_used), _ptr(db),
                                          _stream(stream))
    _check(st, "fp8_quantize_colsum_noalloc")


def fp8_linear_fwd_workspace(M: int, N: int, K: int) -> int:
    return int(_lib.fp8_linear_fwd_workspace(M, N, K))


def fp8_linear_fwd_x8_offset(M: int, N: int, K: int) -> int:
    return int(_lib.fp8_linear_fwd_x8_offset(M, N, K))


def fp8_linear_fwd_w8_offset(M: int, N: int, K: int) -> int:
    return int(_lib.fp8_linear_fwd_w8_offset(M, N, K))


def fp8_linear_bwd_workspace(M: int, N: int, K: int) -> int:
    return int(_lib.fp8_linear_bwd_workspace(M, N, K))


def fp8_linear_bwd_workspace_codes(M: int, N: int, K: int) -> int:
    return int(_lib.fp8_linear_bwd_workspace_codes(M, N, K))


def fp8_linear_fwd(x, w, bias, M, N, K, fmt, dynamic, margin, ring_x: Ring | None,
                   ring_w: Ring | None, workspace: torch.Tensor, scales_out: torch.Tensor,
                   out: torch.Tensor, stream=None, fmt_bwd: int = E5M2,
                   x8_bwd: torch.Tensor | None = None, w8_bwd: torch.Tensor | None = None) -> None:
    """Forward of the linear layer; with x8_bwd / w8_bwd (delayed scaling)
    the same pass also writes x's and w's codes in fmt_bwd for the backward;
    see fp8lin.h."""
    M, N, K = int(M), int(N), int(K)
    if min(M, N, K) < 0:
        raise ValueError("fp8_linear_fwd: negative size")
    _buf(x, "x", M * K, _BYTE2, nullable=False)
    _buf(w, "w", N * K, _BYTE2, nullable=False)
    _buf(bias, "bias", N, _BYTE2)
    _buf(scales_out, "scales_out", 2, _F32)
    _buf(out, "out", M * N, _BYTE2, nullable=False)
    _buf(x8_bwd, "x8_bwd", M * K, _BYTE1)
    _buf(w8_bwd, "w8_bwd", N * K, _BYTE1)
    _linear_fwd_call(x, w, bias, M, N, K, fmt, dynamic, margin, ring_x, ring_w, workspace,
                     scales_out, out, stream, fmt_bwd, x8_bwd, w8_bwd)


def _linear_fwd_call(x, w, bias, M, N, K, fmt, dynamic, margin, ring_x, ring_w, workspace,
                     scales_out, out, stream, fmt_bwd, x8_bwd, w8_bwd) -> None:
    """fp8_linear_fwd's call itself, for callers whose buffers are sized and
    typed for (M, N, K) by construction (the autograd layer allocates them
    from the operands' own shapes): no per-buffer checks beyond the device
    one."""
    st = _lib.fp8_linear_fwd(_ptr(x), _ptr(w), _ptr(bias), M, N, K, fmt, int(dynamic), margin,
                             _ring_ref(ring_x), _ring_ref(ring_w), _ptr(workspace),
                             _ws_bytes(workspace, "workspace"), _ptr(scales_out), _ptr(out),
                             fmt_bwd,
                             _ptr(x8_bwd), _ptr(w8_bwd), _stream(stream))
    _check(st, "fp8_linear_fwd")


def fp8_linear_bwd(g, x, w, M, N, K, fmt, dynamic, margin, scales_fwd, ring_g: Ring | None,
                   workspace: torch.Tensor, scales_out, dx, dw, db, stream=None,
                   x8_bwd: torch.Tensor | None = None, w8_bwd: torch.Tensor | None = None) -> None:
    """Gradients of the linear layer; x8_bwd / w8_bwd (delayed scaling) are
    the forward's backward-format codes, used instead of quantizing x / w;
    see fp8lin.h."""
    M, N, K = int(M), int(N), int(K)
    if min(M, N, K) < 0:
        raise ValueError("fp8_linear_bwd: negative size")
    _buf(g, "g", M * N, _BYTE2, nullable=False)
    _buf(x, "x", M * K, _BYTE2)
    _buf(w, "w", N * K, _BYTE2)
    _buf(scales_fwd, "scales_fwd", 2, _F32)
    _buf(scales_out, "scales_out", 3, _F32)
    _buf(dx, "dx", M * K, _BYTE2)
    _buf(dw, "dw", N * K, _BYTE2)
    _buf(db, "db", N, _BYTE2)
    _buf(x8_bwd, "x8_bwd", M * K, _BYTE1)
    _buf(w8_bwd, "w8_bwd", N * K, _BYTE1)
    _linear_bwd_call(g, x, w, M, N, K, fmt, dynamic, margin, scales_fwd, ring_g, workspace,
                     scales_out, dx, dw, db, stream, x8_bwd, w8_bwd)


def _linear_bwd_call(g, x, w, M, N, K, fmt, dynamic, margin, scales_fwd, ring_g, workspace,
                     scales_out, dx, dw, db, stream, x8_bwd, w8_bwd) -> None:
    """fp8_linear_bwd's call itself (see _linear_fwd_call)."""
    st = _lib.fp8_linear_bwd(_ptr(g), _ptr(x), _ptr(w), M, N, K, fmt, int(dynamic), margin,
                             _ptr(scales_fwd), _ring_ref(ring_g), _ptr(workspace),
                             _ws_bytes(workspace, "workspace"), _ptr(scales_out), _ptr(dx),
                             _ptr(dw), _ptr(db),
                             _ptr(x8_bwd), _ptr(w8_bwd), _stream(stream))
    _check(st, "fp8_linear_bwd")
