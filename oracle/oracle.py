"""Python side of the CPU oracle of the FP8 linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the HIP library or its binding: the arithmetic lives in
``fp8_oracle.c`` (plain loops, fp64 sums, IEEE fp32 where the method computes
in fp32) and the orchestration below follows the steps of the pages in their
order.

Sources (AstrAI repository web pages, by ViperEkura):
  [CMP]  compare view 3e57cc8...main: astrai/extension/fp8.py
         (FP8Recipe, _ScaleRing, fp8_linear_forward, _LinearFp8.backward),
         csrc/kernels/fp8/quantize.cuh (publish_amax, fp8_quantize_kernel)
  [LOG1] commit log at 3e57cc8 (scale snapshot, forward scale reused by the
         gradients, amax from raw values)

Data conventions: bf16 tensors are numpy ``uint16`` bit patterns, fp8
tensors are numpy ``uint8`` codes, scales are ``numpy.float32``.

Readings of points the pages leave open (each listed in the design notes):
  * seed(): the hidden body is read as "fold the tensor's amax into the
    current slot, then publish the scale" (the same step as the in-kernel
    fold), which for <= history_len steps equals a fill of the window.
  * HYBRID: forward E4M3 (x, w), backward E5M2 (g, and x, w re-quantized in
    E5M2).  Delayed backward reuses the forward's sx, sw; dynamic backward
    re-measures them in the backward format, as the pages' backward does.
  * fp8 GEMM output: out_scale is the output's step (the removed op calls it
    the quantization step of the output); the codes follow the quantize's
    convention, fp32(y) times the fp32 reciprocal of the step, then the
    saturating cast.  An fp8 bias is in the operands' format; its value is
    the fp32 product of the decoded code and bias_scale.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

E4M3 = 0
E5M2 = 1
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-std=c11", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    lib.orc_decode.argtypes = [ctypes.c_uint8, I]
    lib.orc_decode.restype = F
    lib.orc_encode.argtypes = [F, I]
    lib.orc_encode.restype = ctypes.c_uint8
    lib.orc_encode_array.argtypes = [P, I64, I, P]
    lib.orc_encode_bits_range.argtypes = [ctypes.c_uint32, I64, I, P]
    lib.orc_bf16_from_f64.argtypes = [ctypes.c_double]
    lib.orc_bf16_from_f64.restype = ctypes.c_uint16
    lib.orc_bf16_from_f64_array.argtypes = [P, I64, P]
    lib.orc_amax.argtypes = [P, I64]
    lib.orc_amax.restype = F
    lib.orc_scale_from_peak.argtypes = [F, I, I]
    lib.orc_scale_from_peak.restype = F
    lib.orc_multiplier.argtypes = [F]
    lib.orc_multiplier.restype = F
    lib.orc_quantize.argtypes = [P, I64, I, F, P]
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = F
    lib.orc_amax_in.argtypes = [P, I64, I]
    lib.orc_amax_in.restype = F
    lib.orc_quantize_in.argtypes = [P, I64, I, I, F, P]
    lib.orc_gemm.argtypes = [P, P, I, I, I, I64, I64, I64, I64, I64, I64, I64, I64,
                             F, F, P, P]
    lib.orc_gemm_sampled.argtypes = [P, P, I, I, I, I64, I64, I64, I64, I64, F, F, P,
                                     I64, P, P, P, P, P, P]
    lib.orc_gemm_absdot.argtypes = [P, P, I, I, I, I64, I64, I64, I64, I64, I64, I64,
                                    I64, F, F, P]
    lib.orc_gemm_groupmax.argtypes = [P, P, I, I, I, I64, I64, I64, I64, I64, I64, I64,
                                      I64, F, F, P]
    lib.orc_gemm_stats.argtypes = [P, P, I, I, I, I64, I64, I64, I64, I64, I64, I64,
                                   I64, F, F, P, P]
    lib.orc_colsum.argtypes = [P, I64, I64, P]
    lib.orc_out_code.argtypes = [ctypes.c_double, I, F]
    lib.orc_out_code.restype = ctypes.c_uint8
    lib.orc_out_code_array.argtypes = [P, I64, I, F, P]
    lib.orc_gemm_ex.argtypes = [P, P, I, I, I, I64, I64, I64, I64, I64, F, F, P, I, F, I, F,
                                I64, P, P, P, P, P, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# Scalar and elementwise definitions (fp8_oracle.c)
# --------------------------------------------------------------------------

def decode(code: int, fmt: int) -> float:
    return float(_load().orc_decode(int(code), fmt))


def decode_array(codes: np.ndarray, fmt: int) -> np.ndarray:
    table = np.array([_load().orc_decode(c, fmt) for c in range(256)], np.float32)
    return table[np.asarray(codes, np.uint8)]


def encode(v: float, fmt: int) -> int:
    return int(_load().orc_encode(float(v), fmt))


def encode_array(v: np.ndarray, fmt: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_encode_array(_ptr(v), v.size, fmt, _ptr(out))
    return out


def encode_bits_range(first: int, n: int, fmt: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    _load().orc_encode_bits_range(first, n, fmt, _ptr(out))
    return out


def bf16_from_f64(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().orc_bf16_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def amax(x: np.ndarray) -> np.float32:
    """max |x_i| over the raw bf16 values ([CMP] quantize.cuh)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return np.float32(_load().orc_amax(_ptr(x), x.size))


def quantize_t(x: np.ndarray, fmt: int, s) -> tuple[np.ndarray, np.ndarray]:
    """Transposed / dual-orientation quantize of a bf16 [rows][cols] matrix
    ([CMP] quantize.cuh fp8_quantize_tiled_kernel, layouts Transposed and
    Dual; fp8.py _LinearFp8.backward feeds the NT GEMMs with them): the
    codes of quantize() in row-major order and their transpose
    ([cols][rows]).  amax is that of the untransposed values."""
    q = quantize(x, fmt, s)
    return q, np.ascontiguousarray(q.T)


IN_BF16, IN_F16, IN_F32 = 0, 1, 2


def _in_array(x: np.ndarray, in_type: int) -> np.ndarray:
    dt = np.float32 if in_type == IN_F32 else np.uint16
    return np.ascontiguousarray(x, dtype=dt)


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    """IEEE binary16 bits -> fp32, from the format's definition."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    lib = _load()
    return np.array([lib.orc_f16_to_f32(int(v)) for v in h.ravel()], np.float32).reshape(h.shape)


def amax_in(x: np.ndarray, in_type: int) -> np.float32:
    """max |x_i| over raw inputs of type in_type (0 bf16 bits, 1 fp16 bits,
    2 fp32) ([CMP] quantize.cuh quant_in_traits)."""
    x = _in_array(x, in_type)
    return np.float32(_load().orc_amax_in(_ptr(x), x.size, in_type))


def quantize_in(x: np.ndarray, in_type: int, fmt: int, s) -> np.ndarray:
    """q_i = encode(fp32(fp32(x_i) * fp32(1/s))) for any input type."""
    x = _in_array(x, in_type)
    out = np.empty(x.shape, np.uint8)
    _load().orc_quantize_in(_ptr(x), x.size, in_type, fmt, float(np.float32(s)), _ptr(out))
    return out


def scale_from_peak(peak, fmt: int, margin: int = 0) -> np.float32:
    """(peak / FP8_MAX) / 2^margin, clamped at 1e-12 ([CMP] FP8Recipe)."""
    return np.float32(_load().orc_scale_from_peak(float(np.float32(peak)), fmt, margin))


def multiplier(s) -> np.float32:
    return np.float32(_load().orc_multiplier(float(np.float32(s))))


def quantize(x: np.ndarray, fmt: int, s) -> np.ndarray:
    """q_i = encode(fp32(x_i * fp32(1/s))) ([CMP] fp8_quantize_kernel)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty(x.shape, np.uint8)
    _load().orc_quantize(_ptr(x), x.size, fmt, float(np.float32(s)), _ptr(out))
    return out


def gemm(a: np.ndarray, b: np.ndarray, fmt: int, trans_a: bool, trans_b: bool,
         M: int, N: int, K: int, sa, sb, bias: np.ndarray | None = None,
         batch: int = 1, stride_a: int | None = None, stride_b: int | None = None,
         lda: int | None = None, ldb: int | None = None) -> np.ndarray:
    """out[b,i,j] = bf16(sum_k A[b,i,k] B[b,k,j] * fp32(sa*sb) + bias[j]).

    ``a`` holds A as [M][K] (trans_a False) or [K][M] (trans_a True); ``b``
    holds B as [K][N] (trans_b False) or [N][K] (trans_b True).  A batch
    stride of 0 broadcasts that operand over the batch.
    """
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    if lda is None:
        lda = M if trans_a else K
    if ldb is None:
        ldb = K if trans_b else N
    if stride_a is None:
        stride_a = M * K
    if stride_b is None:
        stride_b = K * N
    out = np.empty((batch, M, N), np.uint16)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    _load().orc_gemm(_ptr(a), _ptr(b), fmt, int(trans_a), int(trans_b), M, N, K, lda,
                     ldb, batch, stride_a, stride_b, float(np.float32(sa)),
                     float(np.float32(sb)), _ptr(bias), _ptr(out))
    return out if batch > 1 else out[0]


def _gemm_dims(M, N, K, trans_a, trans_b, lda, ldb, stride_a, stride_b):
    if lda is None:
        lda = M if trans_a else K
    if ldb is None:
        ldb = K if trans_b else N
    if stride_a is None:
        stride_a = M * K
    if stride_b is None:
        stride_b = K * N
    return lda, ldb, stride_a, stride_b


def gemm_sampled(a, b, fmt, trans_a, trans_b, M, N, K, sa, sb, bias, samples,
                 batch=1, stride_a=None, stride_b=None, lda=None, ldb=None):
    """The same definition at sample coordinates ``samples`` = (bi, i, j).
    Returns (out, bound): the bf16 outputs and accumulation_bound() of each
    sample."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    lda, ldb, stride_a, stride_b = _gemm_dims(M, N, K, trans_a, trans_b, lda, ldb, stride_a,
                                              stride_b)
    bi, ii, jj = (np.ascontiguousarray(s, dtype=np.int64) for s in samples)
    n = bi.size
    out = np.empty(n, np.uint16)
    absdot = np.empty(n, np.float64)
    groupmax = np.empty(n, np.float64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    _load().orc_gemm_sampled(_ptr(a), _ptr(b), fmt, int(trans_a), int(trans_b), K, lda,
                             ldb, stride_a, stride_b, float(np.float32(sa)),
                             float(np.float32(sb)), _ptr(bias), n, _ptr(bi), _ptr(ii),
                             _ptr(jj), _ptr(out), _ptr(absdot), _ptr(groupmax))
    return out, accumulation_bound(absdot, groupmax, K)


def _gemm_stat(fn, a, b, fmt, trans_a, trans_b, M, N, K, sa, sb, batch, stride_a, stride_b,
               lda, ldb):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    lda, ldb, stride_a, stride_b = _gemm_dims(M, N, K, trans_a, trans_b, lda, ldb, stride_a,
                                              stride_b)
    out = np.empty((batch, M, N), np.float64)
    fn(_ptr(a), _ptr(b), fmt, int(trans_a), int(trans_b), M, N, K, lda, ldb, batch, stride_a,
       stride_b, float(np.float32(sa)), float(np.float32(sb)), _ptr(out))
    return out if batch > 1 else out[0]


def gemm_absdot(a, b, fmt, trans_a, trans_b, M, N, K, sa, sb, batch=1,
                stride_a=None, stride_b=None, lda=None, ldb=None) -> np.ndarray:
    """sum_k |A B| * |fp32(sa*sb)| per output: the scale of fp32 rounding."""
    return _gemm_stat(_load().orc_gemm_absdot, a, b, fmt, trans_a, trans_b, M, N, K, sa, sb,
                      batch, stride_a, stride_b, lda, ldb)


def gemm_groupmax(a, b, fmt, trans_a, trans_b, M, N, K, sa, sb, batch=1,
                  stride_a=None, stride_b=None, lda=None, ldb=None) -> np.ndarray:
    """sum over the aligned groups of 8 consecutive k of max |A B|, times
    |fp32(sa*sb)|, per output."""
    return _gemm_stat(_load().orc_gemm_groupmax, a, b, fmt, trans_a, trans_b, M, N, K, sa,
                      sb, batch, stride_a, stride_b, lda, ldb)


# Accumulation model of a correct fp8 GEMM on gfx950 (tolerance tooling, not
# the method): the matrix instructions add each aligned group of 8
# consecutive k after aligning its products to the largest one and keeping 13
# bits below that product's leading bit, so at most 7 products per group lose
# less than 2^-13 of the group's largest |product| each; the group sums and
# partial sums are then added in fp32 in some order (Higham: gamma_K times
# sum |products|).  Measured on crafted inputs by the GPU test of the model.
MFMA_GROUP = 8
MFMA_GROUP_CUT = 7 * 2.0 ** -13


def accumulation_bound(absdot, groupmax, K: int):
    """|kernel - exact| bound of a scaled fp8 dot product over K terms:
    MFMA_GROUP_CUT * groupmax + gamma_K * absdot, gamma_K = K u / (1 - K u),
    u = 2^-24 (absdot and groupmax already scaled by |s|)."""
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    return MFMA_GROUP_CUT * np.asarray(groupmax, np.float64) + gamma * np.asarray(
        absdot, np.float64)


def gemm_bound(a, b, fmt, trans_a, trans_b, M, N, K, sa, sb, batch=1,
               stride_a=None, stride_b=None, lda=None, ldb=None) -> np.ndarray:
    """accumulation_bound() of every output, [batch][M][N] (or [M][N])."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    lda, ldb, stride_a, stride_b = _gemm_dims(M, N, K, trans_a, trans_b, lda, ldb, stride_a,
                                              stride_b)
    absdot = np.empty((batch, M, N), np.float64)
    groupmax = np.empty((batch, M, N), np.float64)
    _load().orc_gemm_stats(_ptr(a), _ptr(b), fmt, int(trans_a), int(trans_b), M, N, K, lda,
                           ldb, batch, stride_a, stride_b, float(np.float32(sa)),
                           float(np.float32(sb)), _ptr(absdot), _ptr(groupmax))
    out = accumulation_bound(absdot, groupmax, K)
    return out if batch > 1 else out[0]


# Output types of gemm_ex: bf16, or fp8 codes of E4M3 / E5M2.
OUT_BF16, OUT_E4M3, OUT_E5M2 = 0, 1, 2


def out_codes(y: np.ndarray, out_type: int, out_scale) -> np.ndarray:
    """fp8 output codes of fp64 values y: enc(fp32(fp32(y) * fp32(1/out_scale)))
    in E4M3 (out_type OUT_E4M3) or E5M2 (OUT_E5M2), nearest even, saturating."""
    assert out_type in (OUT_E4M3, OUT_E5M2)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.uint8)
    _load().orc_out_code_array(_ptr(y), y.size, 0 if out_type == OUT_E4M3 else 1,
                               float(np.float32(out_scale)), _ptr(out))
    return out


def gemm_ex(a, b, fmt, trans_a, trans_b, M, N, K, sa, sb, bias=None, bias_scale=None,
            out_type=OUT_BF16, out_scale=None, samples=None, batch=1, stride_a=None,
            stride_b=None, lda=None, ldb=None):
    """GEMM with an fp8 bias (``bias`` uint8 codes of ``fmt`` and a float
    ``bias_scale``) or a bf16 one (uint16 bits, no scale), and a bf16 or fp8
    output ([CMP] the removed fp8_gemm op; [LOG1] bias_scale):

        y   = sum_k A B * fp32(sa*sb) + bias value   (fp64)
        out = bf16(y), or enc(fp32(fp32(y) * fp32(1/out_scale)))

    At ``samples`` = (bi, i, j) coordinates, else at every output in
    [batch][M][N] order.  Returns (out, y, bound) as flat arrays, bound the
    accumulation_bound() of each output."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    if lda is None:
        lda = M if trans_a else K
    if ldb is None:
        ldb = K if trans_b else N
    if stride_a is None:
        stride_a = M * K
    if stride_b is None:
        stride_b = K * N
    if samples is None:
        bi, ii, jj = (np.ascontiguousarray(v.ravel(), dtype=np.int64)
                      for v in np.indices((batch, M, N)))
    else:
        bi, ii, jj = (np.ascontiguousarray(v, dtype=np.int64) for v in samples)
    n = bi.size
    bias_fp8 = bias_scale is not None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint8 if bias_fp8 else np.uint16)
    assert out_type == OUT_BF16 or out_scale is not None, "an fp8 output needs out_scale"
    out = np.empty(n, np.uint16 if out_type == OUT_BF16 else np.uint8)
    y = np.empty(n, np.float64)
    absdot = np.empty(n, np.float64)
    groupmax = np.empty(n, np.float64)
    _load().orc_gemm_ex(_ptr(a), _ptr(b), fmt, int(trans_a), int(trans_b), K, lda, ldb,
                        stride_a, stride_b, float(np.float32(sa)), float(np.float32(sb)),
                        _ptr(bias), int(bias_fp8),
                        float(np.float32(bias_scale if bias_fp8 else 0.0)), out_type,
                        float(np.float32(out_scale if out_scale is not None else 1.0)), n,
                        _ptr(bi), _ptr(ii), _ptr(jj), _ptr(out), _ptr(y), _ptr(absdot),
                        _ptr(groupmax))
    return out, y, accumulation_bound(absdot, groupmax, K)


def colsum(g: np.ndarray, M: int, N: int) -> np.ndarray:
    """db[j] = bf16(sum_m g[m, j]) ([CMP] _LinearFp8.backward grad_b)."""
    g = np.ascontiguousarray(g, dtype=np.uint16)
    out = np.empty(N, np.uint16)
    _load().orc_colsum(_ptr(g), M, N, _ptr(out))
    return out


# --------------------------------------------------------------------------
# Delayed-scaling state ([CMP] fp8.py _ScaleRing; quantize.cuh publish_amax)
# --------------------------------------------------------------------------

@dataclass
class Ring:
    """One operand's amax history: window ``hist``, published ``scale``,
    host-side slot ``idx`` and the ``initialized`` flag."""

    n: int = 16
    margin: int = 0
    hist: np.ndarray = field(default=None)
    scale: np.float32 = np.float32(0.0)
    idx: int = 0
    initialized: bool = False

    def __post_init__(self):
        if self.hist is None:
            self.hist = np.zeros(self.n, np.float32)

    def fold(self, a, fmt: int) -> None:
        """Record amax in the current slot, publish the next scale from the
        window's max (the quantize kernel's last-block step)."""
        self.hist[self.idx] = np.float32(a)
        peak = np.float32(self.hist.max())
        self.scale = scale_from_peak(peak, fmt, self.margin)

    def seed(self, x: np.ndarray, fmt: int) -> None:
        """First use: measure the tensor and fold it (reading of seed())."""
        self.fold(amax(x), fmt)
        self.initialized = True

    def advance(self) -> None:
        self.idx = (self.idx + 1) % self.n

    def state(self) -> np.ndarray:
        """The fp32 state buffer [hist n | scale | legacy | amax | done]
        after a launch (the amax and done slots are cleaned to zero)."""
        s = np.zeros(self.n + 4, np.float32)
        s[: self.n] = self.hist
        s[self.n] = self.scale
        return s


# --------------------------------------------------------------------------
# Linear layer ([CMP] fp8.py fp8_linear_forward, _LinearFp8.backward)
# --------------------------------------------------------------------------

@dataclass
class FwdResult:
    out: np.ndarray
    sx: np.float32
    sw: np.float32
    x8: np.ndarray
    w8: np.ndarray


def linear_fwd(x, w, bias, M, N, K, fmt, dynamic, ring_x: Ring | None = None,
               ring_w: Ring | None = None, margin: int = 0) -> FwdResult:
    """out = x w^T * (sx*sw) + bias, with x [M,K], w [N,K] bf16.

    Dynamic: sx, sw come from the current amax.  Delayed: the rings are
    seeded on first use, their scales are snapshotted, x and w are quantized
    with the snapshots while the in-kernel fold records the current amax and
    publishes the next scale; the GEMM dequantizes with the snapshots; the
    slots advance.
    """
    if dynamic:
        sx = scale_from_peak(amax(x), fmt, margin)
        sw = scale_from_peak(amax(w), fmt, margin)
        x8 = quantize(x, fmt, sx)
        w8 = quantize(w, fmt, sw)
    else:
        if not ring_w.initialized:
            ring_w.seed(w, fmt)
        if not ring_x.initialized:
            ring_x.seed(x, fmt)
        sx, sw = np.float32(ring_x.scale), np.float32(ring_w.scale)  # snapshot
        x8 = quantize(x, fmt, sx)
        ring_x.fold(amax(x), fmt)
        w8 = quantize(w, fmt, sw)
        ring_w.fold(amax(w), fmt)
    out = gemm(x8, w8, fmt, False, True, M, N, K, sx, sw, bias)
    if not dynamic:
        ring_x.advance()
        ring_w.advance()
    return FwdResult(out, sx, sw, x8, w8)


@dataclass
class BwdResult:
    dx: np.ndarray | None
    dw: np.ndarray | None
    db: np.ndarray | None
    sg: np.float32
    sx: np.float32
    sw: np.float32
    g8: np.ndarray


def linear_bwd(g, x, w, M, N, K, fmt, dynamic, sx_fwd=None, sw_fwd=None,
               ring_g: Ring | None = None, need_dx=True, need_dw=True, need_db=True,
               margin: int = 0) -> BwdResult:
    """dX = g w * (sg*sw) (NN), dW = g^T x * (sg*sx) (TN), db = colsum(g).

    g [M,N], x [M,K], w [N,K] bf16; every operand is quantized in the
    backward format ``fmt``.  Delayed: sg is the g ring's snapshot (seeded
    on first use), sx and sw are the forward's snapshots.  Dynamic: sg, sx,
    sw are measured now in the backward format.
    """
    if dynamic:
        sg = scale_from_peak(amax(g), fmt, margin)
        sx = scale_from_peak(amax(x), fmt, margin)
        sw = scale_from_peak(amax(w), fmt, margin)
        g8 = quantize(g, fmt, sg)
    else:
        if not ring_g.initialized:
            ring_g.seed(g, fmt)
        sg = np.float32(ring_g.scale)  # snapshot before the fold publishes
        sx, sw = np.float32(sx_fwd), np.float32(sw_fwd)
        g8 = quantize(g, fmt, sg)
        ring_g.fold(amax(g), fmt)
    dx = dw = db = None
    if need_dx:
        w8 = quantize(w, fmt, sw)
        dx = gemm(g8, w8, fmt, False, False, M, K, N, sg, sw)       # NN
    if need_dw:
        x8 = quantize(x, fmt, sx)
        dw = gemm(g8, x8, fmt, True, False, N, K, M, sg, sx)        # TN
    if need_db:
        db = colsum(g, M, N)
    if not dynamic:
        ring_g.advance()
    return BwdResult(dx, dw, db, sg, sx, sw, g8)
