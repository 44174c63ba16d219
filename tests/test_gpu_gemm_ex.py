"""GPU parity of fp8_mm_ex (fp8 bias, fp8 output) against the CPU oracle.

fp8 output codes are checked with check_fp8_codes: each code lies between
the codes of the oracle's exact value minus and plus the fp32 accumulation
bound, and almost all equal the code of the exact value.  bf16 outputs with
an fp8 bias use check_gemm.  Shapes reach every kernel the dispatcher
picks (256, 128 and 64 tiles, the short-A kernel, the general fallback),
both store forms (whole 16-byte rows through LDS, 4-element stores, ragged
tails), every layout and both formats; the square 4096 configuration is
checked at sampled coordinates.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import (check_fp8_codes, check_gemm, chosen_tile_config, dev_f32,
                            from_dev_bf16, from_dev_u8, to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
OUT_BF16, OUT_E4M3, OUT_E5M2 = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    import fp8_tensor_scaled_amd as f
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return f


def prequant(orc, x_bits, fmt):
    s = orc.scale_from_peak(orc.amax(x_bits), fmt)
    return orc.quantize(x_bits, fmt, s), s


def storage(mat, trans):
    return np.ascontiguousarray(np.swapaxes(mat, -1, -2) if trans else mat)


def run_mm_ex(lib, a_st, b_st, fmt, ta, tb, M, N, K, sa, sb, bias=None, bias_scale=None,
              out_type=OUT_E4M3, out_scale=None, batch=1, stride_b=None, out_shift=0):
    """One fp8_mm_ex call; out_shift > 0 offsets the output by that many
    elements from a 256-byte boundary (misaligned stores)."""
    lda = M if ta else K
    ldb = K if tb else N
    stride_b = K * N if stride_b is None else stride_b
    ad, bd = to_dev_u8(a_st.ravel()), to_dev_u8(b_st.ravel())
    n_out = batch * M * N
    if out_type == OUT_BF16:
        buf = torch.full((n_out + out_shift,), 0x7FC1, dtype=torch.int16, device="cuda")
    else:
        buf = torch.full((n_out + out_shift,), 0x7F, dtype=torch.uint8, device="cuda")
    out = buf[out_shift:]
    bd_ = None
    if bias is not None:
        bd_ = to_dev_u8(bias) if bias_scale is not None else to_dev_bf16(bias)
    lib.fp8_mm_ex(ad, bd, fmt, ta, tb, M, N, K, lda, ldb, batch, M * K, stride_b, dev_f32(sa),
                  dev_f32(sb), bd_, None if bias_scale is None else dev_f32(bias_scale),
                  out_type, None if out_scale is None else dev_f32(out_scale), out)
    torch.cuda.synchronize()
    return from_dev_bf16(out) if out_type == OUT_BF16 else from_dev_u8(out)


def make_bias(orc, kind, N, fmt, seed):
    """(bias, bias_scale): none, bf16, or fp8 codes with their step."""
    if kind == "none":
        return None, None
    b = wl.normal_bf16((N,), 0.5, seed)
    if kind == "bf16":
        return b, None
    b8, s = prequant(orc, b, fmt)
    return b8, s


def out_step(orc, y, out_type, headroom=1.0):
    """A delayed-scaling-like output step from the values' peak (headroom
    < 1 makes the largest outputs saturate)."""
    fo = E4M3 if out_type == OUT_E4M3 else E5M2
    return orc.scale_from_peak(np.float32(np.abs(y).max() * headroom), fo)


SHAPES = [
    (272, 304, 400),   # 128 tiles (m > 64), ragged m, n % 16 == 0
    (512, 520, 256),   # 128 tiles, n % 16 == 8: 4-element stores
    (48, 80, 112),     # 64 tiles (short m, not NT) / short-A kernel (NT)
    (33, 17, 100),     # general fallback (k % 16 != 0), ragged everything
    (5, 300, 64),      # short-A kernel (NT), ragged n
]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("ta,tb", [(0, 1), (0, 0), (1, 0)], ids=["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_type", [OUT_E4M3, OUT_E5M2])
def test_mm_ex_fp8_out_full_compare(lib, orc, fmt, ta, tb, M, N, K, out_type):
    a8, sa = prequant(orc, wl.normal_bf16((M, K), 1.0, M + 3 * K), fmt)
    b8, sb = prequant(orc, wl.normal_bf16((K, N), 1.0, N + 5 * K), fmt)
    kind = ("none", "bf16", "fp8")[(M + N + out_type) % 3]
    bias, bs = make_bias(orc, kind, N, fmt, N + 7)
    A, B = storage(a8, ta), storage(b8, tb)
    _, y, _ = orc.gemm_ex(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias, bs)
    so = out_step(orc, y, out_type, headroom=0.8)
    ref, y, bound = orc.gemm_ex(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias, bs,
                                 out_type, so)
    got = run_mm_ex(lib, A, B, fmt, ta, tb, M, N, K, sa, sb, bias, bs, out_type, so)
    check_fp8_codes(orc, got, y, bound, out_type, so,
                    f"{M}x{N}x{K} t{ta}{tb} f{fmt} o{out_type} bias {kind}")
    # saturation: the largest outputs (above the step's range) give +-max
    fo_max = 0x7E if out_type == OUT_E4M3 else 0x7B
    big = np.abs(y) * np.float64(orc.multiplier(so)) > (448.0 if out_type == OUT_E4M3
                                                         else 57344.0) * 1.01
    assert ((got[big] & 0x7F) == fo_max).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("ta,tb", [(0, 1), (0, 0), (1, 0)], ids=["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", [(272, 304, 400), (33, 17, 100), (5, 300, 64)])
def test_mm_ex_fp8_bias_bf16_out(lib, orc, fmt, ta, tb, M, N, K):
    a8, sa = prequant(orc, wl.normal_bf16((M, K), 1.0, M + 11 * K), fmt)
    b8, sb = prequant(orc, wl.normal_bf16((K, N), 1.0, N + 13 * K), fmt)
    bias, bs = make_bias(orc, "fp8", N, fmt, N + 17)
    A, B = storage(a8, ta), storage(b8, tb)
    ref, _, bound = orc.gemm_ex(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias, bs)
    got = run_mm_ex(lib, A, B, fmt, ta, tb, M, N, K, sa, sb, bias, bs, OUT_BF16, None)
    check_gemm(got.reshape(M, N), ref.reshape(M, N), bound.reshape(M, N),
               f"fp8 bias {M}x{N}x{K} t{ta}{tb} f{fmt}")


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mm_ex_fp8_bias_every_code(lib, orc, fmt):
    """A = 0: the output is the bias value alone, so every finite fp8 code
    goes through the kernel's decode, its step and the bf16 rounding (the
    oracle's exact result: one rounding of an fp32 value)."""
    M, K = 64, 128
    codes = np.arange(256, dtype=np.uint8)
    finite = ~(((codes & 0x7F) == 0x7F) if fmt == E4M3 else ((codes & 0x7C) == 0x7C))
    bias = codes[finite]
    N = bias.size
    A = np.zeros((M, K), np.uint8)
    B = wl.random_codes((N, K), fmt, 5)
    bs = np.float32(0.3)
    for M_ in (M, 300):  # short-A kernel, then the tiled kernels
        A = np.zeros((M_, K), np.uint8)
        ref, _, _ = orc.gemm_ex(A, B, fmt, False, True, M_, N, K, 1.0, 1.0, bias, bs)
        got = run_mm_ex(lib, A, B, fmt, 0, 1, M_, N, K, 1.0, 1.0, bias, bs, OUT_BF16, None)
        assert np.array_equal(got, ref), M_


def test_mm_ex_plain_form_is_fp8_mm(lib, orc):
    """No bias step and a bf16 output: the plain kernels, the same bits."""
    M, N, K = 512, 512, 512
    a8 = wl.random_codes((M, K), E4M3, 61)
    b8 = wl.random_codes((N, K), E4M3, 62)
    bias = wl.normal_bf16((N,), 0.5, 63)
    got = run_mm_ex(lib, a8, b8, E4M3, 0, 1, M, N, K, 0.5, 0.25, bias, None, OUT_BF16, None)
    out = torch.empty(M * N, dtype=torch.int16, device="cuda")
    lib.fp8_mm(to_dev_u8(a8), to_dev_u8(b8), E4M3, 0, 1, M, N, K, K, K, 1, 0, 0, dev_f32(0.5),
               dev_f32(0.25), to_dev_bf16(bias), out)
    torch.cuda.synchronize()
    assert np.array_equal(got, from_dev_bf16(out))


@pytest.mark.parametrize("shift", [1, 4, 8])
def test_mm_ex_misaligned_output(lib, orc, shift):
    """Output not 16-byte aligned: the direct store forms."""
    fmt, M, N, K = E4M3, 256, 272, 256
    a8, sa = prequant(orc, wl.normal_bf16((M, K), 1.0, 71), fmt)
    b8, sb = prequant(orc, wl.normal_bf16((N, K), 1.0, 72), fmt)
    bias, bs = make_bias(orc, "fp8", N, fmt, 73)
    _, y, _ = orc.gemm_ex(a8, b8, fmt, False, True, M, N, K, sa, sb, bias, bs)
    so = out_step(orc, y, OUT_E4M3)
    ref, y, bound = orc.gemm_ex(a8, b8, fmt, False, True, M, N, K, sa, sb, bias, bs,
                                 OUT_E4M3, so)
    got = run_mm_ex(lib, a8, b8, fmt, 0, 1, M, N, K, sa, sb, bias, bs, OUT_E4M3, so,
                    out_shift=shift)
    check_fp8_codes(orc, got, y, bound, OUT_E4M3, so, f"misaligned by {shift}")


def test_mm_ex_batched_broadcast(lib, orc):
    fmt, batch, M, N, K = E5M2, 3, 96, 160, 192
    a8, sa = prequant(orc, wl.normal_bf16((batch, M, K), 1.0, 81), fmt)
    b8, sb = prequant(orc, wl.normal_bf16((N, K), 1.0, 82), fmt)  # broadcast [N][K]
    _, y, _ = orc.gemm_ex(a8, b8, fmt, False, True, M, N, K, sa, sb, batch=batch, stride_b=0)
    so = out_step(orc, y, OUT_E4M3)
    ref, y, bound = orc.gemm_ex(a8, b8, fmt, False, True, M, N, K, sa, sb, out_type=OUT_E4M3,
                                 out_scale=so, batch=batch, stride_b=0)
    got = run_mm_ex(lib, a8, b8, fmt, 0, 1, M, N, K, sa, sb, None, None, OUT_E4M3, so,
                    batch=batch, stride_b=0)
    check_fp8_codes(orc, got, y, bound, OUT_E4M3, so, "batched broadcast")


# The extended epilogue on the 128 x 256 and 256 x 128 tiles, ragged in m, n
# and k (these shapes take those configurations: least rounds of 256 tiles
# x tile time), every output: fp8 codes out with an fp8 bias, and bf16 out
# with an fp8 bias.
HALF_TILES = [("wide", 0, 1, 2032, 4080, 272), ("tall", 0, 0, 4084, 2032, 272),
              ("wide", 1, 0, 2032, 4080, 272), ("tall", 0, 1, 4084, 2036, 272)]


@pytest.mark.parametrize("cfg,ta,tb,M,N,K", HALF_TILES,
                         ids=[f"{c[0]}-t{c[1]}{c[2]}" for c in HALF_TILES])
def test_mm_ex_half_tiles_full_compare(lib, orc, cfg, ta, tb, M, N, K):
    assert chosen_tile_config(M, N) == cfg
    fmt = E4M3 if (ta, tb) == (0, 1) else E5M2
    a8, sa = prequant(orc, wl.normal_bf16((M, K), 1.0, 61 + ta), fmt)
    b8, sb = prequant(orc, wl.normal_bf16((K, N), 1.0, 62 + tb), fmt)
    bias, bs = make_bias(orc, "fp8", N, fmt, 63)
    A, B = storage(a8, ta), storage(b8, tb)
    ref, y, bound = orc.gemm_ex(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias, bs)
    got = run_mm_ex(lib, A, B, fmt, ta, tb, M, N, K, sa, sb, bias, bs, OUT_BF16, None)
    check_gemm(got.reshape(M, N), ref.reshape(M, N), bound.reshape(M, N),
               f"{cfg} fp8 bias {M}x{N}x{K} t{ta}{tb}")
    out_type = OUT_E4M3 if ta == 0 else OUT_E5M2
    so = out_step(orc, y, out_type, headroom=0.8)
    ref, y, bound = orc.gemm_ex(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias, bs,
                                 out_type, so)
    got = run_mm_ex(lib, A, B, fmt, ta, tb, M, N, K, sa, sb, bias, bs, out_type, so)
    check_fp8_codes(orc, got, y, bound, out_type, so, f"{cfg} {M}x{N}x{K} t{ta}{tb} o{out_type}")


@pytest.mark.parametrize("ta,tb,out_type", [(0, 1, OUT_E4M3), (0, 1, OUT_E5M2),
                                             (0, 0, OUT_E4M3), (1, 0, OUT_E5M2)],
                         ids=["NT-e4m3", "NT-e5m2", "NN-e4m3", "TN-e5m2"])
def test_config_square_4096_fp8_out(lib, orc, ta, tb, out_type):
    """The square 4096 configuration (E4M3 operands, fp8 bias) with an fp8
    output on the 256-tile kernels, sampled.  The two draws are taken as
    the operands' storage in the layout under test."""
    d = wl.square(4096)
    n = 4096
    a8, sa = prequant(orc, d["a"], E4M3)
    b8, sb = prequant(orc, d["b"], E4M3)
    bias, bs = make_bias(orc, "fp8", n, E4M3, 91)
    rng = np.random.default_rng(3)
    s = (np.zeros(3004, np.int64), np.concatenate([rng.integers(0, n, 3000), [0, n - 1, 0, n - 1]]),
         np.concatenate([rng.integers(0, n, 3000), [0, n - 1, n - 1, 0]]))
    _, y, _ = orc.gemm_ex(a8, b8, E4M3, bool(ta), bool(tb), n, n, n, sa, sb, bias, bs,
                          samples=s)
    so = out_step(orc, y, out_type, headroom=1.25)
    ref, y, bound = orc.gemm_ex(a8, b8, E4M3, bool(ta), bool(tb), n, n, n, sa, sb, bias, bs,
                                 out_type, so, samples=s)
    got = run_mm_ex(lib, a8, b8, E4M3, ta, tb, n, n, n, sa, sb, bias, bs, out_type, so)
    got = got.reshape(n, n)[s[1], s[2]]
    check_fp8_codes(orc, got, y, bound, out_type, so, f"square 4096 t{ta}{tb} o{out_type}")
