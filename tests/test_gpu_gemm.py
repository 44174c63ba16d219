"""GPU parity of fp8_mm against the CPU oracle.

Small problems are compared element by element over the whole output
(several tiles plus ragged tails, every layout, both formats, batched and
broadcast operands, with and without bias).  The configurations' full sizes
are run in the same launch configuration the benchmark uses and compared at
sampled output coordinates the oracle evaluates one by one.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import check_gemm, dev_f32, from_dev_bf16, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def lib():
    import fp8_tensor_scaled_amd as f
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return f


def prequant(orc, x_bits, fmt):
    """Operands 'pre-quantized from bf16 with per-tensor scales': dynamic
    scale from the tensor's amax, oracle quantize."""
    s = orc.scale_from_peak(orc.amax(x_bits), fmt)
    return orc.quantize(x_bits, fmt, s), s


def storage(mat, trans):
    """[..., r, c] logical matrix -> its storage (transposed if trans)."""
    return np.ascontiguousarray(np.swapaxes(mat, -1, -2) if trans else mat)


def run_mm(lib, a_st, b_st, fmt, ta, tb, M, N, K, sa, sb, bias=None, batch=1, stride_a=None,
           stride_b=None, lda=None, ldb=None):
    if lda is None:
        lda = M if ta else K
    if ldb is None:
        ldb = K if tb else N
    if stride_a is None:
        stride_a = M * K
    if stride_b is None:
        stride_b = K * N
    ad, bd = to_dev_u8(a_st.ravel()), to_dev_u8(b_st.ravel())
    out = torch.full((batch * M * N,), 0x7FC1, dtype=torch.int16, device="cuda")
    lib.fp8_mm(ad, bd, fmt, ta, tb, M, N, K, lda, ldb, batch, stride_a, stride_b, dev_f32(sa),
               dev_f32(sb), None if bias is None else to_dev_bf16(bias), out)
    torch.cuda.synchronize()
    return from_dev_bf16(out).reshape((batch, M, N) if batch > 1 else (M, N))


LAYOUTS = [(0, 1), (0, 0), (1, 0), (1, 1)]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=["NT", "NN", "TN", "TT"])
@pytest.mark.parametrize("M,N,K", [(272, 304, 400), (64, 512, 256), (512, 256, 1024),
                                   (48, 80, 112), (33, 17, 100), (1, 1, 1), (5, 300, 7)])
def test_mm_small_full_compare(lib, orc, fmt, ta, tb, M, N, K):
    a_bits = wl.normal_bf16((M, K), 1.0, M * 7 + K)
    b_bits = wl.normal_bf16((K, N), 1.0, N * 11 + K)  # logical B [K][N]
    a8, sa = prequant(orc, a_bits, fmt)
    b8, sb = prequant(orc, b_bits, fmt)
    bias = wl.normal_bf16((N,), 0.1, N) if (M + N) % 2 else None
    got = run_mm(lib, storage(a8, ta), storage(b8, tb), fmt, ta, tb, M, N, K, sa, sb, bias)
    ref = orc.gemm(storage(a8, ta), storage(b8, tb), fmt, bool(ta), bool(tb), M, N, K, sa, sb,
                   bias)
    absdot = orc.gemm_absdot(storage(a8, ta), storage(b8, tb), fmt, bool(ta), bool(tb), M, N,
                             K, sa, sb)
    check_gemm(got, ref, absdot, K, f"{M}x{N}x{K} t{ta}{tb} f{fmt}")


@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=["NT", "NN", "TN", "TT"])
def test_mm_padded_leading_dims(lib, orc, ta, tb):
    """Row strides larger than the logical width (16-aligned: tiled path;
    odd: general path)."""
    M, N, K = 96, 160, 256
    for pad in (16, 3):
        a8 = wl.random_codes((M, K), E4M3, 1)
        b8 = wl.random_codes((K, N), E4M3, 2)
        a_st, b_st = storage(a8, ta), storage(b8, tb)
        a_pad = np.zeros((a_st.shape[0], a_st.shape[1] + pad), np.uint8)
        a_pad[:, : a_st.shape[1]] = a_st
        b_pad = np.zeros((b_st.shape[0], b_st.shape[1] + pad), np.uint8)
        b_pad[:, : b_st.shape[1]] = b_st
        got = run_mm(lib, a_pad, b_pad, E4M3, ta, tb, M, N, K, 0.01, 0.02,
                     lda=a_pad.shape[1], ldb=b_pad.shape[1])
        ref = orc.gemm(a_pad, b_pad, E4M3, bool(ta), bool(tb), M, N, K, 0.01, 0.02,
                       lda=a_pad.shape[1], ldb=b_pad.shape[1])
        absdot = orc.gemm_absdot(a_pad, b_pad, E4M3, bool(ta), bool(tb), M, N, K, 0.01, 0.02,
                                 lda=a_pad.shape[1], ldb=b_pad.shape[1])
        check_gemm(got, ref, absdot, K, f"pad{pad}", max_frac=1e-2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mm_batched_and_broadcast_small(lib, orc, fmt):
    batch, M, N, K = 3, 144, 208, 384
    a8 = wl.random_codes((batch, M, K), fmt, 5)
    b8 = wl.random_codes((batch, N, K), fmt, 6)
    b1 = wl.random_codes((N, K), fmt, 7)
    a1 = wl.random_codes((M, K), fmt, 8)
    sa, sb = np.float32(1e-3), np.float32(2e-3)
    cases = [(a8, b8, M * K, N * K), (a8, b1, M * K, 0), (a1, b8, 0, N * K)]
    for a, b, stra, strb in cases:
        got = run_mm(lib, a, b, fmt, 0, 1, M, N, K, sa, sb, batch=batch, stride_a=stra,
                     stride_b=strb)
        ref = orc.gemm(a, b, fmt, False, True, M, N, K, sa, sb, batch=batch, stride_a=stra,
                       stride_b=strb)
        absdot = orc.gemm_absdot(a, b, fmt, False, True, M, N, K, sa, sb, batch=batch,
                                 stride_a=stra, stride_b=strb)
        check_gemm(got, ref, absdot, K, f"batched {stra} {strb}", max_frac=1e-2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("M,N,K", [(64, 8200, 2064), (17, 96, 4112), (32, 256, 64),
                                   (1, 40, 16), (48, 264, 1040), (64, 33, 8192)])
def test_mm_short_a_edges(lib, orc, fmt, M, N, K):
    """NT with m <= 64 (the short-A kernel): k ranges that split unevenly over
    the waves (some get none), a partial last k step, ragged n, a single row."""
    a8 = wl.random_codes((M, K), fmt, M + K)
    b8 = wl.random_codes((N, K), fmt, N + K)
    sa, sb = np.float32(2.0 ** -9), np.float32(3e-3)
    bias = wl.normal_bf16((N,), 0.1, N + 1)
    got = run_mm(lib, a8, b8, fmt, 0, 1, M, N, K, sa, sb, bias)
    ref = orc.gemm(a8, b8, fmt, False, True, M, N, K, sa, sb, bias)
    absdot = orc.gemm_absdot(a8, b8, fmt, False, True, M, N, K, sa, sb)
    check_gemm(got, ref, absdot, K, f"short-A {M}x{N}x{K} f{fmt}", max_frac=1e-2)


def test_mm_short_a_batched(lib, orc):
    """Short A with per-batch A and broadcast B (stride 0), and the reverse."""
    batch, M, N, K = 3, 40, 200, 528
    a8 = wl.random_codes((batch, M, K), E4M3, 60)
    b8 = wl.random_codes((batch, N, K), E4M3, 61)
    b1 = wl.random_codes((N, K), E4M3, 62)
    a1 = wl.random_codes((M, K), E4M3, 63)
    for a, b, stra, strb in [(a8, b8, M * K, N * K), (a8, b1, M * K, 0), (a1, b8, 0, N * K)]:
        got = run_mm(lib, a, b, E4M3, 0, 1, M, N, K, 1e-3, 1e-3, batch=batch, stride_a=stra,
                     stride_b=strb)
        ref = orc.gemm(a, b, E4M3, False, True, M, N, K, 1e-3, 1e-3, batch=batch,
                       stride_a=stra, stride_b=strb)
        absdot = orc.gemm_absdot(a, b, E4M3, False, True, M, N, K, 1e-3, 1e-3, batch=batch,
                                 stride_a=stra, stride_b=strb)
        check_gemm(got, ref, absdot, K, f"short-A batched {stra} {strb}", max_frac=1e-2)


def test_mm_extreme_codes(lib, orc):
    """Random codes over the whole E4M3 / E5M2 range (max, subnormals, zeros)."""
    for fmt in (E4M3, E5M2):
        M, N, K = 128, 128, 512
        a8 = wl.random_codes((M, K), fmt, 40)
        b8 = wl.random_codes((N, K), fmt, 41)
        got = run_mm(lib, a8, b8, fmt, 0, 1, M, N, K, 1.0, 1.0)
        ref = orc.gemm(a8, b8, fmt, False, True, M, N, K, 1.0, 1.0)
        absdot = orc.gemm_absdot(a8, b8, fmt, False, True, M, N, K, 1.0, 1.0)
        check_gemm(got, ref, absdot, K, f"extreme f{fmt}", max_frac=1e-2)


def test_mm_deterministic(lib, orc):
    M, N, K = 512, 512, 1024
    a8 = wl.random_codes((M, K), E4M3, 50)
    b8 = wl.random_codes((N, K), E4M3, 51)
    x = run_mm(lib, a8, b8, E4M3, 0, 1, M, N, K, 0.5, 0.5)
    y = run_mm(lib, a8, b8, E4M3, 0, 1, M, N, K, 0.5, 0.5)
    assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# Full-size configurations, sampled outputs
# ---------------------------------------------------------------------------

def sample_coords(batch, M, N, n, seed):
    rng = np.random.default_rng(seed)
    bi = rng.integers(0, batch, n)
    ii = rng.integers(0, M, n)
    jj = rng.integers(0, N, n)
    # always include the corners of the output (tails of every tiling)
    bi = np.concatenate([bi, [0, batch - 1, 0, batch - 1]])
    ii = np.concatenate([ii, [0, M - 1, M - 1, 0]])
    jj = np.concatenate([jj, [0, N - 1, 0, N - 1]])
    return bi, ii, jj


def full_size_case(lib, orc, a_bits, b_bits, fmt, M, N, K, batch=1, bias=None, bcast_b=False,
                   n_samples=3000, seed=0):
    a8, sa = prequant(orc, a_bits, fmt)
    b8, sb = prequant(orc, b_bits, fmt)  # b stored [N][K] (NT)
    stride_b = 0 if bcast_b else N * K
    got = run_mm(lib, a8, b8, fmt, 0, 1, M, N, K, sa, sb, bias, batch=batch, stride_b=stride_b)
    got3 = got.reshape(batch, M, N)
    s = sample_coords(batch, M, N, n_samples, seed)
    ref, absdot = orc.gemm_sampled(a8, b8, fmt, False, True, M, N, K, sa, sb, bias, s,
                                   batch=batch, stride_b=stride_b)
    return check_gemm(got3[s], ref, absdot, K, f"full {batch}x{M}x{N}x{K}")


def test_config_smallm(lib, orc):
    d = wl.smallm()
    full_size_case(lib, orc, d["x"], d["w"], E4M3, 64, 8192, 2048)


@pytest.mark.parametrize("n", [4096, 8192])
def test_config_square(lib, orc, n):
    d = wl.square(n)
    # B stored [N][K]: the second draw is the weight-layout operand
    full_size_case(lib, orc, d["a"], d["b"], E4M3, n, n, n, bias=d["bias"])


def test_config_bmm8(lib, orc):
    d = wl.bmm8()  # the [2048,2048] draws are taken as the [N][K] (NT) storage
    full_size_case(lib, orc, d["a"], d["b"], E4M3, 1024, 2048, 2048, batch=8)


def test_config_bmm64(lib, orc):
    d = wl.bmm64()
    full_size_case(lib, orc, d["a"], d["b"], E4M3, 512, 512, 512, batch=64)


def test_config_bcast8(lib, orc):
    d = wl.bcast8()
    full_size_case(lib, orc, d["a"], d["b"], E4M3, 1024, 2048, 2048, batch=8, bcast_b=True)


def test_mfma_group_precision(lib, orc):
    """Evidence for the accumulation model behind the tolerance fallback:
    with +1024 and -1024 products in the same group of 8 consecutive k, the
    other 6 products of that group (each 2^-4, 14 bits below) are cut, while
    the 120 products in other groups are summed exactly."""
    M = N = 16
    K = 128
    vals_a = np.zeros((M, K), np.float32)
    vals_b = np.zeros((N, K), np.float32)
    vals_a[0, 0], vals_b[0, 0] = 32.0, 32.0
    vals_a[0, 1], vals_b[0, 1] = -32.0, 32.0
    vals_a[0, 2:], vals_b[0, 2:] = 0.25, 0.25  # 2^-4 each
    a8 = orc.encode_array(vals_a, E4M3)
    b8 = orc.encode_array(vals_b, E4M3)
    got = run_mm(lib, a8, b8, E4M3, 0, 1, M, N, K, 1.0, 1.0)
    ref = orc.gemm(a8, b8, E4M3, False, True, M, N, K, 1.0, 1.0)
    y0 = wl.bf16_bits_to_f32(got[0, 0])
    assert wl.bf16_bits_to_f32(ref[0, 0]) == 126 * 2.0 ** -4
    assert y0 == 120 * 2.0 ** -4, y0
    absdot = orc.gemm_absdot(a8, b8, E4M3, False, True, M, N, K, 1.0, 1.0)
    assert abs(y0 - 126 * 2.0 ** -4) <= 2.0 ** -10 * absdot[0, 0]


# ---------------------------------------------------------------------------
# Two independent products from one call (the backward's dX and dW)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (4144, 4176, 272), (256, 512, 320)])
def test_mm_pair_matches_two_calls(lib, orc, fmt, M, N, K):
    """fp8_mm_pair of an NN and a TN product gives the bits of two fp8_mm
    calls: through the paired kernel when both have at least 256 tiles of
    256 x 256 (the first two shapes, the second with ragged tails), as two
    launches otherwise; and it matches the oracle at sampled coordinates."""
    # problem 0, NN: A [M][K], B [K][N]; problem 1, TN: A stored [K][M], B [K][N]
    a0, sa0 = prequant(orc, wl.normal_bf16((M, K), 1.0, 700 + K), fmt)
    b0, sb0 = prequant(orc, wl.normal_bf16((K, N), 0.02, 701 + K), fmt)
    a1, sa1 = prequant(orc, wl.normal_bf16((K, M), 1.0, 702 + K), fmt)
    b1, sb1 = prequant(orc, wl.normal_bf16((K, N), 1.0, 703 + K), fmt)
    d = [to_dev_u8(v.ravel()) for v in (a0, b0, a1, b1)]
    s = [dev_f32(v) for v in (sa0, sb0, sa1, sb1)]
    outs = [torch.full((M * N,), 0x7FC1, dtype=torch.int16, device="cuda") for _ in range(4)]
    p0 = (d[0], d[1], fmt, 0, 0, M, N, K, K, N, 1, 0, 0, s[0], s[1], None)
    p1 = (d[2], d[3], fmt, 1, 0, M, N, K, M, N, 1, 0, 0, s[2], s[3], None)
    lib.fp8_mm_pair(p0 + (outs[0],), p1 + (outs[1],))
    lib.fp8_mm(*(p0 + (outs[2],)))
    lib.fp8_mm(*(p1 + (outs[3],)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
    smp = sample_coords(1, M, N, 1500, K)
    for o, (a, b, ta, sa, sb) in ((outs[0], (a0, b0, False, sa0, sb0)),
                                  (outs[1], (a1, b1, True, sa1, sb1))):
        ref, absdot = orc.gemm_sampled(a, b, fmt, ta, False, M, N, K, sa, sb, None, smp)
        got = from_dev_bf16(o).reshape(1, M, N)
        check_gemm(got[smp], ref, absdot, K, f"pair {'TN' if ta else 'NN'} {M}x{N}x{K}")
