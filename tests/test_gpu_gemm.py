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
from tests.gpu_util import (check_gemm, chosen_tile_config, chosen_tile_config as _chosen,
                            dev_f32, from_dev_bf16, to_dev_bf16, to_dev_u8)

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
    bound = orc.gemm_bound(storage(a8, ta), storage(b8, tb), fmt, bool(ta), bool(tb), M, N,
                             K, sa, sb)
    check_gemm(got, ref, bound, f"{M}x{N}x{K} t{ta}{tb} f{fmt}")


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
        bound = orc.gemm_bound(a_pad, b_pad, E4M3, bool(ta), bool(tb), M, N, K, 0.01, 0.02,
                                 lda=a_pad.shape[1], ldb=b_pad.shape[1])
        check_gemm(got, ref, bound, f"pad{pad}", max_frac=1e-2)


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
        bound = orc.gemm_bound(a, b, fmt, False, True, M, N, K, sa, sb, batch=batch,
                                 stride_a=stra, stride_b=strb)
        check_gemm(got, ref, bound, f"batched {stra} {strb}", max_frac=1e-2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (1, 1)], ids=["NN", "TN", "TT"])
def test_mm_small_m_batched_and_broadcast(lib, orc, fmt, ta, tb):
    """m <= 64 outside the NT short-A kernel: the 64 x 64 tiles, batched,
    with either operand broadcast (batch stride 0), ragged m and k, every
    output against the oracle."""
    batch, M, N, K = 3, 48, 208, 400
    assert chosen_tile_config(M, N, batch) == "small"
    a3 = storage(wl.random_codes((batch, M, K), fmt, 21), ta)
    b3 = storage(wl.random_codes((batch, K, N), fmt, 22), tb)
    a1 = storage(wl.random_codes((M, K), fmt, 23), ta)
    b1 = storage(wl.random_codes((K, N), fmt, 24), tb)
    sa, sb = np.float32(1e-3), np.float32(2e-3)
    for a, b, stra, strb in ((a3, b3, M * K, K * N), (a3, b1, M * K, 0), (a1, b3, 0, K * N)):
        got = run_mm(lib, a, b, fmt, ta, tb, M, N, K, sa, sb, batch=batch, stride_a=stra,
                     stride_b=strb)
        ref = orc.gemm(a, b, fmt, bool(ta), bool(tb), M, N, K, sa, sb, batch=batch,
                       stride_a=stra, stride_b=strb)
        bound = orc.gemm_bound(a, b, fmt, bool(ta), bool(tb), M, N, K, sa, sb, batch=batch,
                               stride_a=stra, stride_b=strb)
        check_gemm(got, ref, bound, f"small m t{ta}{tb} {stra} {strb}", max_frac=1e-2)


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
    bound = orc.gemm_bound(a8, b8, fmt, False, True, M, N, K, sa, sb)
    check_gemm(got, ref, bound, f"short-A {M}x{N}x{K} f{fmt}", max_frac=1e-2)


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
        bound = orc.gemm_bound(a, b, E4M3, False, True, M, N, K, 1e-3, 1e-3, batch=batch,
                                 stride_a=stra, stride_b=strb)
        check_gemm(got, ref, bound, f"short-A batched {stra} {strb}", max_frac=1e-2)


def test_mm_extreme_codes(lib, orc):
    """Random codes over the whole E4M3 / E5M2 range (max, subnormals, zeros)."""
    for fmt in (E4M3, E5M2):
        M, N, K = 128, 128, 512
        a8 = wl.random_codes((M, K), fmt, 40)
        b8 = wl.random_codes((N, K), fmt, 41)
        got = run_mm(lib, a8, b8, fmt, 0, 1, M, N, K, 1.0, 1.0)
        ref = orc.gemm(a8, b8, fmt, False, True, M, N, K, 1.0, 1.0)
        bound = orc.gemm_bound(a8, b8, fmt, False, True, M, N, K, 1.0, 1.0)
        check_gemm(got, ref, bound, f"extreme f{fmt}", max_frac=1e-2)


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
    ref, bound = orc.gemm_sampled(a8, b8, fmt, False, True, M, N, K, sa, sb, bias, s,
                                   batch=batch, stride_b=stride_b)
    return check_gemm(got3[s], ref, bound, f"full {batch}x{M}x{N}x{K}")


# fp32 patterns of the combined step sa*sb whose low 16 bits sit on or next
# to a bf16 rounding boundary: ties with an even and an odd kept bit, one
# below and one above a tie, exact, and the largest cut; positive and negative.
TIE_STEPS = [0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x3F820000, 0x3F80FFFF,
             0xBF818000, 0xBF808000, 0x3FFF8000]


@pytest.mark.parametrize("lay,M", [("NT", 16), ("NT", 256), ("NT", 4096), ("NN", 4096),
                                   ("TN", 4096)])
def test_epilogue_rounding_ties(lib, orc, lay, M):
    """The epilogue's one rounding to bf16 (round to nearest, ties to even)
    on outputs that are exact in fp32 and sit on or beside a bf16 rounding
    boundary: A selects one k per row (code 1.0), B holds powers of two from
    2^-9 to 2^8, so each output is 2^e times the combined step, and the
    step's low 16 bits are a tie, a near tie, exact or the largest cut.  Every
    output must equal the oracle's single rounding, bit for bit, on each
    kernel (M = 16: short-A; 256: 128 x 128 tiles; 4096: 256 x 256 tiles)."""
    fmt = E4M3
    ta, tb = dict(zip(["NT", "NN", "TN", "TT"], LAYOUTS))[lay]
    N, K = M, 16
    av = np.zeros((M, K), np.float32)
    av[np.arange(M), np.arange(M) % K] = 1.0
    rng = np.random.default_rng(M + ta)
    bv = np.ldexp(1.0, rng.integers(-9, 9, (K, N))).astype(np.float32)  # logical [K][N]
    a8, b8 = orc.encode_array(av, fmt), orc.encode_array(bv, fmt)
    assert np.array_equal(orc.decode_array(b8, fmt), bv)
    A, B = storage(a8, ta), storage(b8, tb)
    for bits in TIE_STEPS:
        sa = np.array([bits], np.uint32).view(np.float32)[0]
        got = run_mm(lib, A, B, fmt, ta, tb, M, N, K, sa, 1.0)
        ref = orc.gemm(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, 1.0)
        assert np.array_equal(got, ref), f"{lay} M={M} step {bits:#010x}: " \
            f"{int((got != ref).sum())} outputs differ"


# Shapes that take each large tile configuration: every output compared,
# both formats, with ragged m, n and k tails (for an m- or n-contiguous
# operand the tiled kernels need that extent in multiples of 16, so its tail
# is 16).  The library picks the configuration with the least time in
# rounds of 256 tiles (one per CU) times a tile's time (_chosen restates
# that rule, so each shape is checked to land where its name says).
TILE_SHAPES = {
    ("big", "NT"): [(4096, 4096, 256), (4100, 4120, 272)],
    ("big", "NN"): [(4096, 4096, 256), (4100, 4112, 272)],
    ("big", "TN"): [(4096, 4096, 256), (4112, 4112, 272)],
    ("big", "TT"): [(4096, 4096, 256), (4112, 4120, 272)],
    ("wide", "NT"): [(2048, 4096, 256), (2032, 4080, 272)],
    ("wide", "NN"): [(2048, 4096, 256), (2036, 4080, 272)],
    ("wide", "TN"): [(2048, 4096, 256), (2032, 4080, 272)],
    ("wide", "TT"): [(2048, 4096, 256), (2032, 4084, 272)],
    ("tall", "NT"): [(4096, 2048, 256), (4084, 2036, 272)],
    ("tall", "NN"): [(4096, 2048, 256), (4084, 2032, 272)],
    ("tall", "TN"): [(4096, 2048, 256), (4080, 2032, 272)],
    ("tall", "TT"): [(4096, 2048, 256), (4080, 2036, 272)],
    ("mid", "NT"): [(1024, 1024, 256), (1036, 1032, 272)],
    ("mid", "NN"): [(1024, 1024, 256), (1036, 1040, 272)],
    ("mid", "TN"): [(1024, 1024, 256), (1040, 1040, 272)],
    ("mid", "TT"): [(1024, 1024, 256), (1040, 1032, 272)],
}




@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("cfg,lay", list(TILE_SHAPES), ids=[f"{c}-{l}" for c, l in TILE_SHAPES])
@pytest.mark.parametrize("ragged", [False, True], ids=["whole", "ragged"])
def test_tile_configs_full_compare(lib, orc, fmt, cfg, lay, ragged):
    ta, tb = dict(zip(["NT", "NN", "TN", "TT"], LAYOUTS))[lay]
    M, N, K = TILE_SHAPES[(cfg, lay)][int(ragged)]
    assert _chosen(M, N) == cfg, (M, N, _chosen(M, N))
    seed = 900 + 10 * ta + 20 * tb + int(ragged) + 100 * ["big", "wide", "tall", "mid"].index(cfg)
    a8, sa = prequant(orc, wl.normal_bf16((M, K), 1.0, seed), fmt)
    b8, sb = prequant(orc, wl.normal_bf16((K, N), 1.0, seed + 1), fmt)
    bias = wl.normal_bf16((N,), 0.1, seed + 2) if lay == "NT" else None
    A, B = storage(a8, ta), storage(b8, tb)
    got = run_mm(lib, A, B, fmt, ta, tb, M, N, K, sa, sb, bias)
    ref = orc.gemm(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias)
    bound = orc.gemm_bound(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb)
    what = f"tiles {cfg} {lay} {M}x{N}x{K} f{fmt}"
    st = check_gemm(got, ref, bound, what)
    print(f"[{what}] outside 1e-2|r|+ulp: {st['outside_rel_tol']} of {st['n']}")


# Batched problems on the 256 x 256 tiles (more than 256 of them over the
# batch), ragged in m, n and k inside every batch slice, every output
# compared: tiles of one XCD's range then span batch slices (the remapped
# order at 360 tiles, the plain order at 324), and a stride-0 operand is
# shared by all of them.
BATCHED_BIG = [
    # layout, batch, M, N, K, batch stride of A / B (None: M*K / K*N; 0: broadcast)
    ("NT", 8, 1040, 2064, 144, None, None),
    ("NT", 4, 2064, 2080, 144, None, 0),
    ("NN", 8, 1040, 2064, 144, 0, None),
]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("lay,batch,M,N,K,stra,strb", BATCHED_BIG,
                         ids=[f"{c[0]}-b{c[1]}-{c[2]}x{c[3]}x{c[4]}" for c in BATCHED_BIG])
def test_batched_big_tiles_ragged_full_compare(lib, orc, fmt, lay, batch, M, N, K, stra, strb):
    ta, tb = dict(zip(["NT", "NN", "TN", "TT"], LAYOUTS))[lay]
    assert _chosen(M, N, batch) == "big"
    seed = 1500 + 7 * batch + fmt
    ash = (M, K) if stra == 0 else (batch, M, K)
    bsh = (K, N) if strb == 0 else (batch, K, N)
    a8, sa = prequant(orc, wl.normal_bf16(ash, 1.0, seed), fmt)
    b8, sb = prequant(orc, wl.normal_bf16(bsh, 1.0, seed + 1), fmt)
    bias = wl.normal_bf16((N,), 0.1, seed + 2) if lay == "NT" else None
    A, B = storage(a8, ta), storage(b8, tb)
    sta = M * K if stra is None else stra
    stb = K * N if strb is None else strb
    got = run_mm(lib, A, B, fmt, ta, tb, M, N, K, sa, sb, bias, batch=batch, stride_a=sta,
                 stride_b=stb)
    ref = orc.gemm(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, bias, batch=batch,
                   stride_a=sta, stride_b=stb)
    bound = orc.gemm_bound(A, B, fmt, bool(ta), bool(tb), M, N, K, sa, sb, batch=batch,
                           stride_a=sta, stride_b=stb)
    check_gemm(got, ref, bound, f"batched big {lay} b{batch} {M}x{N}x{K} f{fmt} {sta} {stb}")


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


def group_model_dot(p):
    """Value the fp8 MFMA arithmetic model gives for the products p (fp64,
    each exact): per aligned group of 8 consecutive k, every product is cut
    (toward zero; the cases below only cut non-negative products) to a
    multiple of 2^(E-13), E the exponent of the group's largest |product|;
    the group sums are then added (exactly, for these cases)."""
    p = np.asarray(p, np.float64)
    total = 0.0
    for g in range(0, p.size, 8):
        grp = p[g:g + 8]
        mx = np.abs(grp).max()
        if mx == 0:
            continue
        lsb = 2.0 ** (np.floor(np.log2(mx)) - 13)
        total += float(np.sum(np.trunc(grp / lsb) * lsb))
    return total


def group_cases(K):
    """Crafted dot products (a, b value pairs over k): large cancelling
    products beside small ones in the same aligned group of 8 k, in other
    groups, in the second half of a 64-k step and across a group boundary."""
    small = (0.25, 0.25)  # 2^-4
    cases = {}

    def base():
        return [small] * K

    c = base(); c[0] = (32.0, 32.0); c[1] = (-32.0, 32.0)
    cases["cut_14_below"] = c            # 2^-4 is 14 bits below 2^10: cut
    c = base(); c[0] = (32.0, 32.0); c[1] = (-32.0, 32.0)
    for k in range(2, 8):
        c[k] = (0.5, 0.25)               # 2^-3: 13 bits below 2^10: kept
    cases["keep_13_below"] = c
    c = base(); c[40] = (32.0, 32.0); c[41] = (-32.0, 32.0)
    cases["group_5"] = c                 # k 40..47: second lane half of the step
    c = base(); c[70] = (32.0, 32.0); c[73] = (-32.0, 32.0)
    cases["straddle_8_9"] = c            # k 70 in group 8, k 73 in group 9
    c = base(); c[0] = (28.0, 28.0); c[1] = (-28.0, 28.0)
    for k in range(2, 8):
        c[k] = (0.25, 0.25)              # 784 = 1.53 * 2^9: 2^-4 is 13 below 2^9
    cases["mantissa_product_above_2"] = c
    c = base()
    cases["no_cancellation"] = c
    return cases


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("ta,tb", LAYOUTS[:3], ids=["NT", "NN", "TN"])
@pytest.mark.parametrize("M", [16, 128])
def test_mfma_group_model(lib, orc, fmt, ta, tb, M):
    """Evidence for the accumulation model behind the GEMM tolerance, on every
    kernel that runs an fp8 MFMA (M = 16 NT: the short-A kernel; M = 128: the
    tiled kernels): the products of each aligned group of 8 consecutive k are
    aligned to the group's largest product and kept to 13 bits below its
    leading bit (2^-4 beside +-2^10 is cut, 2^-3 is kept), and groups are
    summed without that cut.  Each crafted case sits on one diagonal output;
    the kernel's value equals the model's, and the oracle's error bound covers
    the difference to the exact sum."""
    K = 128
    cases = group_cases(K)
    names = list(cases)
    N = M
    av = np.zeros((M, K), np.float32)
    bv = np.zeros((K, N), np.float32)  # logical B [K][N]
    for i, name in enumerate(names):
        for k, (x, y) in enumerate(cases[name]):
            av[i, k], bv[k, i] = x, y
    a8, b8 = orc.encode_array(av, fmt), orc.encode_array(bv, fmt)
    assert np.array_equal(orc.decode_array(a8, fmt), av)  # every value exact
    assert np.array_equal(orc.decode_array(b8, fmt), bv)
    got = run_mm(lib, storage(a8, ta), storage(b8, tb), fmt, ta, tb, M, N, K, 1.0, 1.0)
    bound = orc.gemm_bound(storage(a8, ta), storage(b8, tb), fmt, bool(ta), bool(tb), M, N, K,
                           1.0, 1.0)
    for i, name in enumerate(names):
        p = np.array([x * y for x, y in cases[name]], np.float64)
        exact, model = float(p.sum()), group_model_dot(p)
        y = float(wl.bf16_bits_to_f32(got[i, i]))
        assert y == model, f"{name}: kernel {y}, model {model}, exact {exact}"
        assert abs(model - exact) <= bound[i, i], f"{name}: bound {bound[i, i]} too small"


# ---------------------------------------------------------------------------
# Two independent products from one call (the backward's dX and dW)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (4144, 4176, 272), (2064, 1040, 272),
                                   (256, 512, 320)])
def test_mm_pair_matches_two_calls(lib, orc, fmt, M, N, K):
    """fp8_mm_pair of an NN and a TN product gives the bits of two fp8_mm
    calls: through the paired kernel on 256 x 256 tiles when both have at
    least 256 of them (the first two shapes, the second with ragged m, n and
    k tails), on 128 x 128 tiles when the two have at least 256 of those
    between them (the third, ragged), as two launches otherwise; and every
    output of both matches the oracle."""
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
    for o, (a, b, ta, sa, sb) in ((outs[0], (a0, b0, False, sa0, sb0)),
                                  (outs[1], (a1, b1, True, sa1, sb1))):
        ref = orc.gemm(a, b, fmt, ta, False, M, N, K, sa, sb)
        bound = orc.gemm_bound(a, b, fmt, ta, False, M, N, K, sa, sb)
        st = check_gemm(from_dev_bf16(o).reshape(M, N), ref, bound,
                        f"pair {'TN' if ta else 'NN'} {M}x{N}x{K}")
        print(f"[pair {'TN' if ta else 'NN'} {M}x{N}x{K} f{fmt}] outside 1e-2|r|+ulp: "
              f"{st['outside_rel_tol']} of {st['n']}")


@pytest.mark.parametrize("shapes", [((2048, 1024, 4096), (4096, 1024, 2048)),
                                    ((2064, 1040, 4112), (4112, 1040, 2064))],
                         ids=["train2048", "ragged"])
def test_mm_pair_unequal_k(lib, orc, shapes):
    """The paired launch with tiles of unequal area: NN problem 0 with twice
    the k of TN problem 1 (the training layer's dX and dW) runs on 128 x 128
    tiles for problem 0 and 256 x 128 tiles for problem 1; the bits equal two
    fp8_mm calls and every output matches the oracle (E5M2, the backward
    format)."""
    fmt = E5M2
    (M0, N0, K0), (M1, N1, K1) = shapes
    a0, sa0 = prequant(orc, wl.normal_bf16((M0, K0), 1e-3, 1400), fmt)
    b0, sb0 = prequant(orc, wl.normal_bf16((K0, N0), 0.02, 1401), fmt)
    a1, sa1 = prequant(orc, wl.normal_bf16((K1, M1), 1e-3, 1402), fmt)
    b1, sb1 = prequant(orc, wl.normal_bf16((K1, N1), 1.0, 1403), fmt)
    d = [to_dev_u8(v.ravel()) for v in (a0, b0, a1, b1)]
    s = [dev_f32(v) for v in (sa0, sb0, sa1, sb1)]
    outs = [torch.full((M * N,), 0x7FC1, dtype=torch.int16, device="cuda")
            for M, N in ((M0, N0), (M1, N1), (M0, N0), (M1, N1))]
    p0 = (d[0], d[1], fmt, 0, 0, M0, N0, K0, K0, N0, 1, 0, 0, s[0], s[1], None)
    p1 = (d[2], d[3], fmt, 1, 0, M1, N1, K1, M1, N1, 1, 0, 0, s[2], s[3], None)
    lib.fp8_mm_pair(p0 + (outs[0],), p1 + (outs[1],))
    lib.fp8_mm(*(p0 + (outs[2],)))
    lib.fp8_mm(*(p1 + (outs[3],)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
    for o, (a, b, ta, M, N, K, sa, sb) in ((outs[0], (a0, b0, False, M0, N0, K0, sa0, sb0)),
                                           (outs[1], (a1, b1, True, M1, N1, K1, sa1, sb1))):
        ref = orc.gemm(a, b, fmt, ta, False, M, N, K, sa, sb)
        bound = orc.gemm_bound(a, b, fmt, ta, False, M, N, K, sa, sb)
        what = f"pair {'TN' if ta else 'NN'} {M}x{N}x{K}"
        st = check_gemm(from_dev_bf16(o).reshape(M, N), ref, bound, what)
        print(f"[{what}] outside 1e-2|r|+ulp: {st['outside_rel_tol']} of {st['n']}")
