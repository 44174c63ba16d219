"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something independent of it: a
library routine (torch CPU float8 / bfloat16 conversion, float64 matmul and
sum), a closed form printed on or implied by the AstrAI pages, an invariant,
or brute force.  A plausible slip anywhere in the oracle (a dropped bias or
scale, a wrong sign, a transposed operand, double rounding, divide instead of
multiply) fails at least one of them; ``test_planted_mistakes`` checks that
claim by planting such slips in a Python copy of the definitions.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as wl

E4M3, E5M2 = 0, 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_encode(v_f32: np.ndarray, fmt: int) -> np.ndarray:
    """Library routine: clamp to +-max then torch's RNE float8 cast."""
    t = torch.from_numpy(np.ascontiguousarray(v_f32, np.float32))
    m = FMAX[fmt]
    return t.clamp(-m, m).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()


def torch_decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(TORCH_FP8[fmt]).to(torch.float64).numpy()


def is_nan_code(c, fmt):
    c = np.asarray(c)
    if fmt == E4M3:
        return (c & 0x7F) == 0x7F
    return ((c & 0x7C) == 0x7C) & ((c & 0x03) != 0)


# --------------------------------------------------------------------------
# Format constants: the pages print the maxima (FP8_MAX in fp8.py).
# --------------------------------------------------------------------------

def test_golden_format_constants(orc):
    with open(os.path.join(GOLDEN, "format_constants.json")) as f:
        g = json.load(f)
    assert orc.decode(0x7E, E4M3) == g["e4m3_max"] == 448.0
    assert orc.decode(0x7B, E5M2) == g["e5m2_max"] == 57344.0
    assert orc.encode(g["e4m3_max"], E4M3) == 0x7E
    assert orc.encode(g["e5m2_max"], E5M2) == 0x7B
    assert orc.scale_from_peak(g["e4m3_max"], E4M3) == np.float32(1.0)
    assert orc.scale_from_peak(g["e5m2_max"], E5M2) == np.float32(1.0)
    assert orc.scale_from_peak(0.0, E4M3) == np.float32(g["scale_floor"])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_all_codes_vs_torch(orc, fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([orc.decode(c, fmt) for c in codes], np.float64)
    ref = torch_decode(codes, fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_encode_closed_forms(orc):
    # smallest subnormals, the tie below it, 1.5 quanta (tie to even: 2)
    assert orc.encode(2.0 ** -9, E4M3) == 0x01
    assert orc.encode(2.0 ** -10, E4M3) == 0x00
    assert orc.encode(1.5 * 2.0 ** -9, E4M3) == 0x02
    assert orc.encode(2.5 * 2.0 ** -9, E4M3) == 0x02
    assert orc.encode(2.0 ** -16, E5M2) == 0x01
    assert orc.encode(2.0 ** -17, E5M2) == 0x00
    assert orc.encode(-0.0, E4M3) == 0x80
    assert orc.encode(-2.0 ** -12, E4M3) == 0x80
    # satfinite: beyond max, infinity
    for v in (449.0, 464.0, 470.0, 1e30, math.inf):
        assert orc.encode(v, E4M3) == 0x7E
        assert orc.encode(-v, E4M3) == 0xFE
    for v in (61440.0, 1e30, math.inf):
        assert orc.encode(v, E5M2) == 0x7B
    # NaN keeps a NaN code
    assert is_nan_code(orc.encode(math.nan, E4M3), E4M3)
    assert is_nan_code(orc.encode(math.nan, E5M2), E5M2)
    # 1.0 and the binade boundary
    assert orc.encode(1.0, E4M3) == 0x38
    assert orc.encode(1.0, E5M2) == 0x3C
    assert orc.encode(1.0 + 2.0 ** -4, E4M3) == 0x38  # tie -> even
    assert orc.encode(1.0 + 3 * 2.0 ** -4, E4M3) == 0x3A  # tie -> even (up)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_decode_roundtrip(orc, fmt):
    for c in range(256):
        if is_nan_code(c, fmt):
            continue
        v = orc.decode(c, fmt)
        if math.isinf(v):
            assert orc.encode(v, fmt) == (0x7B | (c & 0x80))
        else:
            assert orc.encode(v, fmt) == c


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_bf16_grid_vs_torch(orc, fmt):
    """Every bf16 value times a few multipliers (the inputs a quantize
    actually sees), plus every fp32 within 2 ulp of each fp8 midpoint."""
    allbf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf)]
    mults = np.array([1.0, 3.0, 0.7, 1.0 / 3.0, 448.0 / 3.7, 2.0 ** -20], np.float32)
    with np.errstate(over="ignore"):
        v = (allbf[None, :] * mults[:, None]).ravel()
    assert np.array_equal(orc.encode_array(v, fmt), torch_encode(v, fmt))
    # neighbourhoods of midpoints between consecutive representable values
    pos = np.array([orc.decode(c, fmt) for c in range(128) if not is_nan_code(c, fmt)])
    pos = np.sort(pos[np.isfinite(pos)].astype(np.float64))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    bits = mids.view(np.uint32)
    near = np.concatenate([(bits.astype(np.int64) + d) for d in range(-2, 3)])
    near = near[(near >= 0)].astype(np.uint32).view(np.float32)
    near = np.concatenate([near, -near, pos.astype(np.float32)])
    assert np.array_equal(orc.encode_array(near, fmt), torch_encode(near, fmt))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_exhaustive_vs_torch(orc, fmt):
    """All 2^32 fp32 bit patterns except NaN: oracle == torch clamp+cast."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        ours = orc.encode_bits_range(start, chunk, fmt)
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32)
        ref = torch_encode(v, fmt)
        nan = np.isnan(v)
        ok = (ours == ref) | nan
        if not ok.all():
            i = int(np.argmin(ok))
            raise AssertionError(f"fmt {fmt} bits {bits[i]:#010x}: {ours[i]:#x} vs {ref[i]:#x}")
        assert is_nan_code(ours[nan], fmt).all()


# --------------------------------------------------------------------------
# bf16 rounding (the output type of the GEMM and the bias gradient)
# --------------------------------------------------------------------------

def test_bf16_from_f64_vs_torch_on_fp32_values(orc):
    """On fp32-representable inputs torch's single RNE step is the
    definition (no double rounding possible)."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = orc.bf16_from_f64(v.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_from_f64_single_rounding(orc):
    # 1 + 2^-8 + 2^-30 is above the bf16 midpoint 1 + 2^-8: one rounding
    # gives 1 + 2^-7 (0x3F81); rounding through fp32 first would tie to 1.0.
    assert int(orc.bf16_from_f64(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0]) == 0x3F81
    assert int(orc.bf16_from_f64(np.array([1 + 2.0 ** -8]))[0]) == 0x3F80
    assert int(orc.bf16_from_f64(np.array([-(1 + 3 * 2.0 ** -8)]))[0]) == 0xBF82
    assert int(orc.bf16_from_f64(np.array([3.5e38]))[0]) == 0x7F80
    assert int(orc.bf16_from_f64(np.array([2.0 ** -133]))[0]) == 0x0001
    assert int(orc.bf16_from_f64(np.array([-0.0]))[0]) == 0x8000


# --------------------------------------------------------------------------
# amax, scale, quantize
# --------------------------------------------------------------------------

def test_amax_brute_force(orc):
    for seed, shape in [(1, (7,)), (2, (33, 65)), (3, (1000,))]:
        x = wl.normal_bf16(shape, 3.0, seed)
        f = wl.bf16_bits_to_f32(x)
        a = orc.amax(x)
        assert a == np.float32(np.abs(f).max())
        assert (np.abs(f) <= a).all() and (np.abs(f) == a).any()
    assert orc.amax(np.zeros(5, np.uint16)) == 0.0
    assert orc.amax(np.zeros(0, np.uint16)) == 0.0
    # NaN input is skipped; -0 counts as 0
    x = np.array([0x7FC0, 0x3F80, 0x8000], np.uint16)
    assert orc.amax(x) == 1.0


def test_scale_closed_forms(orc):
    assert orc.scale_from_peak(448.0, E4M3, 0) == 1.0
    assert orc.scale_from_peak(448.0, E4M3, 1) == 0.5
    assert orc.scale_from_peak(448.0, E4M3, 3) == 0.125
    assert orc.scale_from_peak(57344.0, E5M2, 0) == 1.0
    assert orc.scale_from_peak(0.0, E5M2, 0) == np.float32(1e-12)
    assert orc.scale_from_peak(1e-20, E4M3, 0) == np.float32(1e-12)
    # general value: two IEEE fp32 divisions (torch fp32 tensor division)
    for p in (3.0, 0.0123, 77.7, 1e5):
        t = torch.tensor([p], dtype=torch.float32)
        ref = ((t / torch.tensor([448.0])) / torch.tensor([4.0])).item()
        assert orc.scale_from_peak(p, E4M3, 2) == np.float32(ref)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_vs_torch_composition(orc, fmt):
    """encode(fp32(x * fp32(1/s))): torch reciprocal, multiply, clamp, cast."""
    x = wl.normal_bf16((4096,), 2.0, 11)
    for s in (np.float32(2.5 / FMAX[fmt]), np.float32(1e-3), np.float32(0.37), np.float32(1e-12)):
        m = torch.reciprocal(torch.tensor([s], dtype=torch.float32))
        xf = torch.from_numpy(wl.bf16_bits_to_f32(x))
        ref = torch_encode((xf * m).numpy(), fmt)
        assert np.array_equal(orc.quantize(x, fmt, s), ref)
        assert orc.multiplier(s) == m.item()


def test_f16_decode_all_patterns_vs_torch(orc):
    """fp16 decode written from the binary16 definition equals torch's CPU
    float16 -> float32 conversion on all 65536 patterns (NaN stays NaN)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.float16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_in_vs_torch_composition(orc, fmt):
    """fp16 and fp32 inputs: encode(fp32(fp32(x) * fp32(1/s))) by torch's
    widening, reciprocal, multiply, clamp and cast; amax by torch's max of
    |x| (NaN-free data)."""
    rng = np.random.default_rng(21 + fmt)
    x32 = (rng.standard_normal(5000) * 3.0).astype(np.float32)
    x32[:4] = [0.0, -0.0, 1e-30, -6.5e4]
    x16 = x32.astype(np.float16)
    for s in (np.float32(2.5 / FMAX[fmt]), np.float32(0.37), np.float32(1e-12)):
        m = torch.reciprocal(torch.tensor([s], dtype=torch.float32))
        for in_type, x, xt in ((2, x32, torch.from_numpy(x32)),
                               (1, x16.view(np.uint16), torch.from_numpy(x16).float())):
            ref = torch_encode((xt * m).numpy(), fmt)
            assert np.array_equal(orc.quantize_in(x, in_type, fmt, s), ref), (in_type, s)
            assert orc.amax_in(x, in_type) == np.float32(xt.abs().max().item())


def test_quantize_in_reduces_to_the_bf16_path(orc):
    """The same values given as bf16 bits, fp16 bits (values that fit both)
    or fp32 quantize to the same codes and have the same amax; NaN is
    skipped by every amax."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = orc.f16_to_f32(h)
    fits = np.isfinite(f) & ((h & 0x7) == 0)        # 7 fraction bits or fewer
    v = f[fits]
    b = (v.view(np.uint32) >> 16).astype(np.uint16)   # exact bf16 bits of v
    assert np.array_equal(wl.bf16_bits_to_f32(b), v)
    for fmt, s in ((E4M3, np.float32(0.01)), (E5M2, np.float32(3.0))):
        ref = orc.quantize(b, fmt, s)
        assert np.array_equal(orc.quantize_in(b, 0, fmt, s), ref)
        assert np.array_equal(orc.quantize_in(h[fits], 1, fmt, s), ref)
        assert np.array_equal(orc.quantize_in(v, 2, fmt, s), ref)
    assert orc.amax_in(h[fits], 1) == orc.amax(b) == orc.amax_in(v, 2)
    nan32 = np.array([np.nan, 2.0, -3.0], np.float32)
    assert orc.amax_in(nan32, 2) == 3.0
    assert orc.amax_in(np.array([0x7E00, 0x4000, 0xC200], np.uint16), 1) == 3.0


def test_quantize_t_elementwise(orc):
    """Transposed codes: element (c, r) is the encode of x[r][c] * fp32(1/s)
    by the (pinned) scalar encode, on a ragged matrix."""
    x = wl.normal_bf16((37, 53), 2.0, 31)
    s = np.float32(0.02)
    q, qt = orc.quantize_t(x, E4M3, s)
    m = orc.multiplier(s)
    f = wl.bf16_bits_to_f32(x)
    assert qt.shape == (53, 37) and q.shape == (37, 53)
    for r in range(0, 37, 5):
        for c in range(0, 53, 7):
            code = orc.encode(float(np.float32(f[r, c] * m)), E4M3)
            assert q[r, c] == code and qt[c, r] == code


def test_quantize_multiplies_by_reciprocal(orc):
    """x * fp32(1/s) and x / s can round to different codes; the kernel on
    the pages multiplies by the reciprocal (reading of the scale
    convention).  Cases found by search: fp32(x/s) lands exactly on an E4M3
    rounding midpoint while x * fp32(1/s) lands one fp32 ulp off it."""
    cases = [(1.015625, 0.9558822512626648), (1.0078125, 0.7010869979858398),
             (1.078125, 0.5564516186714172)]
    for xv, sv in cases:
        s = np.float32(sv)
        x = wl.f32_to_bf16_bits(np.array([xv], np.float32))
        f = wl.bf16_bits_to_f32(x)
        mul = torch_encode(f * (np.float32(1.0) / s), E4M3)
        div = torch_encode(f / s, E4M3)
        assert mul[0] != div[0]
        assert np.array_equal(orc.quantize(x, E4M3, s), mul)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def _store(mat, trans):
    """Storage of a logical matrix: as is, or its transpose (contiguous)."""
    return np.ascontiguousarray(mat.T if trans else mat)


def _torch_gemm_ref(orc, A, B, fmt, sa, sb, bias):
    """float64 matmul of the decoded logical operands, scale, bias, then a
    single bf16 rounding."""
    a = torch.from_numpy(torch_decode(A, fmt))
    b = torch.from_numpy(torch_decode(B, fmt))
    s = float(np.float32(sa) * np.float32(sb))
    y = torch.matmul(a, b) * s
    if bias is not None:
        y = y + torch.from_numpy(wl.bf16_bits_to_f32(bias).astype(np.float64))
    return orc.bf16_from_f64(y.numpy())


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("trans_a,trans_b", [(0, 1), (0, 0), (1, 0), (1, 1)])
def test_gemm_tiny_bruteforce_vs_matmul(orc, fmt, trans_a, trans_b):
    seed = 100
    for M in range(1, 5):
        for N in range(1, 5):
            for K in range(1, 5):
                seed += 1
                A = wl.random_codes((M, K), fmt, seed)
                B = wl.random_codes((K, N), fmt, seed + 5000)
                # include extremes: max, subnormal, zero
                A.flat[0] = 0x7E if fmt == E4M3 else 0x7B
                B.flat[-1] = 0x01
                bias = wl.normal_bf16((N,), 0.5, seed) if seed % 2 else None
                sa, sb = np.float32(0.75), np.float32(1.0 / 3.0)
                ours = orc.gemm(_store(A, trans_a), _store(B, trans_b), fmt, bool(trans_a),
                                bool(trans_b), M, N, K, sa, sb, bias)
                ref = _torch_gemm_ref(orc, A, B, fmt, sa, sb, bias)
                assert np.array_equal(ours, ref), (M, N, K)


def test_gemm_batched_and_broadcast_vs_matmul(orc):
    fmt = E4M3
    batch, M, N, K = 3, 5, 6, 7
    A = wl.random_codes((batch, M, K), fmt, 1)
    B = wl.random_codes((batch, N, K), fmt, 2)
    B1 = wl.random_codes((N, K), fmt, 3)
    sa, sb = np.float32(0.5), np.float32(0.25)
    ours = orc.gemm(A, B, fmt, False, True, M, N, K, sa, sb, batch=batch)
    for b in range(batch):
        ref = _torch_gemm_ref(orc, A[b], B[b].T, fmt, sa, sb, None)
        assert np.array_equal(ours[b], ref)
    ours = orc.gemm(A, B1, fmt, False, True, M, N, K, sa, sb, batch=batch, stride_b=0)
    for b in range(batch):
        assert np.array_equal(ours[b], _torch_gemm_ref(orc, A[b], B1.T, fmt, sa, sb, None))


def test_gemm_onehot_rows_reproduce_b_times_scale(orc):
    """A = one-hot rows selects rows of B^T exactly, times fp32(sa*sb)."""
    fmt = E4M3
    M, N, K = 4, 9, 6
    B = wl.random_codes((N, K), fmt, 9)  # stored [N][K]
    A = np.zeros((M, K), np.uint8)
    sel = [5, 0, 3, 1]
    for i, k in enumerate(sel):
        A[i, k] = 0x38  # 1.0
    sa, sb = np.float32(2.0), np.float32(0.125)
    out = orc.gemm(A, B, fmt, False, True, M, N, K, sa, sb)
    Bd = torch_decode(B, fmt)
    for i, k in enumerate(sel):
        assert np.array_equal(wl.bf16_bits_to_f32(out[i]), (Bd[:, k] * 0.25).astype(np.float32))


def test_gemm_layouts_agree(orc):
    """NN and TN equal NT on explicitly transposed storage."""
    fmt = E5M2
    M, N, K = 13, 11, 17
    A = wl.random_codes((M, K), fmt, 21)
    B = wl.random_codes((K, N), fmt, 22)
    sa, sb = np.float32(3.0), np.float32(0.001)
    nt = orc.gemm(A, np.ascontiguousarray(B.T), fmt, False, True, M, N, K, sa, sb)
    nn = orc.gemm(A, B, fmt, False, False, M, N, K, sa, sb)
    tn = orc.gemm(np.ascontiguousarray(A.T), B, fmt, True, False, M, N, K, sa, sb)
    tt = orc.gemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), fmt, True, True,
                  M, N, K, sa, sb)
    assert np.array_equal(nt, nn) and np.array_equal(nt, tn) and np.array_equal(nt, tt)


def test_gemm_sampled_matches_full(orc):
    fmt = E4M3
    batch, M, N, K = 2, 17, 19, 40
    A = wl.random_codes((batch, K, M), fmt, 31)
    B = wl.random_codes((batch, K, N), fmt, 32)
    bias = wl.normal_bf16((N,), 0.3, 33)
    full = orc.gemm(A, B, fmt, True, False, M, N, K, 0.5, 0.5, bias, batch=batch)
    rng = np.random.default_rng(0)
    s = (rng.integers(0, batch, 50), rng.integers(0, M, 50), rng.integers(0, N, 50))
    vals, bound = orc.gemm_sampled(A, B, fmt, True, False, M, N, K, 0.5, 0.5, bias, s,
                                   batch=batch)
    assert np.array_equal(vals, full[s])
    fb = orc.gemm_bound(A, B, fmt, True, False, M, N, K, 0.5, 0.5, batch=batch)
    assert np.array_equal(bound, fb[s])
    ad = orc.gemm_absdot(A, B, fmt, True, False, M, N, K, 0.5, 0.5, batch=batch)
    Ad = torch_decode(A, fmt)
    Bd = torch_decode(B, fmt)
    ref = np.abs(np.einsum("bkm,bkn->bmnk", Ad, Bd)).sum(-1) * 0.25
    assert np.allclose(ad, ref, rtol=1e-12, atol=0)


# --------------------------------------------------------------------------
# The GEMM tolerance's accumulation bound (reading c13: outputs that cancel
# to near zero are accepted within the error a correct fp32-accumulating fp8
# kernel may carry).  Tolerance tooling, pinned like the rest.
# --------------------------------------------------------------------------

def _groupmax_bruteforce(Ad, Bd, K):
    """sum over aligned groups of 8 k of max |a_k b_k|, from decoded
    operands Ad [M][K], Bd [K][N] (numpy, independent of the C loops)."""
    p = np.abs(Ad[:, None, :] * Bd.T[None, :, :])  # [M][N][K]
    pad = (-K) % 8
    p = np.concatenate([p, np.zeros(p.shape[:2] + (pad,))], axis=2)
    return p.reshape(p.shape[0], p.shape[1], -1, 8).max(-1).sum(-1)


@pytest.mark.parametrize("trans_a,trans_b", [(0, 1), (0, 0), (1, 0), (1, 1)])
def test_gemm_groupmax_bruteforce(orc, trans_a, trans_b):
    """Group maxima against numpy on small shapes with ragged last groups,
    batched and broadcast."""
    for fmt in (E4M3, E5M2):
        for (M, N, K) in ((3, 5, 1), (4, 3, 7), (5, 6, 8), (2, 7, 21), (6, 4, 64)):
            A = wl.random_codes((M, K), fmt, M * 100 + K)
            B = wl.random_codes((K, N), fmt, N * 100 + K + 7)
            sa, sb = np.float32(0.5), np.float32(3.0)
            got = orc.gemm_groupmax(_store(A, trans_a), _store(B, trans_b), fmt, bool(trans_a),
                                    bool(trans_b), M, N, K, sa, sb)
            ref = _groupmax_bruteforce(torch_decode(A, fmt).astype(np.float64),
                                       torch_decode(B, fmt).astype(np.float64), K) * 1.5
            assert np.allclose(got, ref, rtol=1e-13, atol=0), (fmt, M, N, K)
    batch, M, N, K = 3, 4, 5, 24
    A = wl.random_codes((batch, M, K), E4M3, 71)
    B1 = wl.random_codes((N, K), E4M3, 72)
    got = orc.gemm_groupmax(A, B1, E4M3, False, True, M, N, K, 1.0, 1.0, batch=batch,
                            stride_b=0)
    for b in range(batch):
        ref = _groupmax_bruteforce(torch_decode(A[b], E4M3).astype(np.float64),
                                   torch_decode(B1, E4M3).T.astype(np.float64), K)
        assert np.allclose(got[b], ref, rtol=1e-13, atol=0)


def _crafted_dot(orc, pairs, fmt=E4M3):
    """A 1 x 1 NT product whose k-th terms are the value pairs given."""
    K = len(pairs)
    a = orc.encode_array(np.array([[x for x, _ in pairs]], np.float32), fmt)
    b = orc.encode_array(np.array([[y for _, y in pairs]], np.float32), fmt)
    return a, b, K


def test_gemm_bound_closed_forms(orc):
    """Two crafted cases by hand.  (1) +-2^10 at k = 0, 1 and 126 products of
    2^-4: group maxima 1024 + 15 * 2^-4, |sum| 2048 + 126 * 2^-4.  (2) +2^10 at
    k = 70 and -2^10 at k = 73, on either side of the group boundary at 72:
    group maxima 2 * 1024 + 14 * 2^-4 (an unaligned grouping, e.g. groups
    starting at k = 4, would give 1024 + 15 * 2^-4)."""
    u = 2.0 ** -24
    K = 128
    gamma = K * u / (1 - K * u)
    small = (0.25, 0.25)
    pairs = [small] * K
    pairs[0], pairs[1] = (32.0, 32.0), (-32.0, 32.0)
    a, b, _ = _crafted_dot(orc, pairs)
    gm = orc.gemm_groupmax(a, b, E4M3, False, True, 1, 1, K, 1.0, 1.0)[0, 0]
    ad = orc.gemm_absdot(a, b, E4M3, False, True, 1, 1, K, 1.0, 1.0)[0, 0]
    assert gm == 1024 + 15 * 2.0 ** -4 and ad == 2048 + 126 * 2.0 ** -4
    bound = orc.gemm_bound(a, b, E4M3, False, True, 1, 1, K, 1.0, 1.0)[0, 0]
    assert bound == 7 * 2.0 ** -13 * gm + gamma * ad
    # the cut of the 6 small products beside +-1024 (6 * 2^-4) is inside it
    assert 6 * 2.0 ** -4 <= bound
    pairs = [small] * K
    pairs[70], pairs[73] = (32.0, 32.0), (-32.0, 32.0)
    a, b, _ = _crafted_dot(orc, pairs)
    gm = orc.gemm_groupmax(a, b, E4M3, False, True, 1, 1, K, 1.0, 1.0)[0, 0]
    assert gm == 2 * 1024 + 14 * 2.0 ** -4
    # the scale enters as |fp32(sa * sb)|
    gm_s = orc.gemm_groupmax(a, b, E4M3, False, True, 1, 1, K, -0.5, 0.25)[0, 0]
    assert gm_s == gm * 0.125


def _group_cut_model(p):
    """Worst case of the modelled arithmetic: every product of a group except
    its largest loses just under 2^-13 of the group's leading power of two,
    all in the same direction."""
    total = 0.0
    for g in range(0, p.size, 8):
        grp = p[g:g + 8]
        mx = np.abs(grp).max()
        if mx == 0:
            continue
        lsb = 2.0 ** (np.floor(np.log2(mx)) - 13)
        total += (grp.size - 1) * lsb * (1 - 2.0 ** -20)
    return total


def test_gemm_bound_covers_the_group_model(orc):
    """On random operands over the whole fp8 range the worst-case cut of the
    group model stays inside the oracle's bound, output by output."""
    for fmt in (E4M3, E5M2):
        M, N, K = 6, 5, 200
        A = wl.random_codes((M, K), fmt, 91 + fmt)
        B = wl.random_codes((N, K), fmt, 92 + fmt)
        bound = orc.gemm_bound(A, B, fmt, False, True, M, N, K, 1.0, 1.0)
        Ad = torch_decode(A, fmt).astype(np.float64)
        Bd = torch_decode(B, fmt).astype(np.float64)
        for i in range(M):
            for j in range(N):
                assert _group_cut_model(Ad[i] * Bd[j]) <= bound[i, j]


# --------------------------------------------------------------------------
# GEMM with an fp8 bias and / or an fp8 output ([CMP] the removed fp8_gemm
# op's out_dtype / out_scale; [LOG1] bias_scale)
# --------------------------------------------------------------------------

def _torch_gemm_ex_ref(A, B, fmt, sa, sb, bias, bias_scale, out_type, out_scale):
    """Independent composition: torch float8 decode, float64 matmul, the
    bias value (torch-decoded code times its step in fp32, or bf16), then
    for an fp8 output fp32(y) times the fp32 reciprocal of the step and
    torch's clamped float8 cast.  Returns (codes or None, y)."""
    a = torch.from_numpy(torch_decode(A, fmt))
    b = torch.from_numpy(torch_decode(B, fmt))
    s = float(np.float32(sa) * np.float32(sb))
    y = (torch.matmul(a, b) * s).numpy()
    if bias is not None:
        if bias_scale is not None:
            bv = torch_decode(bias, fmt).astype(np.float32) * np.float32(bias_scale)
        else:
            bv = wl.bf16_bits_to_f32(bias)
        y = y + bv.astype(np.float64)
    if out_type == 0:
        return None, y
    r = np.float32(1.0) / np.float32(out_scale)
    fo = E4M3 if out_type == 1 else E5M2
    return torch_encode(y.astype(np.float32) * r, fo), y


@pytest.mark.parametrize("trans_a,trans_b", [(0, 1), (0, 0), (1, 0)])
def test_gemm_ex_bf16_path_is_gemm(orc, trans_a, trans_b):
    """bf16 bias and bf16 output: exactly the pinned orc.gemm."""
    fmt = E4M3
    M, N, K = 7, 9, 33
    A = wl.random_codes((M, K), fmt, 81)
    B = wl.random_codes((K, N), fmt, 82)
    bias = wl.normal_bf16((N,), 0.5, 83)
    ref = orc.gemm(_store(A, trans_a), _store(B, trans_b), fmt, bool(trans_a), bool(trans_b),
                   M, N, K, 0.5, 0.125, bias)
    out, _, _ = orc.gemm_ex(_store(A, trans_a), _store(B, trans_b), fmt, bool(trans_a),
                            bool(trans_b), M, N, K, 0.5, 0.125, bias)
    assert np.array_equal(out.reshape(M, N), ref)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("out_type", [1, 2])
@pytest.mark.parametrize("bias_kind", ["none", "bf16", "fp8"])
def test_gemm_ex_fp8_out_vs_torch(orc, fmt, out_type, bias_kind):
    """Brute force on small shapes against the torch composition; operands
    of moderate range so that every fp64 sum is exact; out_scale small
    enough that some outputs saturate."""
    seed = 900 + 10 * fmt + out_type
    for M, N, K in ((1, 1, 1), (3, 5, 4), (6, 7, 8), (4, 16, 32)):
        seed += 1
        A = orc.quantize(wl.normal_bf16((M, K), 1.0, seed), fmt, 1.0)
        B = orc.quantize(wl.normal_bf16((K, N), 1.0, seed + 1), fmt, 1.0)
        bias = bias_scale = None
        if bias_kind == "bf16":
            bias = wl.normal_bf16((N,), 2.0, seed + 2)
        elif bias_kind == "fp8":
            bias = orc.quantize(wl.normal_bf16((N,), 2.0, seed + 2), fmt, 1.0)
            bias_scale = np.float32(0.375)
        sa, sb = np.float32(0.75), np.float32(1.5)
        for out_scale in (np.float32(1.0 / 64), np.float32(0.01), np.float32(3.0)):
            out, y, _ = orc.gemm_ex(A, B, fmt, False, False, M, N, K, sa, sb, bias, bias_scale,
                                    out_type, out_scale)
            ref, yref = _torch_gemm_ex_ref(A, B, fmt, sa, sb, bias, bias_scale, out_type,
                                           out_scale)
            assert np.array_equal(y, yref.ravel()), (M, N, K)
            assert np.array_equal(out, ref.ravel()), (M, N, K, out_scale)
            assert np.array_equal(orc.out_codes(y, out_type, out_scale), out)


def test_gemm_ex_out_step_closed_form(orc):
    """out_scale is the output's step: y = 3 with step 0.5 encodes 6.0
    (E4M3 0 1001 100 = 0x4C), with step 2 encodes 1.5 (0x3C); a bf16 bias
    of -1 and an fp8 bias code 0x38 (1.0) with step 0.5 both add after the
    operand scaling and before the output's rounding; y = 1000 saturates at
    448 (0x7E) and y = -1e6 at -448 (0xFE)."""
    fmt = E4M3
    A = np.array([[0x38]], np.uint8)   # 1.0
    B = np.array([[0x40]], np.uint8)   # 2.0
    # y = 1 * 2 * (1.5 * 1) = 3
    out, y, _ = orc.gemm_ex(A, B, fmt, False, False, 1, 1, 1, 1.5, 1.0, out_type=1,
                            out_scale=0.5)
    assert y[0] == 3.0 and out[0] == 0x4C
    out, _, _ = orc.gemm_ex(A, B, fmt, False, False, 1, 1, 1, 1.5, 1.0, out_type=1,
                            out_scale=2.0)
    assert out[0] == 0x3C
    bneg = wl.f32_to_bf16_bits(np.array([-1.0], np.float32))
    out, y, _ = orc.gemm_ex(A, B, fmt, False, False, 1, 1, 1, 1.5, 1.0, bneg, out_type=1,
                            out_scale=0.5)
    assert y[0] == 2.0 and out[0] == 0x48                      # 4.0
    out, y, _ = orc.gemm_ex(A, B, fmt, False, False, 1, 1, 1, 1.5, 1.0,
                            np.array([0x38], np.uint8), 0.5, out_type=1, out_scale=0.5)
    assert y[0] == 3.5 and out[0] == 0x4E                      # 7.0
    assert orc.out_codes(np.array([1000.0, -1e6]), 1, 1.0).tolist() == [0x7E, 0xFE]
    assert orc.out_codes(np.array([1e9, -1e9]), 2, 1.0).tolist() == [0x7B, 0xFB]


def test_planted_mistakes_fp8_out(orc):
    """Slips in the extended epilogue change the oracle's codes."""
    fmt = E4M3
    M, N, K = 4, 6, 8
    A = orc.quantize(wl.normal_bf16((M, K), 1.0, 91), fmt, 1.0)
    B = orc.quantize(wl.normal_bf16((K, N), 1.0, 92), fmt, 1.0)
    b8 = orc.quantize(wl.normal_bf16((N,), 4.0, 93), fmt, 1.0)
    bs, sa, sb, so = np.float32(0.75), np.float32(0.5), np.float32(1.25), np.float32(0.0625)
    out, _, _ = orc.gemm_ex(A, B, fmt, False, False, M, N, K, sa, sb, b8, bs, 1, so)
    Ad, Bd = torch_decode(A, fmt), torch_decode(B, fmt)
    bv = torch_decode(b8, fmt).astype(np.float32) * bs
    s = float(sa * sb)
    r = np.float32(1.0) / so
    variants = {
        "step multiplied, not divided": (Ad @ Bd * s + bv).astype(np.float32) * so,
        "bias scale dropped": (Ad @ Bd * s + torch_decode(b8, fmt)).astype(np.float32) * r,
        "bias added after the output scaling": (Ad @ Bd * s).astype(np.float32) * r + bv,
        "operand scale dropped": (Ad @ Bd + bv).astype(np.float32) * r,
    }
    for name, v in variants.items():
        assert not np.array_equal(torch_encode(np.asarray(v, np.float32), E4M3).ravel(),
                                  out), name


def test_colsum_vs_torch(orc):
    g = wl.normal_bf16((300, 37), 1e-3, 41)
    ours = orc.colsum(g, 300, 37)
    ref = torch.from_numpy(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0).numpy()
    assert np.array_equal(ours, orc.bf16_from_f64(ref))


# --------------------------------------------------------------------------
# Delayed scaling (ring) and the linear layer
# --------------------------------------------------------------------------

def test_ring_train_closed_form(orc):
    """Config 'train' with x_t = s_t z: the x-ring scales and history follow
    in closed form from a = amax(z) (powers of two scale exactly)."""
    d = wl.train(M=64, N=48, K=32)
    M, N, K = d["M"], d["N"], d["K"]
    a = orc.amax(d["z"])
    aw = orc.amax(d["w"])
    rx, rw, rg = orc.Ring(16), orc.Ring(16), orc.Ring(16)
    sxs, sgs, ags = [], [], []
    for t in range(4):
        f = orc.linear_fwd(d["x"][t], d["w"], d["bias"], M, N, K, E4M3, False, rx, rw)
        b = orc.linear_bwd(d["g"][t], d["x"][t], d["w"], M, N, K, E5M2, False, f.sx, f.sw, rg)
        sxs.append(f.sx)
        sgs.append(b.sg)
        ags.append(orc.amax(d["g"][t]))
        assert f.sw == np.float32(aw / np.float32(448.0))
        assert b.sx == f.sx and b.sw == f.sw  # gradients reuse the forward scale
    f448 = np.float32(448.0)
    assert sxs == [a / f448, a / f448, np.float32(4 * a) / f448, np.float32(4 * a) / f448]
    expect_hist = np.zeros(16, np.float32)
    expect_hist[:4] = [a, 4 * a, a / 4, 2 * a]
    assert np.array_equal(rx.hist, expect_hist)
    assert rx.idx == 4 and rw.idx == 4 and rg.idx == 4
    f57 = np.float32(57344.0)
    assert sgs[0] == ags[0] / f57
    for t in range(1, 4):
        assert sgs[t] == np.float32(max(ags[:t])) / f57


def test_two_step_no_scale_ratio_leak(orc):
    """Step 2 (amax x4) dequantizes with the scale it quantized with (a/448),
    not the freshly published 4a/448."""
    d = wl.train(M=32, N=16, K=64, steps=2)
    M, N, K = d["M"], d["N"], d["K"]
    rx, rw = orc.Ring(16), orc.Ring(16)
    orc.linear_fwd(d["x"][0], d["w"], None, M, N, K, E4M3, False, rx, rw)
    f2 = orc.linear_fwd(d["x"][1], d["w"], None, M, N, K, E4M3, False, rx, rw)
    a = orc.amax(d["z"])
    assert f2.sx == a / np.float32(448.0)
    assert rx.scale == np.float32(4 * a) / np.float32(448.0)
    x8 = orc.quantize(d["x"][1], E4M3, f2.sx)
    w8 = orc.quantize(d["w"], E4M3, f2.sw)
    good = orc.gemm(x8, w8, E4M3, False, True, M, N, K, f2.sx, f2.sw)
    leak = orc.gemm(x8, w8, E4M3, False, True, M, N, K, rx.scale, f2.sw)
    assert np.array_equal(f2.out, good) and not np.array_equal(f2.out, leak)
    # leaking variant is off by exactly x4 (powers of two)
    r = wl.bf16_bits_to_f32(leak) / wl.bf16_bits_to_f32(good)
    ok = np.isfinite(r) & (wl.bf16_bits_to_f32(good) != 0)
    assert np.allclose(r[ok], 4.0)


def test_amax_is_raw_not_quantized(orc):
    """With the delayed scale lagging a 4x jump, the recorded amax exceeds
    448*s: it is the raw max, not the saturated quantized max."""
    d = wl.train(M=32, N=16, K=64, steps=2)
    rx, rw = orc.Ring(16), orc.Ring(16)
    orc.linear_fwd(d["x"][0], d["w"], None, 32, 16, 64, E4M3, False, rx, rw)
    f2 = orc.linear_fwd(d["x"][1], d["w"], None, 32, 16, 64, E4M3, False, rx, rw)
    assert rx.hist[1] > 448.0 * f2.sx * 3.9
    x8 = orc.quantize(d["x"][1], E4M3, f2.sx)
    assert ((x8 & 0x7F) == 0x7E).any()  # saturation happened


def test_linear_dynamic_vs_torch(orc):
    """Config linear256 at a reduced size: dynamic scales from the current
    amax, composed with torch library ops."""
    M, N, K = 8, 12, 16
    x = wl.normal_bf16((M, K), 1.0, 101)
    w = wl.normal_bf16((N, K), 0.02, 102)
    bias = wl.normal_bf16((N,), 0.1, 103)
    f = orc.linear_fwd(x, w, bias, M, N, K, E4M3, True)
    xf = torch.from_numpy(wl.bf16_bits_to_f32(x))
    wf = torch.from_numpy(wl.bf16_bits_to_f32(w))
    sx = (xf.abs().max() / 448.0).clamp_min(1e-12)
    sw = (wf.abs().max() / 448.0).clamp_min(1e-12)
    assert f.sx == sx.item() and f.sw == sw.item()
    x8 = torch_encode((xf * torch.reciprocal(sx)).numpy(), E4M3)
    w8 = torch_encode((wf * torch.reciprocal(sw)).numpy(), E4M3)
    ref = _torch_gemm_ref(orc, x8, w8.T, E4M3, sx.item(), sw.item(), bias)
    assert np.array_equal(f.out, ref)


def test_linear_bwd_layouts_vs_torch(orc):
    """dX = g w, dW = g^T x, db = colsum g, against float64 torch matmuls of
    the decoded E5M2 operands."""
    M, N, K = 9, 7, 5
    x = wl.normal_bf16((M, K), 1.0, 1)
    w = wl.normal_bf16((N, K), 0.02, 2)
    g = wl.normal_bf16((M, N), 1e-3, 3)
    sx, sw = np.float32(0.01), np.float32(0.0002)
    rg = orc.Ring(16)
    b = orc.linear_bwd(g, x, w, M, N, K, E5M2, False, sx, sw, rg)
    sg = orc.scale_from_peak(orc.amax(g), E5M2)
    assert b.sg == sg
    g8 = orc.quantize(g, E5M2, sg)
    x8 = orc.quantize(x, E5M2, sx)
    w8 = orc.quantize(w, E5M2, sw)
    assert np.array_equal(b.dx, _torch_gemm_ref(orc, g8, w8, E5M2, sg, sw, None))
    assert np.array_equal(b.dw, _torch_gemm_ref(orc, g8.T, x8, E5M2, sg, sx, None))
    ref_db = torch.from_numpy(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0).numpy()
    assert np.array_equal(b.db, orc.bf16_from_f64(ref_db))
    # dynamic backward measures sx, sw in the backward format
    bd = orc.linear_bwd(g, x, w, M, N, K, E5M2, True)
    assert bd.sx == orc.amax(x) / np.float32(57344.0)
    assert bd.sw == orc.amax(w) / np.float32(57344.0)


# --------------------------------------------------------------------------
# Planted mistakes: each slip in a Python copy of a definition must be
# caught by one of the independent references used above.
# --------------------------------------------------------------------------

def test_planted_mistakes(orc):
    M, N, K = 3, 4, 5
    # moderate magnitudes so that every term is visible at bf16 precision
    A = orc.quantize(wl.normal_bf16((M, K), 1.0, 71), E4M3, 1.0)
    B = orc.quantize(wl.normal_bf16((K, N), 1.0, 72), E4M3, 1.0)
    bias = wl.normal_bf16((N,), 5.0, 73)
    sa, sb = np.float32(0.5), np.float32(0.75)
    ref = _torch_gemm_ref(orc, A, B, E4M3, sa, sb, bias)
    Ad = torch_decode(A, E4M3)
    Bd = torch_decode(B, E4M3)
    bf = wl.bf16_bits_to_f32(bias).astype(np.float64)
    s = float(sa * sb)
    variants = {
        "dropped bias": Ad @ Bd * s,
        "dropped scale": Ad @ Bd + bf,
        "transposed operand": (Ad @ np.ascontiguousarray(Bd[::-1])) * s + bf,
        "wrong sign": -(Ad @ Bd) * s + bf,
        "sa only": Ad @ Bd * float(sa) + bf,
    }
    for name, y in variants.items():
        assert not np.array_equal(orc.bf16_from_f64(y), ref), name
    # a divide-instead-of-multiply quantize and a quantized-amax ring are
    # caught by test_quantize_multiplies_by_reciprocal / test_amax_is_raw.
