"""GPU parity of the quantize stage against the CPU oracle (bit-exact).

Covers fp8_quantize (cast, measure-only, ring fold, scale snapshot),
fp8_scale_ring_finalize and fp8_colsum on the configurations' tensors,
ragged / misaligned / empty inputs, and an exhaustive sweep of the fp32 ->
fp8 conversion through the kernel.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import (check_gemm, dev_f32, from_dev_bf16, from_dev_u8, ring_state_equal,
                            sum_bound, to_dev_bf16)

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def lib():
    import fp8_tensor_scaled_amd as f
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return f


def _is_nan_code(c, fmt):
    c = np.asarray(c)
    if fmt == E4M3:
        return (c & 0x7F) == 0x7F
    return ((c & 0x7C) == 0x7C) & ((c & 0x03) != 0)


def gpu_quantize(lib, x_bits, fmt, s, offset=0):
    """Quantize on the GPU; ``offset`` shifts both buffers to test
    misaligned bases."""
    n = x_bits.size
    xd = torch.zeros(n + offset, dtype=torch.int16, device="cuda")
    if n:
        xd[offset:] = to_dev_bf16(x_bits.ravel())
    out = torch.full((n + offset,), 0xAA, dtype=torch.uint8, device="cuda")
    sd = dev_f32(s)
    used = dev_f32(-1.0)
    lib.fp8_quantize(xd[offset:], fmt, scale=sd, out=out[offset:], scale_used=used)
    torch.cuda.synchronize()
    return from_dev_u8(out[offset:]), float(used.cpu()[0])


CASES = [
    ("linear256.x", lambda: wl.linear256()["x"]),
    ("linear256.w", lambda: wl.linear256()["w"]),
    ("smallm.w", lambda: wl.smallm()["w"]),
    ("train.x1", lambda: wl.train()["x"][1]),
    ("train.g0", lambda: wl.train()["g"][0]),
]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_quantize_config_tensors_bitexact(lib, orc, fmt, name, make):
    x = make()
    a = orc.amax(x)
    for s in (orc.scale_from_peak(a, fmt), orc.scale_from_peak(a / 8, fmt),
              np.float32(0.0137)):
        got, used = gpu_quantize(lib, x, fmt, s)
        ref = orc.quantize(x, fmt, s)
        assert used == np.float32(s)
        assert np.array_equal(got.reshape(ref.shape), ref), (name, fmt, s)


@pytest.mark.parametrize("n,offset", [(1, 0), (15, 0), (16, 0), (17, 0), (1000003, 0),
                                      (4096, 1), (4099, 3), (0, 0)])
def test_quantize_ragged_and_misaligned(lib, orc, n, offset):
    x = wl.normal_bf16((n,), 3.0, 1000 + n)
    for fmt in (E4M3, E5M2):
        s = np.float32(0.01)
        got, _ = gpu_quantize(lib, x, fmt, s, offset)
        assert np.array_equal(got, orc.quantize(x, fmt, s))


def test_quantize_special_values(lib, orc):
    """+-0, subnormal bf16, huge values (saturation), +-inf; NaN -> a NaN code."""
    vals = np.array([0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38, np.inf, -np.inf, 447.9, 449.0,
                     -464.0, 57344.0, 61440.0, 1e-6, 2.0 ** -10, 2.0 ** -17], np.float32)
    x = wl.f32_to_bf16_bits(vals)
    x = np.concatenate([x, np.array([0x7FC0, 0xFFC0], np.uint16)])
    for fmt in (E4M3, E5M2):
        got, _ = gpu_quantize(lib, x, fmt, np.float32(1.0))
        ref = orc.quantize(x, fmt, np.float32(1.0))
        nan = np.zeros(x.size, bool)
        nan[-2:] = True
        assert np.array_equal(got[~nan], ref[~nan])
        assert _is_nan_code(got[nan], fmt).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_conversion_bf16_times_multipliers(lib, orc, fmt):
    """Every bf16 input at several multipliers (fp32 products that round,
    overflow and underflow) through the bf16 quantize."""
    allbf = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for s in (np.float32(1.0), np.float32(1 / 3.0), np.float32(2.0 ** 20), np.float32(7e-5)):
        got, _ = gpu_quantize(lib, allbf, fmt, s)
        ref = orc.quantize(allbf, fmt, s)
        nan = _is_nan_code(ref, fmt)
        assert np.array_equal(got[~nan], ref[~nan])
        assert _is_nan_code(got[nan], fmt).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_conversion_exhaustive_fp32(lib, orc, fmt):
    """The cast on all 2^32 fp32 bit patterns: fp32 inputs through
    fp8_quantize_ex with step 1 (multiplier exactly 1, so the kernel converts
    each pattern itself), in chunks of 2^27 generated on the device, against
    the oracle's encode of the same patterns.  NaN patterns must give a NaN
    code; every other code is bit-exact."""
    chunk = 1 << 27
    one = dev_f32(1.0)
    idx = torch.arange(chunk, dtype=torch.int32, device="cuda")
    q = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for start in range(0, 1 << 32, chunk):
        signed = start - (1 << 32) if start >= (1 << 31) else start
        x = (idx + signed).view(torch.float32)
        lib.fp8_quantize_ex(x, fmt, scale=one, out=q, in_type=2)
        got = q.cpu().numpy()
        ref = orc.encode_bits_range(start, chunk, fmt)
        nan = _is_nan_code(ref, fmt)
        ok = (got == ref) | nan
        if not ok.all():
            i = int(np.argmin(ok))
            raise AssertionError(f"fmt {fmt} bits {start + i:#010x}: {got[i]:#x} vs {ref[i]:#x}")
        assert _is_nan_code(got[nan], fmt).all(), f"fmt {fmt} chunk {start:#x}: NaN codes"


def test_ring_fold_measure_and_quantize(lib, orc):
    """Delayed-scaling ring driven through fp8_quantize over four steps of
    the training config's x: seed (measure-only fold), then quantize with
    the published scale while the kernel folds; hist, scale and the scratch
    slots must match the oracle bit for bit."""
    d = wl.train()
    ring = lib.Ring(16)
    oring = orc.Ring(16)
    fmt = E4M3
    for t in range(4):
        x = d["x"][t]
        xd = to_dev_bf16(x.ravel())
        if t == 0:
            lib.fp8_quantize(xd, fmt, ring=ring)
            oring.seed(x, fmt)
        used = dev_f32(0.0)
        out = torch.empty(x.size, dtype=torch.uint8, device="cuda")
        lib.fp8_quantize(xd, fmt, scale=ring.scale, out=out, ring=ring, scale_used=used)
        s_snap = np.float32(oring.scale)
        ref = orc.quantize(x, fmt, s_snap)
        oring.fold(orc.amax(x), fmt)
        torch.cuda.synchronize()
        assert float(used.cpu()[0]) == s_snap
        assert np.array_equal(from_dev_u8(out), ref.ravel())
        assert ring_state_equal(ring, oring), (t, ring.state.cpu().numpy(), oring.state())
        ring.idx = (ring.idx + 1) % 16
        oring.advance()


def test_ring_fold_many_workgroups_and_empty(lib, orc):
    """A large tensor (thousands of workgroups) and an empty one both fold
    exactly once; a dirty scratch slot written from the host is not part of
    the contract, so the state is re-zeroed first."""
    x = wl.square(4096)["a"]
    ring = lib.Ring(4)
    ring.idx = 3
    lib.fp8_quantize(to_dev_bf16(x.ravel()), E5M2, ring=ring, margin=2)
    torch.cuda.synchronize()
    st = ring.state.cpu().numpy()
    a = orc.amax(x)
    assert st[3] == a
    assert st[4] == orc.scale_from_peak(a, E5M2, 2)
    assert st[6] == 0 and st[7] == 0 and not ring.scratch().cpu().numpy().any()
    # empty input folds amax 0 into slot 0
    ring.idx = 0
    lib.fp8_quantize(torch.empty(0, dtype=torch.int16, device="cuda"), E5M2, ring=ring,
                     margin=2)
    torch.cuda.synchronize()
    st = ring.state.cpu().numpy()
    assert st[0] == 0 and st[4] == orc.scale_from_peak(a, E5M2, 2)
    assert not ring.scratch().cpu().numpy().any()


@pytest.mark.parametrize("blocks", [1, 5, 16, 17, 37, 256])
def test_ring_fold_group_counts(lib, orc, blocks):
    """The fold's two-level reduction over workgroup counts below, at and
    above its 16 groups (uneven group sizes included), for the vector path
    (a ragged tail) and the unaligned scalar path, three folds in a row:
    hist and scale match the oracle, the scratch is zero after each."""
    rng = np.random.default_rng(blocks)
    numel = blocks * 1024 * 16 - 5  # the grid is ceil(numel / 16384) workgroups
    ring = lib.Ring(8)
    oring = orc.Ring(8)
    for t in range(3):
        x = wl.normal_bf16((numel,), float(rng.uniform(0.5, 4.0)), 1000 + 10 * blocks + t)
        offset = t % 2  # odd start: unaligned, scalar path
        xd = to_dev_bf16(np.concatenate([np.zeros(offset, np.uint16), x]))[offset:]
        lib.fp8_quantize(xd, E4M3, ring=ring)
        oring.fold(orc.amax(x), E4M3)
        torch.cuda.synchronize()
        assert ring_state_equal(ring, oring), (blocks, t)
        ring.idx = (ring.idx + 1) % 8
        oring.advance()


def test_scale_ring_finalize(lib, orc):
    ring = lib.Ring(16)
    oring = orc.Ring(16, margin=1)
    rng = np.random.default_rng(5)
    for t in range(20):
        a = np.float32(rng.uniform(0, 100))
        lib.fp8_scale_ring_finalize(ring, E4M3, dev_f32(a), margin=1)
        oring.fold(a, E4M3)
        torch.cuda.synchronize()
        assert ring_state_equal(ring, oring)
        ring.idx = (ring.idx + 1) % 16
        oring.advance()


@pytest.mark.parametrize("M,N", [(2048, 4096), (1, 7), (33, 8), (300, 1000), (70000, 16)])
def test_colsum(lib, orc, M, N):
    from tests.gpu_util import check_gemm, sum_bound
    g = wl.normal_bf16((M, N), 1e-3, 77 + M)
    ws = torch.empty(lib.fp8_colsum_workspace(M, N), dtype=torch.uint8, device="cuda")
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    lib.fp8_colsum(to_dev_bf16(g), M, N, db, ws)
    torch.cuda.synchronize()
    got = from_dev_bf16(db)
    ref = orc.colsum(g, M, N)
    absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
    check_gemm(got, ref, sum_bound(absg, M), what="colsum")
    # deterministic
    db2 = torch.empty_like(db)
    lib.fp8_colsum(to_dev_bf16(g), M, N, db2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(db2), got)


def test_invalid_arguments_raise(lib):
    x = torch.zeros(16, dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError):
        lib.fp8_quantize(x, 2, scale=dev_f32(1.0), out=torch.empty(16, dtype=torch.uint8,
                                                                   device="cuda"))
    with pytest.raises(ValueError):
        lib.fp8_quantize(x, 0)  # neither out nor ring
    r = lib.Ring(4)
    r.idx = 4
    with pytest.raises(ValueError):
        lib.fp8_quantize(x, 0, ring=r)


def test_quantize_large_tensor_shape(lib, orc):
    """From 2^25 elements the quantize sweeps in another launch shape (one
    16-element chunk per lane per round, up to 1024 workgroups).  At
    2^25 + 40 elements (a ragged tail): a ring seeded by a measure-only
    pass, then two steps that quantize with the published step while the
    kernel folds, then the dual-format pass and a max-only pass, all against
    the oracle bit for bit."""
    n = (1 << 25) + 40
    x = wl.normal_bf16((n,), 2.0, 4242)
    xd = to_dev_bf16(x)
    ring, oring = lib.Ring(16), orc.Ring(16)
    fmt = E4M3
    lib.fp8_quantize(xd, fmt, ring=ring)
    oring.seed(x, fmt)
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    used = dev_f32(0.0)
    for t in range(2):
        lib.fp8_quantize(xd, fmt, scale=ring.scale, out=out, ring=ring, scale_used=used)
        s_snap = np.float32(oring.scale)
        oring.fold(orc.amax(x), fmt)
        torch.cuda.synchronize()
        assert float(used.cpu()[0]) == s_snap, t
        assert np.array_equal(from_dev_u8(out), orc.quantize(x, fmt, s_snap)), t
        assert ring_state_equal(ring, oring), t
        ring.idx = (ring.idx + 1) % 16
        oring.advance()
    s = np.float32(0.0123)
    q2 = torch.empty(n, dtype=torch.uint8, device="cuda")
    lib.fp8_quantize2(xd, E4M3, dev_f32(s), out, E5M2, q2)
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    lib.fp8_quantize(xd, fmt, amax_out=am)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_u8(out), orc.quantize(x, E4M3, s))
    assert np.array_equal(from_dev_u8(q2), orc.quantize(x, E5M2, s))
    assert float(am.cpu()[0]) == orc.amax(x)


@pytest.mark.parametrize("fmt,fmt2", [(E4M3, E5M2), (E5M2, E4M3), (E4M3, E4M3)])
@pytest.mark.parametrize("numel,offset", [(4096 * 1024, 0), (100003, 0), (5000, 1)])
def test_quantize2_matches_two_single_quantizes(lib, orc, fmt, fmt2, numel, offset):
    """fp8_quantize2 writes, from one pass, the codes two fp8_quantize calls
    with the same step give (the second without a ring), and folds the ring
    like the first; checked against the oracle too.  `offset` misaligns the
    tensors (scalar path)."""
    x_all = wl.normal_bf16((numel + offset,), 3.0, 77 + numel % 13)
    x = x_all[offset:]
    s = np.float32(0.0123)
    xd = to_dev_bf16(x_all)[offset:]
    q1 = torch.empty(numel + offset, dtype=torch.uint8, device="cuda")[offset:]
    q2 = torch.empty(numel + offset, dtype=torch.uint8, device="cuda")[offset:]
    r1, r2 = lib.Ring(16), lib.Ring(16)
    sd = dev_f32(s)
    used = torch.zeros(1, dtype=torch.float32, device="cuda")
    lib.fp8_quantize2(xd, fmt, sd, q1, fmt2, q2, ring=r1, scale_used=used)
    a1 = torch.empty(numel, dtype=torch.uint8, device="cuda")
    a2 = torch.empty(numel, dtype=torch.uint8, device="cuda")
    lib.fp8_quantize(xd, fmt, scale=sd, out=a1, ring=r2)
    lib.fp8_quantize(xd, fmt2, scale=sd, out=a2)
    torch.cuda.synchronize()
    assert torch.equal(q1, a1) and torch.equal(q2, a2)
    assert np.array_equal(from_dev_u8(q1), orc.quantize(x, fmt, s))
    assert np.array_equal(from_dev_u8(q2), orc.quantize(x, fmt2, s))
    assert torch.equal(r1.state, r2.state)
    assert used.item() == s


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("M,N,offset", [(2048, 4096, 0), (777, 264, 0), (300, 136, 1),
                                         (50, 13, 0), (4096, 8, 0)])
def test_quantize_colsum_matches_separate_calls(lib, orc, fmt, M, N, offset):
    """fp8_quantize_colsum gives exactly fp8_quantize's codes, ring and
    scale_used and fp8_colsum's db (fused path for 8-column multiples on
    16-byte aligned rows, separate launches otherwise), and matches the
    oracle (codes bit-exact, db within the GEMM tolerance)."""
    g_all = wl.normal_bf16((M * N + offset,), 1e-3, M + N)
    g = g_all[offset:].reshape(M, N)
    gd = to_dev_bf16(g_all)[offset:]
    s = np.float32(1e-3 / 57344.0 * 4.0) if fmt else np.float32(1e-3 / 448.0 * 4.0)
    sd = dev_f32(s)
    ws = torch.empty(lib.fp8_colsum_workspace(M, N), dtype=torch.uint8, device="cuda")
    q1 = torch.empty(M * N, dtype=torch.uint8, device="cuda")
    db1 = torch.empty(N, dtype=torch.int16, device="cuda")
    u1 = torch.zeros(1, dtype=torch.float32, device="cuda")
    r1, r2 = lib.Ring(16), lib.Ring(16)
    lib.fp8_quantize_colsum(gd, M, N, fmt, sd, q1, db1, ws, ring=r1, scale_used=u1)
    q2 = torch.empty(M * N, dtype=torch.uint8, device="cuda")
    db2 = torch.empty(N, dtype=torch.int16, device="cuda")
    u2 = torch.zeros(1, dtype=torch.float32, device="cuda")
    lib.fp8_quantize(gd, fmt, scale=sd, out=q2, ring=r2, scale_used=u2)
    lib.fp8_colsum(gd, M, N, db2, ws)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(db1, db2)
    assert torch.equal(r1.state, r2.state) and torch.equal(u1, u2)
    assert np.array_equal(from_dev_u8(q1), orc.quantize(g.ravel(), fmt, s))
    ref = orc.colsum(g.ravel(), M, N)
    absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
    check_gemm(from_dev_bf16(db1), ref, sum_bound(absg, M), what=f"colsum {M}x{N}")


# ---------------------------------------------------------------------------
# fp16 and fp32 inputs (fp8_quantize_ex)
# ---------------------------------------------------------------------------

def gpu_quantize_ex(lib, x, in_type, fmt, s, offset=0, ring=None):
    """x: numpy uint16 bits (bf16 / fp16) or float32; ``offset`` elements of
    padding in front misalign both buffers."""
    n = x.size
    if in_type == 2:
        xd = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
        if n:
            xd[offset:] = torch.from_numpy(np.ascontiguousarray(x, np.float32).ravel()).cuda()
    else:
        xd = torch.zeros(n + offset, dtype=torch.int16, device="cuda")
        if n:
            xd[offset:] = torch.from_numpy(
                np.ascontiguousarray(x, np.uint16).ravel().view(np.int16)).cuda()
    out = torch.full((n + offset,), 0xAA, dtype=torch.uint8, device="cuda")
    used = dev_f32(-1.0)
    lib.fp8_quantize_ex(xd[offset:], fmt, scale=dev_f32(s), out=out[offset:], ring=ring,
                        scale_used=used, in_type=in_type)
    torch.cuda.synchronize()
    return from_dev_u8(out[offset:]), float(used.cpu()[0])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_ex_all_f16_patterns(lib, orc, fmt):
    """Every fp16 bit pattern at several multipliers, bit-exact against the
    oracle (NaN inputs give a NaN code)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    nan = np.isnan(orc.f16_to_f32(h))
    for s in (np.float32(1.0), np.float32(1 / 3.0), np.float32(2.0 ** 10), np.float32(7e-5)):
        got, used = gpu_quantize_ex(lib, h, 1, fmt, s)
        ref = orc.quantize_in(h, 1, fmt, s)
        assert used == s
        assert np.array_equal(got[~nan], ref[~nan]), s
        assert _is_nan_code(got[nan], fmt).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("n,offset", [(1, 0), (17, 0), (100003, 0), (4096, 1), (4099, 3)])
def test_quantize_ex_f32_and_f16_ragged(lib, orc, fmt, n, offset):
    """fp32 and fp16 inputs on ragged lengths and misaligned bases (scalar
    path), including values beyond bf16 precision and the formats' ranges."""
    rng = np.random.default_rng(n + offset)
    x32 = (rng.standard_normal(n) * rng.choice([1e-3, 1.0, 300.0, 1e5], n)).astype(np.float32)
    x16 = np.clip(x32, -6e4, 6e4).astype(np.float16).view(np.uint16)
    s = np.float32(0.0173)
    for in_type, x in ((2, x32), (1, x16)):
        got, _ = gpu_quantize_ex(lib, x, in_type, fmt, s, offset)
        assert np.array_equal(got, orc.quantize_in(x, in_type, fmt, s)), in_type


def test_quantize_ex_ring_fold_and_same_values(lib, orc):
    """The fold with fp16 / fp32 inputs records max |x| exactly, and the same
    values given as bf16, fp16 and fp32 give the same codes and amax."""
    v = wl.bf16_bits_to_f32(wl.normal_bf16((3000,), 2.0, 77))
    v = v[np.abs(v) < 6e4]
    v16 = v.astype(np.float16)
    v = v16.astype(np.float32)[np.isfinite(v16)]
    keep = (v.view(np.uint32) & 0xFFFF) == 0  # exact in bf16 as well
    v = v[keep]
    b = (v.view(np.uint32) >> 16).astype(np.uint16)
    h = v.astype(np.float16).view(np.uint16)
    for fmt in (E4M3, E5M2):
        s = orc.scale_from_peak(orc.amax(b), fmt)
        codes = [gpu_quantize_ex(lib, x, t, fmt, s)[0] for t, x in ((0, b), (1, h), (2, v))]
        assert np.array_equal(codes[0], codes[1]) and np.array_equal(codes[0], codes[2])
        assert np.array_equal(codes[0], orc.quantize(b, fmt, s))
    x32 = (np.random.default_rng(5).standard_normal(50000) * 7.0).astype(np.float32)
    for in_type, x in ((2, x32), (1, x32.astype(np.float16).view(np.uint16))):
        ring, oring = lib.Ring(4), orc.Ring(4)
        for t in range(3):
            xt = x if in_type == 1 else x * np.float32(1 + t)
            gpu_quantize_ex(lib, xt, in_type, E4M3, np.float32(1.0), ring=ring)
            oring.fold(orc.amax_in(xt, in_type), E4M3)
            assert ring_state_equal(ring, oring), (in_type, t)
            ring.idx = (ring.idx + 1) % 4
            oring.advance()


# ---------------------------------------------------------------------------
# Transposed / dual-orientation quantize (fp8_quantize_t)
# ---------------------------------------------------------------------------

def gpu_quantize_t(lib, x, fmt, s, dual, offset=0, ring=None):
    rows, cols = x.shape
    n = x.size
    xd = torch.zeros(n + offset, dtype=torch.int16, device="cuda")
    xd[offset:] = to_dev_bf16(x.ravel())
    out_t = torch.full((n + offset,), 0xAA, dtype=torch.uint8, device="cuda")
    out = torch.full((n + offset,), 0xAA, dtype=torch.uint8, device="cuda") if dual else None
    used = dev_f32(-1.0)
    lib.fp8_quantize_t(xd[offset:], rows, cols, fmt, dev_f32(s), out_t[offset:],
                       out=None if out is None else out[offset:], ring=ring, scale_used=used)
    torch.cuda.synchronize()
    q = from_dev_u8(out[offset:]).reshape(rows, cols) if dual else None
    return q, from_dev_u8(out_t[offset:]).reshape(cols, rows), float(used.cpu()[0])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rows,cols,offset", [(4096, 4096, 0), (256, 384, 0), (272, 136, 0),
                                              (16, 8, 0), (100, 36, 0), (33, 17, 0),
                                              (128, 128, 1), (2048, 1024, 0)])
def test_quantize_t_matches_oracle(lib, orc, fmt, rows, cols, offset):
    """Transposed and dual-orientation codes, bit-exact, on full tiles,
    partial tiles, the per-element path (rows % 16, cols % 8, misaligned
    base) and the training config's x shape."""
    x = wl.normal_bf16((rows, cols), 2.0, rows * 7 + cols)
    s = orc.scale_from_peak(orc.amax(x), fmt)
    q_ref, qt_ref = orc.quantize_t(x, fmt, s)
    for dual in (False, True):
        q, qt, used = gpu_quantize_t(lib, x, fmt, s, dual, offset)
        assert used == s
        assert np.array_equal(qt, qt_ref), dual
        if dual:
            assert np.array_equal(q, q_ref)


def test_quantize_t_ring_fold(lib, orc):
    """The dual pass folds max |x| into its ring like the quantize."""
    ring, oring = lib.Ring(8), orc.Ring(8)
    for t in range(3):
        x = wl.normal_bf16((512, 768), 1.0 + t, 40 + t)
        gpu_quantize_t(lib, x, E5M2, np.float32(0.5), True, ring=ring)
        oring.fold(orc.amax(x), E5M2)
        assert ring_state_equal(ring, oring), t
        ring.idx = (ring.idx + 1) % 8
        oring.advance()


def test_backward_nt_only_route(lib, orc):
    """The pages' NT-only backward (dual quantize of g, transposed copies of
    x and w, two NT GEMMs) against the oracle's dX and dW."""
    M, N, K = 2048, 1024, 512
    g = wl.normal_bf16((M, N), 1e-3, 60)
    x = wl.normal_bf16((M, K), 1.0, 61)
    w = wl.normal_bf16((N, K), 0.02, 62)
    fmt = E5M2
    sg = orc.scale_from_peak(orc.amax(g), fmt)
    sx = orc.scale_from_peak(orc.amax(x), fmt)
    sw = orc.scale_from_peak(orc.amax(w), fmt)
    g8, g8t = (torch.empty(M * N, dtype=torch.uint8, device="cuda") for _ in range(2))
    x8t = torch.empty(M * K, dtype=torch.uint8, device="cuda")
    w8t = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    dsg, dsx, dsw = dev_f32(sg), dev_f32(sx), dev_f32(sw)
    lib.fp8_quantize_t(to_dev_bf16(g.ravel()), M, N, fmt, dsg, g8t, out=g8)
    lib.fp8_quantize_t(to_dev_bf16(x.ravel()), M, K, fmt, dsx, x8t)
    lib.fp8_quantize_t(to_dev_bf16(w.ravel()), N, K, fmt, dsw, w8t)
    dx = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dw = torch.empty(N * K, dtype=torch.int16, device="cuda")
    # dX[M][K] = g8 [M][N] . w8^T stored [K][N] (NT);  dW[N][K] = g8^T [N][M] . x8^T [K][M] (NT)
    lib.fp8_mm(g8, w8t, fmt, 0, 1, M, K, N, N, N, 1, 0, 0, dsg, dsw, None, dx)
    lib.fp8_mm(g8t, x8t, fmt, 0, 1, N, K, M, M, M, 1, 0, 0, dsg, dsx, None, dw)
    torch.cuda.synchronize()
    g8r, x8r, w8r = orc.quantize(g, fmt, sg), orc.quantize(x, fmt, sx), orc.quantize(w, fmt, sw)
    assert np.array_equal(from_dev_u8(g8), g8r.ravel())
    ref_dx = orc.gemm(g8r, w8r, fmt, False, False, M, K, N, sg, sw)
    ad_dx = orc.gemm_bound(g8r, w8r, fmt, False, False, M, K, N, sg, sw)
    check_gemm(from_dev_bf16(dx).reshape(M, K), ref_dx, ad_dx, "nt-route dX")
    ref_dw = orc.gemm(g8r, x8r, fmt, True, False, N, K, M, sg, sx)
    ad_dw = orc.gemm_bound(g8r, x8r, fmt, True, False, N, K, M, sg, sx)
    check_gemm(from_dev_bf16(dw).reshape(N, K), ref_dw, ad_dw, "nt-route dW")


# ---------------------------------------------------------------------------
# amax_out: the quantize's max |x| output
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("numel,offset", [(4096 * 4096, 0), (65536 * 3 + 5, 0), (1000, 1),
                                          (16, 0), (1, 3), (0, 0)])
def test_amax_out_without_ring(lib, orc, numel, offset):
    """No ring: a quantizing call and a measure-only call both return the
    oracle's amax bit for bit, over many workgroups (atomic max after the
    arming launch), on the scalar path and for empty input (+0).  The
    output starts with garbage: the library arms it."""
    x = wl.normal_bf16((numel,), 3.0, numel % 1000 + offset)
    if numel > 7:
        x[numel // 3] = wl.f32_to_bf16_bits(np.array([-1234.0], np.float32))[0]
    xd = torch.zeros(numel + offset, dtype=torch.int16, device="cuda")
    if numel:
        xd[offset:] = to_dev_bf16(x)
    ref = np.float32(orc.amax(x)) if numel else np.float32(0.0)
    for out in (True, False):
        amax = dev_f32(-7.0)
        q = torch.empty(numel + offset, dtype=torch.uint8, device="cuda") if out else None
        s = dev_f32(0.5)
        lib.fp8_quantize(xd[offset:], E4M3, scale=s if out else None,
                         out=q[offset:] if out else None, amax_out=amax)
        torch.cuda.synchronize()
        got = amax.cpu().numpy()[0]
        assert got == ref and not np.signbit(got), (numel, offset, out, got, ref)
        if out and numel:
            assert np.array_equal(from_dev_u8(q[offset:]), orc.quantize(x, E4M3, 0.5))


def test_amax_out_with_ring_equals_fold(lib, orc):
    """With a ring the folding workgroup writes amax_out: the value it puts
    into hist[idx], over several calls that move idx."""
    ring = lib.Ring(4)
    oring = orc.Ring(4)
    for t, factor in enumerate((1.0, 8.0, 0.25)):
        x = wl.scaled_bf16(wl.normal_bf16((2048, 1024), 1.0, 70 + t), factor)
        amax = dev_f32(-1.0)
        lib.fp8_quantize(to_dev_bf16(x), E5M2, ring=ring, amax_out=amax)
        torch.cuda.synchronize()
        oring.fold(orc.amax(x), E5M2)
        got = amax.cpu().numpy()[0]
        assert got == np.float32(orc.amax(x)) == ring.state.cpu().numpy()[ring.idx]
        assert ring_state_equal(ring, oring)
        ring.idx = (ring.idx + 1) % ring.len
        oring.advance()


@pytest.mark.parametrize("dt,in_type", [(torch.float16, 1), (torch.float32, 2)])
def test_amax_out_fp16_fp32_inputs(lib, orc, dt, in_type):
    x = (torch.randn(1 << 20, generator=torch.Generator().manual_seed(5)) * 7).to(dt)
    x[777] = -60000.0 if dt == torch.float16 else -1e9
    amax = dev_f32(-1.0)
    lib.fp8_quantize_ex(x.cuda(), E4M3, amax_out=amax)
    torch.cuda.synchronize()
    raw = x.numpy().view(np.uint16 if dt == torch.float16 else np.float32)
    assert amax.cpu().numpy()[0] == np.float32(orc.amax_in(raw, in_type))
