"""GPU parity of the linear-layer entry points against the CPU oracle.

linear256: dynamic-scaling E4M3 forward at 256^3 (full output compare).
train: delayed-scaling HYBRID forward + backward over four steps with the
input scaled 1, 4, 0.25, 2 -- scales, rings and fp8 operands bit-exact every
step, GEMM outputs at sampled coordinates, bias gradient in full.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import (check_gemm, from_dev_bf16, from_dev_u8, ring_state_equal, sum_bound,
                            to_dev_bf16)

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def lib():
    import fp8_tensor_scaled_amd as f
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return f


class Fwd:
    def __init__(self, lib, M, N, K):
        self.ws = torch.zeros(lib.fp8_linear_fwd_workspace(M, N, K), dtype=torch.uint8,
                              device="cuda")
        self.x8_off = lib.fp8_linear_fwd_x8_offset(M, N, K)
        self.w8_off = lib.fp8_linear_fwd_w8_offset(M, N, K)
        self.scales = torch.zeros(2, dtype=torch.float32, device="cuda")
        self.out = torch.empty(M * N, dtype=torch.int16, device="cuda")
        self.M, self.N, self.K = M, N, K

    def x8(self):
        return from_dev_u8(self.ws[self.x8_off: self.x8_off + self.M * self.K])

    def w8(self):
        return from_dev_u8(self.ws[self.w8_off: self.w8_off + self.N * self.K])


def test_linear256_dynamic_forward(lib, orc):
    d = wl.linear256()
    M, N, K = d["M"], d["N"], d["K"]
    f = Fwd(lib, M, N, K)
    # The workspace's scratch rings re-arm themselves: the second call (other
    # amaxes, so a scale left over from the first would fail) reuses it.
    for rep, (fx, fw) in enumerate(((1.0, 1.0), (4.0, 0.25))):
        x, w = wl.scaled_bf16(d["x"], fx), wl.scaled_bf16(d["w"], fw)
        lib.fp8_linear_fwd(to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(d["bias"]),
                           M, N, K, E4M3, True, 0, None, None, f.ws, f.scales, f.out)
        torch.cuda.synchronize()
        ref = orc.linear_fwd(x, w, d["bias"], M, N, K, E4M3, True)
        sc = f.scales.cpu().numpy()
        assert sc[0] == ref.sx and sc[1] == ref.sw, rep
        assert np.array_equal(f.x8(), ref.x8.ravel()), rep
        assert np.array_equal(f.w8(), ref.w8.ravel()), rep
        bound = orc.gemm_bound(ref.x8, ref.w8, E4M3, False, True, M, N, K, ref.sx, ref.sw)
        check_gemm(from_dev_bf16(f.out).reshape(M, N), ref.out, bound, f"linear256 {rep}")


def test_dynamic_backward_reused_workspace(lib, orc):
    # Tensors of 8 to 20 quantize workgroups, so every amax reduction uses
    # several group lines of its scratch ring; the g8 codes the first call
    # writes sit right after those rings.  Second call: other amaxes.
    M, N, K = 256, 384, 640
    x0 = wl.normal_bf16((M, K), 1.0, 31)
    w0 = wl.normal_bf16((N, K), 0.02, 32)
    g0 = wl.normal_bf16((M, N), 1e-3, 33)
    ws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    dummy = torch.zeros(2, dtype=torch.float32, device="cuda")
    so = torch.zeros(3, dtype=torch.float32, device="cuda")
    dx = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dw = torch.empty(N * K, dtype=torch.int16, device="cuda")
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    g8_off = lib.fp8_linear_fwd_x8_offset(M, N, K)
    for rep, (fg, fx, fw) in enumerate(((1.0, 1.0, 1.0), (8.0, 0.5, 4.0))):
        g, x, w = wl.scaled_bf16(g0, fg), wl.scaled_bf16(x0, fx), wl.scaled_bf16(w0, fw)
        lib.fp8_linear_bwd(to_dev_bf16(g), to_dev_bf16(x), to_dev_bf16(w), M, N, K, E5M2, True,
                           0, dummy, None, ws, so, dx, dw, db)
        torch.cuda.synchronize()
        rb = orc.linear_bwd(g, x, w, M, N, K, E5M2, True, 0.0, 0.0, None)
        s = so.cpu().numpy()
        assert (s[0], s[1], s[2]) == (rb.sg, rb.sx, rb.sw), rep
        assert np.array_equal(from_dev_u8(ws[g8_off: g8_off + M * N]), rb.g8.ravel()), rep
        w8b = orc.quantize(w, E5M2, rb.sw)
        ad = orc.gemm_bound(rb.g8, w8b, E5M2, False, False, M, K, N, rb.sg, rb.sw)
        check_gemm(from_dev_bf16(dx).reshape(M, K), rb.dx, ad, f"dx {rep}")
        x8b = orc.quantize(x, E5M2, rb.sx)
        ad = orc.gemm_bound(rb.g8, x8b, E5M2, True, False, N, K, M, rb.sg, rb.sx)
        check_gemm(from_dev_bf16(dw).reshape(N, K), rb.dw, ad, f"dw {rep}")
        absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
        check_gemm(from_dev_bf16(db), rb.db, sum_bound(absg, M), f"db {rep}")


def _samples(M, N, n, seed):
    rng = np.random.default_rng(seed)
    return (np.zeros(n, np.int64), rng.integers(0, M, n), rng.integers(0, N, n))


def test_train_delayed_hybrid_four_steps(lib, orc):
    d = wl.train()
    M, N, K = d["M"], d["N"], d["K"]
    f = Fwd(lib, M, N, K)
    bws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    rx, rw, rg = lib.Ring(16), lib.Ring(16), lib.Ring(16)
    ox, ow, og = orc.Ring(16), orc.Ring(16), orc.Ring(16)
    wd, bd = to_dev_bf16(d["w"]), to_dev_bf16(d["bias"])
    dx = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dw = torch.empty(N * K, dtype=torch.int16, device="cuda")
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    sb = torch.zeros(3, dtype=torch.float32, device="cuda")
    for t in range(4):
        xd, gd = to_dev_bf16(d["x"][t]), to_dev_bf16(d["g"][t])
        lib.fp8_linear_fwd(xd, wd, bd, M, N, K, E4M3, False, 0, rx, rw, f.ws, f.scales, f.out)
        lib.fp8_linear_bwd(gd, xd, wd, M, N, K, E5M2, False, 0, f.scales, rg, bws, sb, dx, dw,
                           db)
        torch.cuda.synchronize()
        rf = orc.linear_fwd(d["x"][t], d["w"], d["bias"], M, N, K, E4M3, False, ox, ow)
        rb = orc.linear_bwd(d["g"][t], d["x"][t], d["w"], M, N, K, E5M2, False, rf.sx, rf.sw,
                            og)
        # scales, rings and fp8 operands: bit-exact
        sc = f.scales.cpu().numpy()
        assert (sc[0], sc[1]) == (rf.sx, rf.sw), t
        sbh = sb.cpu().numpy()
        assert (sbh[0], sbh[1], sbh[2]) == (rb.sg, rb.sx, rb.sw), t
        for gr, orr in ((rx, ox), (rw, ow), (rg, og)):
            assert ring_state_equal(gr, orr), t
            assert gr.idx == orr.idx and gr.initialized == orr.initialized
        assert np.array_equal(f.x8(), rf.x8.ravel())
        assert np.array_equal(f.w8(), rf.w8.ravel())
        g8_off = lib.fp8_linear_fwd_x8_offset(M, N, K)
        g8 = from_dev_u8(bws[g8_off: g8_off + M * N])
        assert np.array_equal(g8, rb.g8.ravel())
        # GEMM outputs at sampled coordinates
        s = _samples(M, N, 2000, t)
        ref, ad = orc.gemm_sampled(rf.x8, rf.w8, E4M3, False, True, M, N, K, rf.sx, rf.sw,
                                   d["bias"], s)
        check_gemm(from_dev_bf16(f.out).reshape(M, N)[s[1], s[2]], ref, ad, f"fwd {t}")
        w8b = orc.quantize(d["w"], E5M2, rb.sw)
        x8b = orc.quantize(d["x"][t], E5M2, rb.sx)
        s = _samples(M, K, 2000, 10 + t)
        ref, ad = orc.gemm_sampled(rb.g8, w8b, E5M2, False, False, M, K, N, rb.sg, rb.sw, None,
                                   s)
        check_gemm(from_dev_bf16(dx).reshape(M, K)[s[1], s[2]], ref, ad, f"dX {t}")
        s = _samples(N, K, 2000, 20 + t)
        ref, ad = orc.gemm_sampled(rb.g8, x8b, E5M2, True, False, N, K, M, rb.sg, rb.sx, None,
                                   s)
        check_gemm(from_dev_bf16(dw).reshape(N, K)[s[1], s[2]], ref, ad, f"dW {t}")
        absg = np.abs(wl.bf16_bits_to_f32(d["g"][t]).astype(np.float64)).sum(0)
        check_gemm(from_dev_bf16(db), rb.db, sum_bound(absg, M), f"db {t}")


@pytest.mark.parametrize("dynamic", [True, False])
def test_backward_masks_and_dynamic_small(lib, orc, dynamic):
    M, N, K = 96, 80, 112
    x = wl.normal_bf16((M, K), 1.0, 1)
    w = wl.normal_bf16((N, K), 0.02, 2)
    g = wl.normal_bf16((M, N), 1e-3, 3)
    sx, sw = np.float32(0.004), np.float32(2e-4)
    scales_fwd = torch.tensor([sx, sw], dtype=torch.float32, device="cuda")
    ws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    for need in [(1, 1, 1), (1, 0, 0), (0, 1, 0), (0, 0, 1)]:
        rg = None if dynamic else lib.Ring(16)
        og = None if dynamic else orc.Ring(16)
        dx = torch.empty(M * K, dtype=torch.int16, device="cuda") if need[0] else None
        dw = torch.empty(N * K, dtype=torch.int16, device="cuda") if need[1] else None
        db = torch.empty(N, dtype=torch.int16, device="cuda") if need[2] else None
        lib.fp8_linear_bwd(to_dev_bf16(g), to_dev_bf16(x), to_dev_bf16(w), M, N, K, E5M2,
                           dynamic, 0, scales_fwd, rg, ws, None, dx, dw, db)
        torch.cuda.synchronize()
        rb = orc.linear_bwd(g, x, w, M, N, K, E5M2, dynamic, sx, sw, og, bool(need[0]),
                            bool(need[1]), bool(need[2]))
        if need[0]:
            w8b = orc.quantize(w, E5M2, rb.sw)
            ad = orc.gemm_bound(rb.g8, w8b, E5M2, False, False, M, K, N, rb.sg, rb.sw)
            check_gemm(from_dev_bf16(dx).reshape(M, K), rb.dx, ad, "dx")
        if need[1]:
            x8b = orc.quantize(x, E5M2, rb.sx)
            ad = orc.gemm_bound(rb.g8, x8b, E5M2, True, False, N, K, M, rb.sg, rb.sx)
            check_gemm(from_dev_bf16(dw).reshape(N, K), rb.dw, ad, "dw")
        if need[2]:
            absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
            check_gemm(from_dev_bf16(db), rb.db, sum_bound(absg, M), "db")
        if not dynamic:
            assert ring_state_equal(rg, og)


@pytest.mark.parametrize("M,N,K", [(48, 256, 128), (80, 96, 40), (300, 136, 272)])
def test_delayed_steps_on_every_gemm_kernel(lib, orc, M, N, K):
    """Delayed scaling over three steps (the input rescaled each step, so
    every fold changes the window) on shapes whose forward GEMM takes each
    kernel family: short-A (M <= 64), the general kernel (K not a multiple
    of 16) and the tiled one with ragged tiles.  The linear calls gather
    each ring's amax in their quantize and fold it in a later launch (an
    extra workgroup of the tiled forward GEMM or of the paired backward,
    else a launch of its own): every step's steps, rings, codes and
    outputs against the oracle."""
    x0 = wl.normal_bf16((M, K), 1.0, 41)
    w = wl.normal_bf16((N, K), 0.02, 42)
    bias = wl.normal_bf16((N,), 0.1, 43)
    f = Fwd(lib, M, N, K)
    bws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    rx, rw, rg = lib.Ring(16), lib.Ring(16), lib.Ring(16)
    ox, ow, og = orc.Ring(16), orc.Ring(16), orc.Ring(16)
    dx = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dw = torch.empty(N * K, dtype=torch.int16, device="cuda")
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    sb = torch.zeros(3, dtype=torch.float32, device="cuda")
    wd, bd = to_dev_bf16(w), to_dev_bf16(bias)
    for t, s in enumerate((1.0, 8.0, 0.125)):
        x = wl.scaled_bf16(x0, s)
        g = wl.normal_bf16((M, N), 1e-3 * (t + 1), 44 + t)
        xd, gd = to_dev_bf16(x), to_dev_bf16(g)
        lib.fp8_linear_fwd(xd, wd, bd, M, N, K, E4M3, False, 0, rx, rw, f.ws, f.scales, f.out)
        lib.fp8_linear_bwd(gd, xd, wd, M, N, K, E5M2, False, 0, f.scales, rg, bws, sb, dx, dw,
                           db)
        torch.cuda.synchronize()
        rf = orc.linear_fwd(x, w, bias, M, N, K, E4M3, False, ox, ow)
        rb = orc.linear_bwd(g, x, w, M, N, K, E5M2, False, rf.sx, rf.sw, og)
        sc = f.scales.cpu().numpy()
        assert (sc[0], sc[1]) == (rf.sx, rf.sw), t
        sbh = sb.cpu().numpy()
        assert (sbh[0], sbh[1], sbh[2]) == (rb.sg, rb.sx, rb.sw), t
        for gr, orr in ((rx, ox), (rw, ow), (rg, og)):
            assert ring_state_equal(gr, orr), t
            assert gr.idx == orr.idx
        assert np.array_equal(f.x8(), rf.x8.ravel()), t
        assert np.array_equal(f.w8(), rf.w8.ravel()), t
        bound = orc.gemm_bound(rf.x8, rf.w8, E4M3, False, True, M, N, K, rf.sx, rf.sw)
        check_gemm(from_dev_bf16(f.out).reshape(M, N), rf.out, bound, f"fwd {t}")
        w8b = orc.quantize(w, E5M2, rb.sw)
        x8b = orc.quantize(x, E5M2, rb.sx)
        ad = orc.gemm_bound(rb.g8, w8b, E5M2, False, False, M, K, N, rb.sg, rb.sw)
        check_gemm(from_dev_bf16(dx).reshape(M, K), rb.dx, ad, f"dx {t}")
        ad = orc.gemm_bound(rb.g8, x8b, E5M2, True, False, N, K, M, rb.sg, rb.sx)
        check_gemm(from_dev_bf16(dw).reshape(N, K), rb.dw, ad, f"dw {t}")
        absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
        check_gemm(from_dev_bf16(db), rb.db, sum_bound(absg, M), f"db {t}")


def test_linear_invalid_arguments(lib):
    M, N, K = 32, 32, 32
    ws = torch.zeros(16, dtype=torch.uint8, device="cuda")
    x = torch.zeros(M * K, dtype=torch.int16, device="cuda")
    sc = torch.zeros(2, dtype=torch.float32, device="cuda")
    out = torch.empty(M * N, dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        lib.fp8_linear_fwd(x, x, None, M, N, K, E4M3, True, 0, None, None, ws, sc, out)
    ws = torch.zeros(lib.fp8_linear_fwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="ring"):
        lib.fp8_linear_fwd(x, x, None, M, N, K, E4M3, False, 0, None, None, ws, sc, out)


def test_benchmark_step_4096_vs_oracle(lib, orc):
    """The benchmark's own step (bench.Layer at M = N = K = 4096, delayed
    HYBRID, ring 16, bias), in the launch configuration the benchmark
    times: seeded, then two steps.  Every code array, step and ring is
    compared bit for bit with the oracle's quantize and fold; the NT output,
    dX and dW at sampled coordinates, and the bias gradient in full, within
    the GEMM tolerance."""
    import bench
    n = 4096
    L = bench.Layer(lib, torch, n)
    host = {k: from_dev_bf16(getattr(L, k)) for k in ("x", "w", "bias", "g")}
    x, w, bias, g = host["x"], host["w"], host["bias"], host["g"]
    ox, ow, og = orc.Ring(16), orc.Ring(16), orc.Ring(16)
    L.seed(lib)
    ow.seed(w, E4M3)
    ox.seed(x, E4M3)
    og.seed(g, E5M2)
    amax_x, amax_w, amax_g = orc.amax(x), orc.amax(w), orc.amax(g)
    absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
    for t in range(2):
        L.step(lib)
        torch.cuda.synchronize()
        # the oracle's steps, in the kernels' order
        sx, sw, sg = np.float32(ox.scale), np.float32(ow.scale), np.float32(og.scale)
        x8, x8b = orc.quantize(x, E4M3, sx), orc.quantize(x, E5M2, sx)
        ox.fold(amax_x, E4M3)
        w8, w8b = orc.quantize(w, E4M3, sw), orc.quantize(w, E5M2, sw)
        ow.fold(amax_w, E4M3)
        g8 = orc.quantize(g, E5M2, sg)
        og.fold(amax_g, E5M2)
        for r in (ox, ow, og):
            r.advance()
        sc = L.sfwd.cpu().numpy()
        assert (sc[0], sc[1], L.sg.cpu().numpy()[0]) == (sx, sw, sg), t
        for got, ref, name in ((L.x8, x8, "x8"), (L.x8b, x8b, "x8b"), (L.w8, w8, "w8"),
                               (L.w8b, w8b, "w8b"), (L.g8, g8, "g8")):
            assert np.array_equal(from_dev_u8(got), ref.ravel()), (t, name)
        for gr, orr in ((L.rx, ox), (L.rw, ow), (L.rg, og)):
            assert ring_state_equal(gr, orr) and gr.idx == orr.idx, t
        s = _samples(n, n, 2000, 40 + t)
        ref, ad = orc.gemm_sampled(x8, w8, E4M3, False, True, n, n, n, sx, sw, bias, s)
        check_gemm(from_dev_bf16(L.out).reshape(n, n)[s[1], s[2]], ref, ad, f"step fwd {t}")
        s = _samples(n, n, 2000, 50 + t)
        ref, ad = orc.gemm_sampled(g8, w8b, E5M2, False, False, n, n, n, sg, sw, None, s)
        check_gemm(from_dev_bf16(L.dx).reshape(n, n)[s[1], s[2]], ref, ad, f"step dX {t}")
        s = _samples(n, n, 2000, 60 + t)
        ref, ad = orc.gemm_sampled(g8, x8b, E5M2, True, False, n, n, n, sg, sx, None, s)
        check_gemm(from_dev_bf16(L.dw).reshape(n, n)[s[1], s[2]], ref, ad, f"step dW {t}")
        check_gemm(from_dev_bf16(L.db), orc.colsum(g, n, n), sum_bound(absg, n), f"step db {t}")


def test_delayed_forward_two_tensor_quantize_large_shape(lib, orc):
    """x [3001, 4200] and w [5003, 4200]: 2^25 elements and more in all, so
    the forward's one-launch quantize of x and w (one chunk per lane per
    round) runs at its grid cap, 1024 workgroups split in proportion to the
    sizes, several rounds each, with ragged tensor ends.  Three delayed steps
    with the backward's codes written by the same pass: every code array,
    step and ring bit-exact against the oracle, the output sampled."""
    M, N, K = 3001, 5003, 4200
    assert M * K + N * K >= 1 << 25
    x = wl.normal_bf16((M, K), 1.0, 91)
    w = wl.normal_bf16((N, K), 0.02, 92)
    bias = wl.normal_bf16((N,), 0.1, 93)
    xd, wd, bd = to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(bias)
    f = Fwd(lib, M, N, K)
    rx, rw = lib.Ring(16), lib.Ring(16)
    ox, ow = orc.Ring(16), orc.Ring(16)
    lib.fp8_quantize(wd, E4M3, ring=rw)
    lib.fp8_quantize(xd, E4M3, ring=rx)
    rx.initialized = rw.initialized = True
    ow.seed(w, E4M3)
    ox.seed(x, E4M3)
    amax_x, amax_w = orc.amax(x), orc.amax(w)
    x8b = torch.empty(M * K, dtype=torch.uint8, device="cuda")
    w8b = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    for t in range(3):
        lib.fp8_linear_fwd(xd, wd, bd, M, N, K, E4M3, False, 0, rx, rw, f.ws, f.scales, f.out,
                           fmt_bwd=E5M2, x8_bwd=x8b, w8_bwd=w8b)
        torch.cuda.synchronize()
        sx, sw = np.float32(ox.scale), np.float32(ow.scale)
        x8, w8 = orc.quantize(x, E4M3, sx), orc.quantize(w, E4M3, sw)
        ox.fold(amax_x, E4M3)
        ow.fold(amax_w, E4M3)
        for r in (ox, ow):
            r.advance()
        sc = f.scales.cpu().numpy()
        assert (sc[0], sc[1]) == (sx, sw), t
        assert np.array_equal(f.x8(), x8.ravel()), t
        assert np.array_equal(f.w8(), w8.ravel()), t
        assert np.array_equal(from_dev_u8(x8b), orc.quantize(x, E5M2, sx).ravel()), t
        assert np.array_equal(from_dev_u8(w8b), orc.quantize(w, E5M2, sw).ravel()), t
        for gr, orr in ((rx, ox), (rw, ow)):
            assert ring_state_equal(gr, orr) and gr.idx == orr.idx, t
        s = _samples(M, N, 2000, 70 + t)
        ref, ad = orc.gemm_sampled(x8, w8, E4M3, False, True, M, N, K, sx, sw, bias, s)
        check_gemm(from_dev_bf16(f.out).reshape(M, N)[s[1], s[2]], ref, ad, f"large fwd {t}")


@pytest.mark.parametrize("M,N,K", [(512, 640, 384), (96, 1024, 256), (33, 17, 19)])
def test_dynamic_forward_launch_paths(lib, orc, M, N, K):
    """Dynamic forward with x and w both above the one-launch size (measure
    and cast passes), one above and one below it, and both small with
    ragged sizes (the one-launch kernel's scalar tail): same codes, steps
    and outputs as the oracle."""
    x = wl.normal_bf16((M, K), 1.0, M + K)
    w = wl.normal_bf16((N, K), 0.02, N + K)
    bias = wl.normal_bf16((N,), 0.1, N)
    f = Fwd(lib, M, N, K)
    lib.fp8_linear_fwd(to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(bias), M, N, K, E4M3, True, 0,
                       None, None, f.ws, f.scales, f.out)
    torch.cuda.synchronize()
    ref = orc.linear_fwd(x, w, bias, M, N, K, E4M3, True)
    sc = f.scales.cpu().numpy()
    assert sc[0] == ref.sx and sc[1] == ref.sw
    assert np.array_equal(f.x8(), ref.x8.ravel())
    assert np.array_equal(f.w8(), ref.w8.ravel())
    bound = orc.gemm_bound(ref.x8, ref.w8, E4M3, False, True, M, N, K, ref.sx, ref.sw)
    check_gemm(from_dev_bf16(f.out).reshape(M, N), ref.out, bound, f"dyn fwd {M}x{N}x{K}")


def test_backward_codes_from_the_forward(lib, orc):
    """Delayed HYBRID over three steps, twice: with bf16 x and w passed to
    the backward, and with the forward writing x's and w's E5M2 codes
    (x8_bwd, w8_bwd) that the backward takes instead (x and w NULL there).
    Outputs, gradients, steps and rings are bit-identical; the codes equal
    the oracle's quantize of x and w with the forward's steps."""
    d = wl.train(M=512, N=768, K=384, steps=3)
    M, N, K = d["M"], d["N"], d["K"]
    wd, bd = to_dev_bf16(d["w"]), to_dev_bf16(d["bias"])
    runs = []
    for use_codes in (False, True):
        f = Fwd(lib, M, N, K)
        bws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8,
                          device="cuda")
        rx, rw, rg = lib.Ring(16), lib.Ring(16), lib.Ring(16)
        x8b = torch.empty(M * K, dtype=torch.uint8, device="cuda")
        w8b = torch.empty(N * K, dtype=torch.uint8, device="cuda")
        rec = []
        for t in range(3):
            xd, gd = to_dev_bf16(d["x"][t]), to_dev_bf16(d["g"][t])
            dx = torch.empty(M * K, dtype=torch.int16, device="cuda")
            dw = torch.empty(N * K, dtype=torch.int16, device="cuda")
            db = torch.empty(N, dtype=torch.int16, device="cuda")
            if use_codes:
                lib.fp8_linear_fwd(xd, wd, bd, M, N, K, E4M3, False, 0, rx, rw, f.ws, f.scales,
                                   f.out, fmt_bwd=E5M2, x8_bwd=x8b, w8_bwd=w8b)
                lib.fp8_linear_bwd(gd, None, None, M, N, K, E5M2, False, 0, f.scales, rg, bws,
                                   None, dx, dw, db, x8_bwd=x8b, w8_bwd=w8b)
                torch.cuda.synchronize()
                sx, sw = (np.float32(v) for v in f.scales.cpu().numpy())
                assert np.array_equal(from_dev_u8(x8b), orc.quantize(d["x"][t], E5M2, sx).ravel())
                assert np.array_equal(from_dev_u8(w8b), orc.quantize(d["w"], E5M2, sw).ravel())
            else:
                lib.fp8_linear_fwd(xd, wd, bd, M, N, K, E4M3, False, 0, rx, rw, f.ws, f.scales,
                                   f.out)
                lib.fp8_linear_bwd(gd, xd, wd, M, N, K, E5M2, False, 0, f.scales, rg, bws, None,
                                   dx, dw, db)
                torch.cuda.synchronize()
            rec.append([t.clone() for t in (f.out, dx, dw, db, f.scales, rx.state, rw.state,
                                             rg.state)])
        runs.append(rec)
    for t in range(3):
        for a, b in zip(runs[0][t], runs[1][t]):
            assert torch.equal(a, b), t


@pytest.mark.gpu
def test_bias_gradient_in_the_pair_launch_ragged(lib, orc):
    """The backward's dX + dW at 4096 x 4112 x 4096 run as one paired launch
    (both products have at least 256 tiles), which also runs db's last pass
    in extra workgroups of 128 columns: 33 of them, the last with 16
    columns.  db equals the oracle's column sums within their fp32 summation
    bound, is bit-identical to fp8_colsum's (its own final launch, 64 columns
    per workgroup), and every column is written (db starts as NaN bits).  dX
    (NN, reduction over N = 4112: a k tail of 16 in every output) and dW
    (TN, a last tile row of 16 rows) match the oracle on the E5M2 codes of
    the dynamic steps: dW on every output of its last tile row plus samples,
    dX on samples."""
    M, N, K = 4096, 4112, 4096
    g = wl.normal_bf16((M, N), 1e-3, 1301)
    x = wl.normal_bf16((M, K), 1.0, 1302)
    w = wl.normal_bf16((N, K), 0.02, 1303)
    gd, xd, wd = to_dev_bf16(g), to_dev_bf16(x), to_dev_bf16(w)
    bws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    dx = torch.empty(M * K, dtype=torch.int16, device="cuda")
    dw = torch.empty(N * K, dtype=torch.int16, device="cuda")
    db = torch.full((N,), 0x7FC1, dtype=torch.int16, device="cuda")
    sb = torch.zeros(3, dtype=torch.float32, device="cuda")
    lib.fp8_linear_bwd(gd, xd, wd, M, N, K, E5M2, True, 0, None, None, bws, sb, dx, dw, db)
    ref = torch.empty(N, dtype=torch.int16, device="cuda")
    cws = torch.empty(lib.fp8_colsum_workspace(M, N), dtype=torch.uint8, device="cuda")
    lib.fp8_colsum(gd, M, N, ref, cws)
    torch.cuda.synchronize()
    assert torch.equal(db, ref)
    absg = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64)).sum(0)
    check_gemm(from_dev_bf16(db), orc.colsum(g, M, N), sum_bound(absg, M), "pair db")
    sg, sx, sw = (orc.scale_from_peak(orc.amax(v), E5M2) for v in (g, x, w))
    assert tuple(sb.cpu().numpy()) == (sg, sx, sw)
    g8, x8, w8 = orc.quantize(g, E5M2, sg), orc.quantize(x, E5M2, sx), orc.quantize(w, E5M2, sw)
    s = _samples(M, K, 2000, 1304)
    r, bnd = orc.gemm_sampled(g8, w8, E5M2, False, False, M, K, N, sg, sw, None, s)
    check_gemm(from_dev_bf16(dx).reshape(M, K)[s[1], s[2]], r, bnd, "pair dX")
    rows, cols = np.meshgrid(np.arange(4096, N), np.arange(K), indexing="ij")
    rs = _samples(N, K, 2000, 1305)
    s = (np.concatenate([np.zeros(rows.size, np.int64), rs[0]]),
         np.concatenate([rows.ravel(), rs[1]]), np.concatenate([cols.ravel(), rs[2]]))
    r, bnd = orc.gemm_sampled(g8, x8, E5M2, True, False, N, K, M, sg, sx, None, s)
    check_gemm(from_dev_bf16(dw).reshape(N, K)[s[1], s[2]], r, bnd, "pair dW")
