"""GPU parity of the fp8 policy / autograd layer: FP8Linear and fp8_linear
under fp8_autocast give the bits of the C-ABI linear entry points driven by
hand (delayed scaling in each format over four steps on [B, L, d] inputs,
rings included),
match the oracle (dynamic scaling; pre-quantized weights), and leave the
plain path alone outside a region."""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import check_gemm, from_dev_bf16, ring_state_equal, sum_bound, to_dev_bf16

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def lib():
    import fp8_tensor_scaled_amd as f
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return f


@pytest.fixture(scope="module")
def fa(lib):
    from fp8_tensor_scaled_amd import autocast
    autocast.fp8_state().reset()
    return autocast


def bf16(bits, shape):
    return to_dev_bf16(bits.ravel()).view(torch.bfloat16).reshape(shape)


@pytest.mark.parametrize("fmt_name,frozen", [("HYBRID", False), ("E4M3", False),
                                             ("E5M2", False), ("HYBRID", True)])
def test_fp8linear_delayed_matches_entry_points(lib, fa, fmt_name, frozen):
    """The delayed route (x and w read once per step, their backward codes
    kept from the forward) against fp8_linear_fwd / _bwd: same bits, same
    rings.  frozen: the weight takes no gradient (no x codes kept, no dW)."""
    d = wl.train()
    M, N, K = d["M"], d["N"], d["K"]
    B = 2
    fmt = fa.FP8Format[fmt_name]
    layer = fa.FP8Linear(K, N).cuda().to(torch.bfloat16)
    with torch.no_grad():
        layer.weight.copy_(bf16(d["w"], (N, K)))
        layer.bias.copy_(bf16(d["bias"], (N,)))
    layer.weight.requires_grad_(not frozen)
    fa.fp8_state().reset()
    # the same steps by hand through the C-ABI
    rx, rw, rg = lib.Ring(16), lib.Ring(16), lib.Ring(16)
    fws = torch.zeros(lib.fp8_linear_fwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    bws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(2, dtype=torch.float32, device="cuda")
    out = torch.empty(M * N, dtype=torch.int16, device="cuda")
    dx, dw = (torch.empty(n, dtype=torch.int16, device="cuda") for n in (M * K, N * K))
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    wd, bd = layer.weight.view(torch.int16), layer.bias.view(torch.int16)
    with fa.fp8_autocast(recipe=fa.FP8Recipe(history_len=16), fp8_format=fmt):
        for t in range(4):
            x = bf16(d["x"][t], (B, M // B, K)).requires_grad_(True)
            g = bf16(d["g"][t], (B, M // B, N))
            layer.zero_grad()
            y = layer(x)
            y.backward(g)
            xd, gd = x.detach().view(torch.int16), g.view(torch.int16)
            lib.fp8_linear_fwd(xd, wd, bd, M, N, K, fmt.fwd(), False, 0, rx, rw, fws, sc, out)
            lib.fp8_linear_bwd(gd, xd, wd, M, N, K, fmt.bwd(), False, 0, sc, rg, bws, None, dx,
                               None if frozen else dw, db)
            torch.cuda.synchronize()
            assert y.shape == (B, M // B, N)
            assert torch.equal(y.detach().reshape(-1).view(torch.int16), out), t
            assert torch.equal(x.grad.reshape(-1).view(torch.int16), dx), t
            if frozen:
                assert layer.weight.grad is None
            else:
                assert torch.equal(layer.weight.grad.reshape(-1).view(torch.int16), dw), t
            assert torch.equal(layer.bias.grad.view(torch.int16), db), t
            meta = fa.fp8_state().get_weight_meta(layer.weight, fa.FP8Recipe(history_len=16))
            for a, b in ((meta.x, rx), (meta.w, rw), (meta.g, rg)):
                assert torch.equal(a.state, b.state) and a.idx == b.idx, t


def test_fp8_linear_dynamic_vs_oracle(lib, fa, orc):
    M, N, K = 256, 384, 512
    xb = wl.normal_bf16((M, K), 1.0, 11)
    wb = wl.normal_bf16((N, K), 0.02, 12)
    gb = wl.normal_bf16((M, N), 1e-3, 13)
    x = bf16(xb, (M, K)).requires_grad_(True)
    w = bf16(wb, (N, K)).requires_grad_(True)
    with fa.fp8_autocast(recipe=fa.FP8Recipe(dynamic=True), fp8_format=fa.FP8Format.HYBRID):
        y = fa.fp8_linear(x, w)
        y.backward(bf16(gb, (M, N)))
    torch.cuda.synchronize()
    rf = orc.linear_fwd(xb, wb, None, M, N, K, E4M3, True)
    ad = orc.gemm_bound(rf.x8, rf.w8, E4M3, False, True, M, N, K, rf.sx, rf.sw)
    check_gemm(from_dev_bf16(y.detach().reshape(-1).view(torch.int16)).reshape(M, N), rf.out,
               ad, "dynamic fwd")
    rb = orc.linear_bwd(gb, xb, wb, M, N, K, E5M2, True)
    w8b, x8b = orc.quantize(wb, E5M2, rb.sw), orc.quantize(xb, E5M2, rb.sx)
    ad = orc.gemm_bound(rb.g8, w8b, E5M2, False, False, M, K, N, rb.sg, rb.sw)
    check_gemm(from_dev_bf16(x.grad.reshape(-1).view(torch.int16)).reshape(M, K), rb.dx, ad,
               "dynamic dX")
    ad = orc.gemm_bound(rb.g8, x8b, E5M2, True, False, N, K, M, rb.sg, rb.sx)
    check_gemm(from_dev_bf16(w.grad.reshape(-1).view(torch.int16)).reshape(N, K), rb.dw, ad,
               "dynamic dW")


def test_fp8_linear_prequantized_weight_vs_oracle(lib, fa, orc):
    """E4M3 weight codes with their step, under FP8Format.E4M3: the forward
    quantizes x only; dX uses the codes as they are."""
    M, N, K = 128, 256, 320
    xb = wl.normal_bf16((M, K), 1.0, 21)
    wb = wl.normal_bf16((N, K), 0.02, 22)
    gb = wl.normal_bf16((M, N), 1e-3, 23)
    sw = orc.scale_from_peak(orc.amax(wb), E4M3)
    w8 = orc.quantize(wb, E4M3, sw)
    w8d = torch.from_numpy(w8).cuda().view(torch.float8_e4m3fn)
    swd = torch.tensor([sw], dtype=torch.float32, device="cuda")
    bb = wl.normal_bf16((N,), 0.1, 24)
    x = bf16(xb, (M, K)).requires_grad_(True)
    b = bf16(bb, (N,)).requires_grad_(True)
    with fa.fp8_autocast(recipe=fa.FP8Recipe(dynamic=True), fp8_format=fa.FP8Format.E4M3):
        y = fa.fp8_linear(x, w8d, b, w_scale=swd)
        y.backward(bf16(gb, (M, N)))
    torch.cuda.synchronize()
    # bias gradient (fused with the g quantize here): the oracle's column sum
    absg = np.abs(wl.bf16_bits_to_f32(gb).astype(np.float64)).sum(0)
    check_gemm(from_dev_bf16(b.grad.view(torch.int16)), orc.colsum(gb, M, N), sum_bound(absg, M),
               "prequant db fused")
    sx = orc.scale_from_peak(orc.amax(xb), E4M3)
    x8 = orc.quantize(xb, E4M3, sx)
    ref = orc.gemm(x8, w8, E4M3, False, True, M, N, K, sx, sw, bb)
    ad = orc.gemm_bound(x8, w8, E4M3, False, True, M, N, K, sx, sw)
    check_gemm(from_dev_bf16(y.detach().reshape(-1).view(torch.int16)).reshape(M, N), ref, ad, "prequant fwd")
    sg = orc.scale_from_peak(orc.amax(gb), E4M3)
    g8 = orc.quantize(gb, E4M3, sg)
    ref = orc.gemm(g8, w8, E4M3, False, False, M, K, N, sg, sw)
    ad = orc.gemm_bound(g8, w8, E4M3, False, False, M, K, N, sg, sw)
    check_gemm(from_dev_bf16(x.grad.reshape(-1).view(torch.int16)).reshape(M, K), ref, ad,
               "prequant dX")
    # bias gradient alone (x without grad: no g quantize)
    b.grad = None
    with fa.fp8_autocast(recipe=fa.FP8Recipe(dynamic=True), fp8_format=fa.FP8Format.E4M3):
        fa.fp8_linear(x.detach(), w8d, b, w_scale=swd).backward(bf16(gb, (M, N)))
    torch.cuda.synchronize()
    check_gemm(from_dev_bf16(b.grad.view(torch.int16)), orc.colsum(gb, M, N), sum_bound(absg, M),
               "prequant db alone")
    with fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
        with pytest.raises(NotImplementedError):
            x2 = bf16(xb, (M, K)).requires_grad_(True)
            fa.fp8_linear(x2, w8d, w_scale=swd).backward(bf16(gb, (M, N)))


def test_masks_and_plain_path(lib, fa):
    M, N, K = 64, 96, 128
    x = torch.randn(M, K, device="cuda").bfloat16().requires_grad_(True)
    w = torch.randn(N, K, device="cuda").bfloat16() * 0.05
    with fa.fp8_autocast(recipe=fa.FP8Recipe(dynamic=True)):
        y = fa.fp8_linear(x, w)   # no bias, w without grad: only dX
        y.sum().backward()
    assert x.grad is not None and x.grad.shape == (M, K) and w.grad is None
    ref = torch.nn.functional.linear(x.detach(), w)
    assert torch.equal(fa.fp8_linear(x.detach(), w), ref)  # outside a region: plain linear


def test_binding_launches_on_torch_current_stream(lib):
    """The binding's default stream is torch's current one (also inside a
    torch.cuda.stream context), and work enqueued there is ordered with
    torch's own work on that stream."""
    side = torch.cuda.Stream()
    handle = (lambda: lib._stream().value or 0)  # c_void_p(0).value is None
    assert handle() == torch.cuda.current_stream().cuda_stream
    x = torch.randn(1 << 20, device="cuda").to(torch.bfloat16)
    q = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(side):
        assert handle() == side.cuda_stream
        side.wait_stream(torch.cuda.default_stream())
        lib.fp8_quantize(x.view(torch.int16), 0, scale=s, out=q)
        ref = x.float().clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        same = torch.equal(q, ref)  # torch's compare runs on the same side stream
    torch.cuda.synchronize()
    assert same


def test_prequantized_weight_and_fp8_bias_vs_oracle(lib, fa, orc):
    """E4M3 weight codes and E4M3 bias codes with their steps (w8 / b8):
    the forward against the oracle's GEMM with an fp8 bias; neither takes a
    gradient; an fp8 bias without fp8 weights is refused."""
    M, N, K = 192, 320, 256
    xb = wl.normal_bf16((M, K), 1.0, 31)
    w8, sw = orc.quantize(wl.normal_bf16((N, K), 0.02, 32), E4M3, np.float32(2e-4)), \
        np.float32(2e-4)
    b8, sbias = orc.quantize(wl.normal_bf16((N,), 0.5, 33), E4M3, np.float32(0.01)), \
        np.float32(0.01)
    w8d = torch.from_numpy(w8).cuda().view(torch.float8_e4m3fn)
    b8d = torch.from_numpy(b8).cuda().view(torch.float8_e4m3fn)
    swd = torch.tensor([sw], device="cuda")
    sbd = torch.tensor([sbias], device="cuda")
    x = bf16(xb, (M, K)).requires_grad_(True)
    with fa.fp8_autocast(recipe=fa.FP8Recipe(dynamic=True), fp8_format=fa.FP8Format.E4M3):
        y = fa.fp8_linear(x, w8d, b8d, w_scale=swd, b_scale=sbd)
        y.sum().backward()
    torch.cuda.synchronize()
    sx = orc.scale_from_peak(orc.amax(xb), E4M3)
    x8 = orc.quantize(xb, E4M3, sx)
    ref, _, ad = orc.gemm_ex(x8, w8, E4M3, False, True, M, N, K, sx, sw, b8, sbias)
    check_gemm(from_dev_bf16(y.detach().reshape(-1).view(torch.int16)).reshape(M, N),
               ref.reshape(M, N), ad.reshape(M, N), "w8/b8 fwd")
    assert x.grad is not None and x.grad.shape == (M, K)
    with fa.fp8_autocast():
        with pytest.raises(ValueError, match="fp8 bias"):
            fa.fp8_linear(x, bf16(wl.normal_bf16((N, K), 0.02, 34), (N, K)), b8d, b_scale=sbd)


def _cos_and_norm_ratio(got, ref):
    got, ref = got.double().ravel(), ref.double().ravel()
    cos = float((got @ ref) / (got.norm() * ref.norm()))
    return cos, float(got.norm() / ref.norm())


@pytest.mark.parametrize("dynamic", [True, False])
def test_backward_outside_region_and_vs_bf16(lib, fa, dynamic):
    """The fp8 backward runs wherever backward() is called: outside the
    fp8_autocast region of the forward it gives the bits it gives inside
    (dynamic scaling; under delayed scaling each run moves the rings, so only
    the comparison below applies), and the gradients follow the bf16
    reference (fp32 math) in direction and norm within E5M2 noise."""
    M, N, K = 512, 768, 1024
    gen = torch.Generator(device="cuda").manual_seed(7)
    x0 = torch.randn(M, K, device="cuda", generator=gen).bfloat16()
    w0 = (torch.randn(N, K, device="cuda", generator=gen) * 0.02).bfloat16()
    b0 = (torch.randn(N, device="cuda", generator=gen) * 0.1).bfloat16()
    g = (torch.randn(M, N, device="cuda", generator=gen) * 1e-3).bfloat16()
    recipe = fa.FP8Recipe(dynamic=dynamic)

    def run(backward_inside):
        fa.fp8_state().reset()
        x, w, b = (t.clone().requires_grad_(True) for t in (x0, w0, b0))
        with fa.fp8_autocast(recipe=recipe):
            y = fa.fp8_linear(x, w, b)
            if backward_inside:
                y.backward(g)
        if not backward_inside:
            y.backward(g)  # outside the region
        torch.cuda.synchronize()
        return x.grad, w.grad, b.grad

    outside = run(False)
    inside = run(True)
    if dynamic:
        for a, c in zip(outside, inside):
            assert torch.equal(a, c)
    ref = (g.float() @ w0.float(), g.float().t() @ x0.float(), g.float().sum(0))
    for name, got, r in zip(("dX", "dW", "db"), outside, ref):
        cos, ratio = _cos_and_norm_ratio(got, r)
        assert cos > 0.99 and abs(ratio - 1) < 0.03, (name, cos, ratio)


def test_no_grad_keeps_no_backward_codes(lib, fa, monkeypatch):
    """Under torch.no_grad() / inference_mode a delayed HYBRID FP8Linear
    with a trainable weight quantizes x and w in the forward format only (no
    backward codes written or kept); with grad mode on the forward also
    writes both tensors' E5M2 codes.  The outputs are the same bits."""
    seen = []
    real = fa._linear_fwd_call

    def recording(*a):
        seen.append(sum(t is not None for t in a[-2:]))  # x8_bwd, w8_bwd
        return real(*a)

    monkeypatch.setattr(fa, "_linear_fwd_call", recording)
    torch.manual_seed(3)
    x = torch.randn(64, 256, device="cuda").to(torch.bfloat16).requires_grad_()
    outs = []
    for mode in ("no_grad", "inference", "grad"):
        layer = fa.FP8Linear(256, 128).cuda().to(torch.bfloat16)
        with torch.no_grad():
            layer.weight.copy_(torch.linspace(-1, 1, 128 * 256, device="cuda").reshape(128, 256))
            layer.bias.zero_()
        fa.fp8_state().reset()
        seen.clear()
        with fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
            if mode == "no_grad":
                with torch.no_grad():
                    y = layer(x)
            elif mode == "inference":
                with torch.inference_mode():
                    y = layer(x)
            else:
                y = layer(x)
        torch.cuda.synchronize()
        assert seen == [2 if mode == "grad" else 0], (mode, seen)
        outs.append(y.detach().clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_workspace_cache_stays_bounded(lib, fa):
    """Linear calls of many token counts on one stream share one workspace
    that only grows to the largest call's size."""
    fa._WS.clear()
    layer = fa.FP8Linear(256, 384).cuda().to(torch.bfloat16)
    sizes = []
    with fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
        for M in (64, 512, 96, 1024, 32, 700):
            x = torch.randn(M, 256, device="cuda").to(torch.bfloat16).requires_grad_()
            layer(x).float().sum().backward()
            torch.cuda.synchronize()
            assert len(fa._WS) == 1, len(fa._WS)
            sizes.append(next(iter(fa._WS.values())).numel())
    need = max(max(lib.fp8_linear_fwd_workspace(M, 384, 256),
                   lib.fp8_linear_bwd_workspace_codes(M, 384, 256))
               for M in (64, 512, 96, 1024, 32, 700))
    assert sizes[-1] == need and sizes == sorted(sizes)


def test_stock_linear_routed_under_autocast(lib, fa):
    """fp8_linear_enable(): a stock torch.nn.Linear inside fp8_autocast gives
    the bits of FP8Linear with the same weights (forward, input and weight
    gradients, bias gradient, over two delayed steps, then under no_grad and
    inference_mode), and outside the region the bits of torch's own linear;
    switched off, nothing is routed."""
    torch.manual_seed(7)
    K, N = 512, 384
    xs = [torch.randn(3, 64, K, device="cuda").to(torch.bfloat16) for _ in range(2)]
    gs = [torch.randn(3, 64, N, device="cuda").to(torch.bfloat16) * 1e-3 for _ in range(2)]

    def run(layer):
        fa.fp8_state().reset()
        res = []
        for x0, g in zip(xs, gs):
            x = x0.clone().requires_grad_()
            layer.zero_grad()
            with fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
                y = layer(x)
            y.backward(g)
            res += [y.detach(), x.grad, layer.weight.grad.clone(), layer.bias.grad.clone()]
        with torch.no_grad(), fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
            res.append(layer(xs[1]).clone())
        with torch.inference_mode(), fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
            res.append(layer(xs[0]).clone())
        return res

    ref_layer = fa.FP8Linear(K, N).cuda().to(torch.bfloat16)
    stock = torch.nn.Linear(K, N).cuda().to(torch.bfloat16)
    with torch.no_grad():
        stock.weight.copy_(ref_layer.weight)
        stock.bias.copy_(ref_layer.bias)
    want = run(ref_layer)
    plain = stock(xs[0]).detach()  # before routing: torch's own linear
    fa.fp8_linear_enable(True)
    try:
        assert fa.fp8_linear_enabled()
        got = run(stock)
        outside = stock(xs[0]).detach()
        f_out = torch.nn.functional.linear(xs[0], stock.weight, stock.bias).detach()
    finally:
        fa.fp8_linear_enable(False)
    assert not fa.fp8_linear_enabled()
    for a, b in zip(got, want):
        assert torch.equal(a, b)
    assert torch.equal(outside, plain) and torch.equal(f_out, plain)
    # off again: inside a region a stock layer no longer takes the fp8 path
    with fa.fp8_autocast(fp8_format=fa.FP8Format.HYBRID):
        assert torch.equal(stock(xs[0]).detach(), plain)
