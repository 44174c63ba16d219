"""The Python binding checks every buffer against the sizes and element
types the C entry point will assume, before calling it (no GPU needed: the
checks run before any device access, and a well-sized CPU tensor is refused
for not being on a GPU)."""

import pytest
import torch

import fp8_tensor_scaled_amd as f

u8 = lambda n: torch.empty(n, dtype=torch.uint8)      # noqa: E731
b16 = lambda n: torch.empty(n, dtype=torch.int16)     # noqa: E731
f32 = lambda n: torch.empty(n, dtype=torch.float32)   # noqa: E731


def raises(needle, fn, *a, **kw):
    with pytest.raises(ValueError, match=needle):
        fn(*a, **kw)


def test_quantize_buffers():
    raises("out: 9 elements, needs at least 10", f.fp8_quantize, b16(10), f.E4M3, f32(1), u8(9))
    raises("x: dtype torch.float32", f.fp8_quantize, f32(10), f.E4M3, f32(1), u8(10))
    raises("out: dtype torch.int16", f.fp8_quantize, b16(10), f.E4M3, f32(1), b16(10))
    raises("scale: dtype torch.float64", f.fp8_quantize, b16(10), f.E4M3,
           torch.empty(1, dtype=torch.float64), u8(10))
    raises("amax_out: 0 elements", f.fp8_quantize, b16(10), f.E4M3, amax_out=f32(0))
    raises("x: tensor must be contiguous", f.fp8_quantize, b16(20)[::2], f.E4M3, f32(1),
           u8(10))
    raises("is on cpu, not a GPU", f.fp8_quantize, b16(10), f.E4M3, f32(1), u8(10))


def test_quantize_variants_buffers():
    raises("x: dtype torch.int16", f.fp8_quantize_ex, b16(8), f.E4M3, f32(1), u8(8),
           in_type=f.IN_F32)
    raises("out: 7 elements", f.fp8_quantize_ex, f32(8), f.E4M3, f32(1), u8(7))
    raises("bad input type", f.fp8_quantize_ex, f32(8), f.E4M3, f32(1), u8(8), in_type=5)
    raises("out2: 3 elements", f.fp8_quantize2, b16(4), f.E4M3, f32(1), u8(4), f.E5M2, u8(3))
    raises("out_t: 11 elements", f.fp8_quantize_t, b16(12), 3, 4, f.E4M3, f32(1), u8(11))
    raises("x: 11 elements", f.fp8_quantize_t, b16(11), 3, 4, f.E4M3, f32(1), u8(12))
    raises("amax: 0 elements", f.fp8_scale_ring_finalize, None, f.E4M3, f32(0))


def mm(**over):
    """fp8_mm arguments of an NT 3 x 5 x 8 product, two batches, with
    overrides."""
    a = dict(a=u8(2 * 3 * 8), b=u8(2 * 5 * 8), fmt=f.E4M3, trans_a=0, trans_b=1, m=3, n=5, k=8,
             lda=8, ldb=8, batch=2, stride_a=24, stride_b=40, scale_a=f32(1), scale_b=f32(1),
             bias=None, out=b16(2 * 3 * 5))
    a.update(over)
    return a


def test_mm_buffers():
    raises("a: 47 elements, needs at least 48", lambda: f.fp8_mm(**mm(a=u8(47))))
    raises("b: 79 elements, needs at least 80", lambda: f.fp8_mm(**mm(b=u8(79))))
    # a padded leading dimension and a broadcast B change the extents
    raises("a: 55 elements, needs at least 56", lambda: f.fp8_mm(**mm(a=u8(55), lda=9,
                                                                    stride_a=30)))
    raises("is on cpu, not a GPU", lambda: f.fp8_mm(**mm(b=u8(40), stride_b=0)))
    # transposed storage: B stored [k][n] with ldb >= n
    raises("b: 69 elements, needs at least 77", lambda: f.fp8_mm(**mm(b=u8(69), trans_b=0,
                                                                    ldb=5, stride_b=37)))
    raises("out: 29 elements", lambda: f.fp8_mm(**mm(out=b16(29))))
    raises("out: dtype torch.uint8", lambda: f.fp8_mm(**mm(out=u8(30))))
    raises("bias: 4 elements", lambda: f.fp8_mm(**mm(bias=b16(4))))
    raises("scale_a: required", lambda: f.fp8_mm(**mm(scale_a=None)))
    raises("negative size", lambda: f.fp8_mm(**mm(m=-1)))


def test_mm_ex_and_pair_buffers():
    base = mm()
    ex = dict(base, bias_scale=None, out_type=f.OUT_E4M3, out_scale=f32(1))
    raises("out: dtype torch.int16", lambda: f.fp8_mm_ex(**ex))
    raises("out: 29 elements", lambda: f.fp8_mm_ex(**dict(ex, out=u8(29))))
    raises("bias: dtype torch.uint8", lambda: f.fp8_mm_ex(**dict(ex, out=u8(30), bias=u8(5))))
    raises("bias: dtype torch.int16", lambda: f.fp8_mm_ex(**dict(ex, out=u8(30), bias=b16(5),
                                                                   bias_scale=f32(1))))
    raises("bad output type", lambda: f.fp8_mm_ex(**dict(ex, out_type=7)))
    p = tuple(base.values())
    short = tuple(mm(out=b16(10)).values())
    raises("out: 10 elements", f.fp8_mm_pair, p, short)
    raises("17 arguments", f.fp8_mm_pair, p, p[:-1])


def test_colsum_buffers():
    raises("g: 11 elements", f.fp8_colsum, b16(11), 3, 4, b16(4), u8(1 << 20))
    raises("db: 3 elements", f.fp8_colsum, b16(12), 3, 4, b16(3), u8(1 << 20))
    raises("out: 11 elements", f.fp8_quantize_colsum, b16(12), 3, 4, f.E5M2, f32(1), u8(11),
           b16(4), u8(1 << 20))


def test_linear_buffers():
    M, N, K = 4, 6, 8
    fwd = dict(x=b16(M * K), w=b16(N * K), bias=b16(N), M=M, N=N, K=K, fmt=f.E4M3,
               dynamic=True, margin=0, ring_x=None, ring_w=None, workspace=u8(1 << 16),
               scales_out=f32(2), out=b16(M * N))
    raises("x: 31 elements", lambda: f.fp8_linear_fwd(**dict(fwd, x=b16(31))))
    raises("w: dtype torch.uint8", lambda: f.fp8_linear_fwd(**dict(fwd, w=u8(N * K))))
    raises("bias: 5 elements", lambda: f.fp8_linear_fwd(**dict(fwd, bias=b16(5))))
    raises("scales_out: 1 elements", lambda: f.fp8_linear_fwd(**dict(fwd, scales_out=f32(1))))
    raises("out: 23 elements", lambda: f.fp8_linear_fwd(**dict(fwd, out=b16(23))))
    raises("x8_bwd: 31 elements", lambda: f.fp8_linear_fwd(**dict(fwd, x8_bwd=u8(31))))
    raises("w8_bwd: dtype torch.int16", lambda: f.fp8_linear_fwd(**dict(fwd, w8_bwd=b16(48))))
    bwd = dict(g=b16(M * N), x=b16(M * K), w=b16(N * K), M=M, N=N, K=K, fmt=f.E5M2,
               dynamic=True, margin=0, scales_fwd=None, ring_g=None, workspace=u8(1 << 16),
               scales_out=f32(3), dx=b16(M * K), dw=b16(N * K), db=b16(N))
    raises("g: 23 elements", lambda: f.fp8_linear_bwd(**dict(bwd, g=b16(23))))
    raises("scales_out: 2 elements", lambda: f.fp8_linear_bwd(**dict(bwd, scales_out=f32(2))))
    raises("dx: 31 elements", lambda: f.fp8_linear_bwd(**dict(bwd, dx=b16(31))))
    raises("dw: 47 elements", lambda: f.fp8_linear_bwd(**dict(bwd, dw=b16(47))))
    raises("db: 5 elements", lambda: f.fp8_linear_bwd(**dict(bwd, db=b16(5))))
    raises("x8_bwd: 31 elements", lambda: f.fp8_linear_bwd(**dict(bwd, x8_bwd=u8(31))))
    raises("w8_bwd: 47 elements", lambda: f.fp8_linear_bwd(**dict(bwd, w8_bwd=u8(47))))
    raises("is on cpu, not a GPU", lambda: f.fp8_linear_bwd(**bwd))
