"""Seeded synthetic inputs for the FP8 linear layer, shared by the tests,
the smoke check and the benchmark.

This module draws random numbers and rounds them to bf16 with torch's CPU
conversion; it holds none of the quantize / scale / GEMM arithmetic, so both
the HIP path and the CPU oracle can take their inputs from it.

The shapes and distributions follow the workloads the AstrAI pages measure
(author commit search page: the fp8 GEMM micro-benchmark shapes; compare
view: the fp8 linear layer), in five benchmark configurations:

  linear256   x [256,256] N(0,1), w [256,256] N(0,0.02), bias [256] N(0,0.1);
              dynamic scaling, E4M3 (seeds 101, 102, 103)
  smallm      x [64,2048] N(0,1), w [8192,2048] N(0,0.02), no bias;
              pre-quantized E4M3 (seeds 201, 202)
  square4096  A, B [4096,4096] N(0,1), bias [4096] N(0,0.1) (301, 302, 303)
  square8192  A, B [8192,8192] N(0,1), bias [8192] N(0,0.1) (311, 312, 313)
  bmm8        8 x [1024,2048] x [2048,2048] N(0,1) (401, 402)
  bmm64       64 x [512,512] x [512,512] N(0,1) (411, 412)
  bcast8      8 x [1024,2048], one shared [2048,2048] (421, 422)
  train       x_t = s_t * z, z [2048,1024] N(0,1), s_t = 1, 4, 0.25, 2;
              w [4096,1024] N(0,0.02); bias [4096] N(0,0.1);
              g_t [2048,4096] N(0,1e-3) (z 501, w 502, bias 503, g_t 510+t)

Every draw is numpy PCG64 ``default_rng(seed).standard_normal(shape,
float32) * std`` rounded to bf16 (nearest-even).  Arrays are returned as
numpy ``uint16`` bf16 bit patterns.
"""

from __future__ import annotations

import numpy as np
import torch

TRAIN_STEP_STD = (1.0, 4.0, 0.25, 2.0)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws, PCG64 seeded."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v = v * np.float32(std)
    return f32_to_bf16_bits(v)


def scaled_bf16(h: np.ndarray, factor: float) -> np.ndarray:
    """Multiply bf16 values by a power of two (exact, so the bf16 bits of
    the product are exact)."""
    m, e = np.frexp(factor)
    assert m == 0.5, "factor must be a power of two"
    return f32_to_bf16_bits(bf16_bits_to_f32(h) * np.float32(factor))


def random_codes(shape, fmt: int, seed: int, allow_special: bool = False) -> np.ndarray:
    """Uniform random fp8 codes; NaN (and E5M2 inf) codes are redrawn unless
    ``allow_special``."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if not allow_special:
        if fmt == 0:
            bad = (c & 0x7F) == 0x7F
            c[bad] = c[bad] & 0xF0
        else:
            bad = (c & 0x7C) == 0x7C
            c[bad] = c[bad] & 0xF3
    return c


def linear256():
    return dict(M=256, N=256, K=256,
                x=normal_bf16((256, 256), 1.0, 101),
                w=normal_bf16((256, 256), 0.02, 102),
                bias=normal_bf16((256,), 0.1, 103))


def smallm():
    return dict(M=64, N=8192, K=2048,
                x=normal_bf16((64, 2048), 1.0, 201),
                w=normal_bf16((8192, 2048), 0.02, 202))


def square(n: int):
    base = {4096: 301, 8192: 311}.get(n, 300 + n % 97)
    return dict(M=n, N=n, K=n,
                a=normal_bf16((n, n), 1.0, base),
                b=normal_bf16((n, n), 1.0, base + 1),
                bias=normal_bf16((n,), 0.1, base + 2))


def bmm8():
    return dict(batch=8, M=1024, N=2048, K=2048,
                a=normal_bf16((8, 1024, 2048), 1.0, 401),
                b=normal_bf16((8, 2048, 2048), 1.0, 402))


def bmm64():
    return dict(batch=64, M=512, N=512, K=512,
                a=normal_bf16((64, 512, 512), 1.0, 411),
                b=normal_bf16((64, 512, 512), 1.0, 412))


def bcast8():
    return dict(batch=8, M=1024, N=2048, K=2048,
                a=normal_bf16((8, 1024, 2048), 1.0, 421),
                b=normal_bf16((2048, 2048), 1.0, 422))


def train(M=2048, N=4096, K=1024, steps=4):
    z = normal_bf16((M, K), 1.0, 501)
    return dict(M=M, N=N, K=K, z=z,
                x=[scaled_bf16(z, TRAIN_STEP_STD[t % 4]) for t in range(steps)],
                w=normal_bf16((N, K), 0.02, 502),
                bias=normal_bf16((N,), 0.1, 503),
                g=[normal_bf16((M, N), 1e-3, 510 + t) for t in range(steps)])
