"""The allocation-free entry point fp8_quantize_colsum_noalloc (its column-sum
partials in the library's static scratch) against fp8_quantize_colsum with a
caller workspace: codes, bias gradient, ring state and the step used are the
same bits, on two calls in a row (the second smaller, so stale partials of
the first would show), with and without a ring; shapes above the scratch
are refused before anything is enqueued."""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def lib():
    import fp8_tensor_scaled_amd as f
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return f


def _run(lib, g, M, N, fmt, scale, ring, noalloc):
    out = torch.full((M * N,), 0xAA, dtype=torch.uint8, device="cuda")
    db = torch.full((N,), 0x7FC1, dtype=torch.int16, device="cuda")
    used = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    if noalloc:
        lib.fp8_quantize_colsum_noalloc(g, M, N, fmt, scale, out, db, ring=ring,
                                        scale_used=used)
    else:
        ws = torch.empty(lib.fp8_colsum_workspace(M, N), dtype=torch.uint8, device="cuda")
        lib.fp8_quantize_colsum(g, M, N, fmt, scale, out, db, ws, ring=ring, scale_used=used)
    return out, db, used


@pytest.mark.parametrize("with_ring", [True, False])
def test_noalloc_matches_workspace_entry_point(lib, with_ring):
    assert lib.fp8_quantize_colsum_noalloc_max_bytes() == 1 << 20
    rings = {k: lib.Ring(16) for k in ("ws", "na")} if with_ring else {"ws": None, "na": None}
    for step, (M, N, std) in enumerate(((2048, 4096, 1e-3), (512, 1032, 2e-3))):
        g = to_dev_bf16(wl.normal_bf16((M, N), std, 1500 + step))
        scale = torch.tensor([std * 4 / 57344.0], dtype=torch.float32, device="cuda")
        s_ws = rings["ws"].scale if with_ring else scale
        s_na = rings["na"].scale if with_ring else scale
        if with_ring and step == 0:
            for r in rings.values():  # seed both rings the same way
                lib.fp8_quantize(g, E5M2, ring=r)
        a = _run(lib, g, M, N, E5M2, s_ws, rings["ws"], False)
        b = _run(lib, g, M, N, E5M2, s_na, rings["na"], True)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), (step, M, N)
        assert not torch.equal(b[1], torch.full_like(b[1], 0x7FC1))
        if with_ring:
            assert torch.equal(rings["ws"].state, rings["na"].state)
            for r in rings.values():
                r.idx = (r.idx + 1) % 16


def test_noalloc_refuses_shapes_above_the_scratch(lib):
    M, N = 1, 300_000  # 1.2 MB of partials
    assert lib.fp8_colsum_workspace(M, N) > lib.fp8_quantize_colsum_noalloc_max_bytes()
    g = torch.zeros(M * N, dtype=torch.int16, device="cuda")
    out = torch.empty(M * N, dtype=torch.uint8, device="cuda")
    db = torch.empty(N, dtype=torch.int16, device="cuda")
    scale = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="static scratch"):
        lib.fp8_quantize_colsum_noalloc(g, M, N, E4M3, scale, out, db)
