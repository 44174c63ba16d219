"""Graph capture of the library's launches.  The entry points only enqueue
kernels on the caller's stream (no allocation, no memset, no host
synchronization), so a captured call replays the same kernels; every
replay must give the bits of the same call made eagerly.  The
dynamic-scaling linear forward + backward (its per-call state lives in the
workspace's scratch rings, which each call re-arms) is captured once and
replayed on new inputs copied into the captured buffers, with eager work
and synchronizations between the replays.  (Delayed scaling keeps the
ring's window index on the host, advanced by each call, as the pages'
`_ScaleRing` does; a captured delayed call would replay one window slot,
so it is not captured here.)"""

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


class Step:
    """Buffers of one dynamic-scaling linear step (M x N x K, bias)."""

    def __init__(self, lib, M, N, K):
        dev = "cuda"
        self.lib, self.M, self.N, self.K = lib, M, N, K
        self.x = torch.zeros(M * K, dtype=torch.int16, device=dev)
        self.w = torch.zeros(N * K, dtype=torch.int16, device=dev)
        self.b = torch.zeros(N, dtype=torch.int16, device=dev)
        self.g = torch.zeros(M * N, dtype=torch.int16, device=dev)
        self.fws = torch.zeros(lib.fp8_linear_fwd_workspace(M, N, K), dtype=torch.uint8,
                               device=dev)
        self.bws = torch.zeros(lib.fp8_linear_bwd_workspace(M, N, K), dtype=torch.uint8,
                               device=dev)
        self.sc = torch.zeros(2, dtype=torch.float32, device=dev)
        self.so = torch.zeros(3, dtype=torch.float32, device=dev)
        self.out = torch.empty(M * N, dtype=torch.int16, device=dev)
        self.dx = torch.empty(M * K, dtype=torch.int16, device=dev)
        self.dw = torch.empty(N * K, dtype=torch.int16, device=dev)
        self.db = torch.empty(N, dtype=torch.int16, device=dev)

    def load(self, x, w, b, g):
        for dst, src in ((self.x, x), (self.w, w), (self.b, b), (self.g, g)):
            dst.copy_(to_dev_bf16(src.ravel()))

    def run(self):
        M, N, K, f = self.M, self.N, self.K, self.lib
        f.fp8_linear_fwd(self.x, self.w, self.b, M, N, K, E4M3, True, 0, None, None, self.fws,
                         self.sc, self.out)
        f.fp8_linear_bwd(self.g, self.x, self.w, M, N, K, E5M2, True, 0, self.sc, None, self.bws,
                         self.so, self.dx, self.dw, self.db)

    def results(self):
        return [t.clone() for t in (self.out, self.dx, self.dw, self.db, self.sc, self.so)]


def test_dynamic_linear_step_graph_replays(lib):
    M, N, K = 256, 384, 512
    captured, eager = Step(lib, M, N, K), Step(lib, M, N, K)
    inputs = [(wl.normal_bf16((M, K), s, 40 + r), wl.normal_bf16((N, K), 0.02 * s, 50 + r),
               wl.normal_bf16((N,), 0.1, 60 + r), wl.normal_bf16((M, N), 1e-3 / s, 70 + r))
              for r, s in enumerate((1.0, 8.0, 0.125, 2.0))]
    captured.load(*inputs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, as torch asks
        captured.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured.run()
    torch.cuda.synchronize()
    for rep, inp in enumerate(inputs):
        captured.load(*inp)
        graph.replay()
        torch.cuda.synchronize()
        got = captured.results()
        # eager work between replays: the same step on its own buffers
        eager.load(*inp)
        eager.run()
        torch.cuda.synchronize()
        want = eager.results()
        for name, a, b in zip(("out", "dx", "dw", "db", "scales_fwd", "scales_bwd"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        assert np.isfinite(got[4].cpu().numpy()).all() and (got[4].cpu().numpy() > 0).all()
