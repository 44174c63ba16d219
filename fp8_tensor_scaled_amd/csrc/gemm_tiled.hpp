// LDS-tiled fp8 MFMA GEMM kernels (declarations).
#pragma once

#include "internal.hpp"

namespace fp8lin {

// True when the tiled kernels take this problem: 16-byte aligned operand
// bases, leading dimensions and batch strides; k a multiple of 16 for a
// k-contiguous operand; m (n) a multiple of 16 for an m- (n-) contiguous
// A (B).  Everything else runs on the general kernel.
bool gemm_tiled_supported(const GemmLaunch& g);
// A held-back ring fold (fold.n > 0) runs as one extra workgroup at the end
// of the grid; only plain NT problems take one (gemm_tiled_carries_fold).
bool gemm_tiled_carries_fold(const GemmLaunch& g);
hipError_t launch_gemm_tiled(const GemmLaunch& g, hipStream_t stream,
                             const FoldJob& fold = FoldJob{});

// Two independent problems in one launch: problem 0 NN and problem 1 TN,
// same format, together filling the CUs: 256 x 256 tiles when each has at
// least 256 of them; else 128 x 128 tiles, the problem with about half the
// other's k taking 256 x 128 or 128 x 256 ones, at least 256 between the
// two.
bool gemm_tiled_pair_supported(const GemmLaunch& g0, const GemmLaunch& g1);
// Whether the paired launch of a supported pair can also run `cf` (extra
// workgroups at the end of its grid).
bool gemm_tiled_pair_carries(const GemmLaunch& g0, const GemmLaunch& g1,
                             const ColsumFinalJob& cf);
hipError_t launch_gemm_tiled_pair(const GemmLaunch& g0, const GemmLaunch& g1, hipStream_t stream,
                                  const ColsumFinalJob* cf = nullptr,
                                  const FoldJob& fold = FoldJob{});

}  // namespace fp8lin
