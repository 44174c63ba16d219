// fp8 GEMM for short A (m <= 64), NT layout (declarations).
#pragma once

#include "internal.hpp"

namespace fp8lin {

// True when the skinny kernel takes this problem: NT layout, 1 <= m <= 64,
// 16-byte aligned operand bases, leading dimensions, batch strides and k,
// and 32-bit offsets within each operand slice.
bool gemm_skinny_supported(const GemmLaunch& g);
hipError_t launch_gemm_skinny(const GemmLaunch& g, hipStream_t stream);

}  // namespace fp8lin
