// Scaled fp8 GEMM: out = bf16(acc * fp32(sa*sb) + bias), fp32 accumulation.
//
// Method (AstrAI compare view 3e57cc8...main: astrai/extension/ops/fp8.py
// mm_fp8; csrc/kernels/fp8/common.h operand layout tags and batch strides;
// csrc/kernels/fp8/gemm/epilogue.cuh bias + single bf16 rounding).  The
// extended epilogue (the removed fp8_gemm op's fp8 output with its step;
// the commit log's bias_scale for an fp8 bias) takes the bias as fp8 codes
// times their step and/or writes fp8 codes of the value times the fp32
// reciprocal of the output step, saturating.
//
// This file holds the dispatcher and the general kernel, which accepts any
// layout, size, stride and alignment: every lane gathers its MFMA operand
// bytes one by one (zero outside the matrix) and each wave owns a 16x16
// output tile.  It is the correctness fallback for shapes the fast kernels
// do not take: gemm_skinny.hip (NT with m <= 64, bandwidth-shaped) and
// gemm_tiled.hip (LDS-tiled MFMA, every layout).

#include "common.hpp"
#include "gemm_skinny.hpp"
#include "gemm_tiled.hpp"
#include "internal.hpp"

namespace fp8lin {

struct GenericParams {
    const uint8_t* a;
    const uint8_t* b;
    const float* sa;
    const float* sb;
    const void* bias;
    const float* bias_scale;  // non-null: bias holds fp8 codes of the operands' format
    void* out;
    int out_q;                // -1 bf16 output, else the fp8 output format
    const float* out_scale;
    int64_t m, n, k, lda, ldb;
    int64_t stride_a, stride_b;
    int trans_a, trans_b;
};

constexpr int kGenThreads = 256;  // 4 waves, 2x2 grid of 16x16 tiles

template <int FMT>
__global__ __launch_bounds__(kGenThreads) void gemm_generic_kernel(GenericParams p) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int64_t bz = blockIdx.z;
    const int64_t col0 = (int64_t)blockIdx.x * 32 + (wave % 2) * 16;
    const uint8_t* A = p.a + bz * p.stride_a;
    const uint8_t* B = p.b + bz * p.stride_b;
    const float s = (*p.sa) * (*p.sb);
    const int64_t bc = col0 + lane % 16;  // this lane's column of B
    const int kq = 32 * (lane / 16);
    for (int64_t by = blockIdx.y; by * 32 < p.m; by += gridDim.y) {
    const int64_t row0 = by * 32 + (wave / 2) * 16;
    const int64_t ar = row0 + lane % 16;  // this lane's row of A
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t k0 = 0; k0 < p.k; k0 += 128) {
        union {
            v8i v;
            uint8_t b[32];
        } xa, xb;
#pragma unroll 4
        for (int j = 0; j < 32; ++j) {
            const int64_t kk = k0 + kq + j;
            uint8_t va = 0, vb = 0;
            if (kk < p.k) {
                if (ar < p.m) va = p.trans_a ? A[kk * p.lda + ar] : A[ar * p.lda + kk];
                if (bc < p.n) vb = p.trans_b ? B[bc * p.ldb + kk] : B[kk * p.ldb + bc];
            }
            xa.b[j] = va;
            xb.b[j] = vb;
        }
        acc = mfma16x16x128<FMT>(xa.v, xb.v, acc);
    }
    const int64_t oc = col0 + lane % 16;
    if (oc < p.n) {
        float bias = 0.0f;
        if (p.bias) {
            bias = p.bias_scale
                       ? dec8<FMT, 0>(static_cast<const uint8_t*>(p.bias)[oc]) * (*p.bias_scale)
                       : bf16_to_f32(static_cast<const uint16_t*>(p.bias)[oc]);
        }
        const float rq = p.out_q >= 0 ? __fdiv_rn(1.0f, *p.out_scale) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t orow = row0 + 4 * (lane / 16) + i;
            if (orow >= p.m) continue;
            const int64_t o = (bz * p.m + orow) * p.n + oc;
            const float v = fmaf(acc[i], s, bias);
            if (p.out_q < 0)
                static_cast<uint16_t*>(p.out)[o] = f32_to_bf16(v);
            else
                static_cast<uint8_t*>(p.out)[o] = cvt1_rt(p.out_q, v * rq);
        }
    }
    }
}

static hipError_t launch_generic(const GemmLaunch& g, hipStream_t stream) {
    GenericParams p{};
    p.a = g.a;
    p.b = g.b;
    p.sa = g.scale_a;
    p.sb = g.scale_b;
    p.bias = g.bias;
    p.bias_scale = g.bias_scale;
    p.out = g.out;
    p.out_q = g.out_q;
    p.out_scale = g.out_scale;
    p.m = g.m;
    p.n = g.n;
    p.k = g.k;
    p.lda = g.lda;
    p.ldb = g.ldb;
    p.stride_a = g.batch > 1 ? g.stride_a : 0;
    p.stride_b = g.batch > 1 ? g.stride_b : 0;
    p.trans_a = g.trans_a;
    p.trans_b = g.trans_b;
    const int64_t gy = (g.m + 31) / 32;
    const dim3 grid((unsigned)((g.n + 31) / 32), (unsigned)(gy < 65535 ? gy : 65535),
                    (unsigned)g.batch);
    if (g.fmt == 0)
        hipLaunchKernelGGL(gemm_generic_kernel<0>, grid, dim3(kGenThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_generic_kernel<1>, grid, dim3(kGenThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t stream, FoldJob* fold) {
    const FoldJob none;
    const FoldJob& fj = fold ? *fold : none;
    hipError_t e;
    if (gemm_skinny_supported(g)) {
        e = launch_gemm_skinny(g, stream);
    } else if (fj.n > 0 && gemm_tiled_carries_fold(g)) {
        e = launch_gemm_tiled(g, stream, fj);  // the fold rides along
        if (e == hipSuccess) fold->n = 0;
        return e;
    } else if (gemm_tiled_supported(g)) {
        e = launch_gemm_tiled(g, stream);
    } else {
        e = launch_generic(g, stream);
    }
    if (e != hipSuccess || fj.n <= 0) return e;
    e = launch_fold_job(fj, stream);
    if (e == hipSuccess) fold->n = 0;
    return e;
}

hipError_t launch_gemm_pair(const GemmLaunch& g0, const GemmLaunch& g1, hipStream_t stream,
                            const ColsumFinalJob* cf, FoldJob* fold) {
    const bool job = cf && cf->db;
    if (!gemm_skinny_supported(g0) && !gemm_skinny_supported(g1) &&
        gemm_tiled_pair_supported(g0, g1) && (!job || gemm_tiled_pair_carries(g0, g1, *cf))) {
        const FoldJob none;
        hipError_t e = launch_gemm_tiled_pair(g0, g1, stream, job ? cf : nullptr,
                                              fold ? *fold : none);
        if (e == hipSuccess && fold) fold->n = 0;
        return e;
    }
    hipError_t e = launch_gemm(g0, stream, fold);
    if (e != hipSuccess) return e;
    e = launch_gemm(g1, stream);
    if (e != hipSuccess || !job) return e;
    return launch_colsum_final_job(*cf, stream);
}

}  // namespace fp8lin
