// Device helpers shared by the fp8 linear-layer kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace fp8lin {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Largest finite value of each OCP format.
template <int FMT>
__device__ __forceinline__ constexpr float fmt_max() {
    return FMT ? 57344.0f : 448.0f;
}

// bf16 bit pattern -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16 bit patterns, round to nearest even, by gfx950's
// v_cvt_pk_bf16_f32 (two values per instruction).  The GEMM parity tests
// check its results against the oracle's single rounding, among them
// outputs whose low 16 bits are an exact tie, a near tie either way, zero
// and the largest cut, at 18 exponents, on the short-A, 128 x 128 and
// 256 x 256 kernels.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Saturating clamp to +-max that keeps NaN, so the hardware conversion that
// follows rounds to nearest even within range and never overflows.
template <int FMT>
__device__ __forceinline__ float sat(float v) {
    const float c = __builtin_amdgcn_fmed3f(v, -fmt_max<FMT>(), fmt_max<FMT>());
    return v != v ? v : c;
}

// Four fp32 -> four fp8 codes packed little-endian in one dword.
// v_cvt_pk_{fp8,bf8}_f32 round to nearest even on gfx950 (OCP encodings).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    int w;
    if constexpr (FMT) {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(sat<FMT>(a), sat<FMT>(b), 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(sat<FMT>(c), sat<FMT>(d), w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(sat<FMT>(a), sat<FMT>(b), 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(sat<FMT>(c), sat<FMT>(d), w, true);
    }
    return (uint32_t)w;
}

template <int FMT>
__device__ __forceinline__ uint8_t cvt1(float a) {
    int w;
    if constexpr (FMT)
        w = __builtin_amdgcn_cvt_pk_bf8_f32(sat<FMT>(a), 0.0f, 0, false);
    else
        w = __builtin_amdgcn_cvt_pk_fp8_f32(sat<FMT>(a), 0.0f, 0, false);
    return (uint8_t)(w & 0xff);
}

// One fp8 code (byte SEL of w) -> fp32, exact: v_cvt_f32_{fp8,bf8}, which
// decode the OCP encodings on gfx950.
template <int FMT, int SEL>
__device__ __forceinline__ float dec8(uint32_t w) {
    if constexpr (FMT)
        return __builtin_amdgcn_cvt_f32_bf8((int)w, SEL);
    else
        return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// cvt4 / cvt1 with the format chosen at run time (0 E4M3, 1 E5M2).
__device__ __forceinline__ uint32_t cvt4_rt(int fmt, float a, float b, float c, float d) {
    return fmt ? cvt4<1>(a, b, c, d) : cvt4<0>(a, b, c, d);
}
__device__ __forceinline__ uint8_t cvt1_rt(int fmt, float a) {
    return fmt ? cvt1<1>(a) : cvt1<0>(a);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// A held-back ring fold (one wave; every lane calls it).  The new amax is
// the largest of the group lines' maxima, taken by atomics of an earlier
// launch (non-negative floats order as their bits); hist[idx] = amax; the
// step max(peak / fmax / 2^margin, 1e-12) from the window's peak, with the
// quantize's own fold's two IEEE divisions; the lines back to zero for the
// next launch.
__device__ __forceinline__ void fold_ring_lines(const RingFold& f) {
    // the lane from the hardware's lane count, not from threadIdx: a GEMM
    // kernel that carries the fold must not keep a value shared with its
    // tile code alive across the tile loop
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    float* hist = f.state;
    uint32_t* lines = reinterpret_cast<uint32_t*>(f.state + ring_groups_offset(f.len));
    uint32_t m = 0;
    if (lane < kRingGroups)
        m = __hip_atomic_load(lines + kRingGroupWords * lane, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    float w = 0.0f;
    for (int i = lane; i < f.len; i += kWave)
        if (i != f.idx) w = fmaxf(w, hist[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = __shfl_xor(m, off, kWave);
        m = o > m ? o : m;
    }
    const float amax = __uint_as_float(m);
    const float peak = fmaxf(wave_max(w), amax);
    if (lane < kRingGroups)
        __hip_atomic_store(lines + kRingGroupWords * lane, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) {
        hist[f.idx] = amax;
        const float t = __fdiv_rn(peak, f.fmax);
        const float s = __fdiv_rn(t, f.pow2_margin);
        hist[f.len] = fmaxf(s, 1e-12f);
    }
}

// Bias gradient, last pass: db[c] = bf16 of the sum over chunks k of the
// partial column sums part[k][c], for the T/4 columns c0 .. c0 + T/4 - 1 of
// one workgroup of T lanes.  Lane group q (T/4 lanes, one column each) adds
// the q-th quarter of the chunks in chunk order; the four quarter sums are
// then added as ((0 + 1) + 2) + 3 and rounded once (RNE).  The arithmetic
// depends on the chunk count and the data only, not on T.  `red` is T
// floats of LDS.  Every lane of the workgroup must call it.
template <int T>
__device__ __forceinline__ void colsum_final_cols(const float* part, int64_t chunks, int64_t n,
                                                  int64_t c0, uint16_t* db, float* red) {
    constexpr int kCols = T / 4;
    const int col = threadIdx.x % kCols;
    const int q = threadIdx.x / kCols;
    const int64_t c = c0 + col;
    float acc = 0.0f;
    if (c < n) {
        const int64_t per = (chunks + 3) / 4;
        const int64_t b = q * per;
        const int64_t e = b + per < chunks ? b + per : chunks;
        // 8 loads in flight, then their adds in chunk order
        for (int64_t k = b; k < e; k += 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = k + i < e ? part[(k + i) * n + c] : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (k + i < e) acc += v[i];
        }
    }
    red[q * kCols + col] = acc;
    __syncthreads();
    if (q == 0 && c < n)
        db[c] = f32_to_bf16(((red[col] + red[kCols + col]) + red[2 * kCols + col]) +
                            red[3 * kCols + col]);
}

// One fp8 MFMA: D(16x16, fp32) += X(16x128) . Y(16x128)^T.
// Lane l holds row l%16 of X and of Y, bytes k = 32*(l/16) .. +31; the
// result row 4*(l/16)+i, column l%16 sits in register i.
template <int FMT>
__device__ __forceinline__ v4f mfma16x16x128(const v8i& x, const v8i& y, v4f acc) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, FMT, FMT, 0, 0, 0, 0);
}

}  // namespace fp8lin
