// bf16 -> fp8 quantize with fused amax and the delayed-scaling ring fold,
// the standalone ring finalize, and the bias-gradient column sum.
//
// Method (AstrAI compare view 3e57cc8...main, csrc/kernels/fp8/quantize.cuh:
// fp8_quantize_kernel and publish_amax; astrai/extension/fp8.py:
// FP8Recipe.scale_from_history and _ScaleRing): each element is multiplied
// by the reciprocal of the step and converted with round-to-nearest-even and
// saturation; the running max of |x| is taken over the raw inputs; every
// workgroup contributes its max with one atomic, and the workgroup that
// finishes last records the amax in the history slot, publishes the next
// step from the window's max and re-arms its scratch slots, so the delayed
// update costs no extra launch.
//
// gfx950 design: one workgroup = 4 waves of 64; each lane streams 32 bytes
// of bf16 per iteration (two 16-byte loads) and stores the 16 fp8 codes with
// one 16-byte store; conversions use v_cvt_pk_{fp8,bf8}_f32 after a med3
// clamp (satfinite).  The grid is sized to keep every CU busy with several
// resident workgroups.  Cross-XCD correctness of the fold uses agent-scope
// atomics: the amax slot is an atomic max on fp32 bits (non-negative
// floats order like unsigned ints) and the done counter an acq_rel add.

#include "common.hpp"
#include "internal.hpp"

namespace fp8lin {

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;
constexpr int kElemsPerIter = 16;  // per lane

struct QuantParams {
    const uint16_t* x;
    int64_t numel;
    const float* scale;
    uint8_t* out;
    float* hist;          // ring window (null: no fold)
    float* scale_out;     // ring scale slot
    uint32_t* amax_slot;  // ring scratch: running amax bits
    uint32_t* done;       // ring scratch: finished-workgroup counter
    int32_t len;
    int32_t idx;
    float fmax;
    float pow2_margin;
    float* scale_used;
    int vec;  // 1: x and out are 16-byte aligned
};

// Last-workgroup fold: hist[idx] = amax; scale = max(peak/fmax/2^m, 1e-12).
__device__ __forceinline__ void fold_ring(const QuantParams& p, float s_read) {
    const int lane = threadIdx.x;  // wave 0 only
    float amax = 0.0f;
    if (lane == 0) {
        amax = __uint_as_float(
            __hip_atomic_load(p.amax_slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT));
        p.hist[p.idx] = amax;
    }
    amax = __shfl(amax, 0, kWave);
    float peak = 0.0f;
    for (int i = lane; i < p.len; i += kWave) peak = fmaxf(peak, i == p.idx ? amax : p.hist[i]);
    peak = wave_max(peak);
    if (lane == 0) {
        const float t = __fdiv_rn(peak, p.fmax);
        const float s = __fdiv_rn(t, p.pow2_margin);
        *p.scale_out = fmaxf(s, 1e-12f);
        if (p.scale_used) *p.scale_used = s_read;
        __hip_atomic_store(p.amax_slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.done, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Workgroup max -> one atomic; the last workgroup folds the ring.
__device__ __forceinline__ void publish_amax(const QuantParams& p, float v, float s_read) {
    __shared__ float slots[kQuantWaves];
    __shared__ int is_last;
    v = wave_max(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) slots[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kQuantWaves; ++w) v = fmaxf(v, slots[w]);
        __hip_atomic_fetch_max(p.amax_slot, __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t nblocks = gridDim.x;
        const uint32_t ticket =
            __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (ticket == nblocks - 1u);
    }
    __syncthreads();
    if (is_last && threadIdx.x < kWave) fold_ring(p, s_read);
}

template <int FMT, bool MEASURE_ONLY>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(QuantParams p) {
    float m = 0.0f, s_read = 0.0f;
    if constexpr (!MEASURE_ONLY) {
        s_read = *p.scale;
        m = __fdiv_rn(1.0f, s_read);
    }
    float amax = 0.0f;
    const int64_t tid = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    const int64_t nvec = p.vec ? p.numel / kElemsPerIter : 0;
    const uint4* xv = reinterpret_cast<const uint4*>(p.x);
    uint4* ov = reinterpret_cast<uint4*>(p.out);
    for (int64_t i = tid; i < nvec; i += stride) {
        const uint4 r0 = xv[2 * i];
        const uint4 r1 = xv[2 * i + 1];
        const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        float f[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f[2 * j] = bf16_lo(w[j]);
            f[2 * j + 1] = bf16_hi(w[j]);
        }
#pragma unroll
        for (int j = 0; j < 16; j += 2) amax = fmaxf(amax, fmaxf(fabsf(f[j]), fabsf(f[j + 1])));
        if constexpr (!MEASURE_ONLY) {
            uint4 o;
            o.x = cvt4<FMT>(f[0] * m, f[1] * m, f[2] * m, f[3] * m);
            o.y = cvt4<FMT>(f[4] * m, f[5] * m, f[6] * m, f[7] * m);
            o.z = cvt4<FMT>(f[8] * m, f[9] * m, f[10] * m, f[11] * m);
            o.w = cvt4<FMT>(f[12] * m, f[13] * m, f[14] * m, f[15] * m);
            ov[i] = o;
        }
    }
    // Scalar tail (everything when the bases are not 16-byte aligned).
    for (int64_t i = nvec * kElemsPerIter + tid; i < p.numel; i += stride) {
        const float f = bf16_to_f32(p.x[i]);
        amax = fmaxf(amax, fabsf(f));
        if constexpr (!MEASURE_ONLY) p.out[i] = cvt1<FMT>(f * m);
    }
    if (p.hist) {
        publish_amax(p, amax, s_read);
    } else if constexpr (!MEASURE_ONLY) {
        if (p.scale_used && blockIdx.x == 0 && threadIdx.x == 0) *p.scale_used = s_read;
    }
}

static int quant_grid(int64_t numel, int vec) {
    const int64_t per_block = (int64_t)kQuantThreads * (vec ? kElemsPerIter : 1);
    int64_t blocks = (numel + per_block - 1) / per_block;
    const int64_t cap = 256 * 8;  // 8 resident workgroups per CU on 256 CUs
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

hipError_t launch_quantize(const QuantLaunch& q, hipStream_t stream) {
    QuantParams p{};
    p.x = q.x;
    p.numel = q.numel;
    p.scale = q.scale;
    p.out = q.out;
    if (q.ring_state) {
        p.hist = q.ring_state;
        p.scale_out = q.ring_state + q.ring_len;
        p.amax_slot = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 2);
        p.done = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 3);
        p.len = q.ring_len;
        p.idx = q.ring_idx;
    }
    p.fmax = q.fmt ? 57344.0f : 448.0f;
    p.pow2_margin = q.pow2_margin;
    p.scale_used = q.scale_used;
    const uintptr_t al = reinterpret_cast<uintptr_t>(q.x) | reinterpret_cast<uintptr_t>(q.out);
    p.vec = (al & 15) == 0;
    const dim3 grid(quant_grid(q.numel, p.vec)), block(kQuantThreads);
    const bool measure = q.out == nullptr;
    if (q.fmt == 0) {
        if (measure)
            hipLaunchKernelGGL((quantize_kernel<0, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((quantize_kernel<0, false>), grid, block, 0, stream, p);
    } else {
        if (measure)
            hipLaunchKernelGGL((quantize_kernel<1, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((quantize_kernel<1, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Standalone fold of an externally measured amax (one wave).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void ring_finalize_kernel(float* state, int32_t len,
                                                               int32_t idx, float fmax,
                                                               float pow2_margin,
                                                               const float* amax_in) {
    const int lane = threadIdx.x;
    const float amax = *amax_in;
    float peak = 0.0f;
    for (int i = lane; i < len; i += kWave) peak = fmaxf(peak, i == idx ? amax : state[i]);
    peak = wave_max(peak);
    if (lane == 0) {
        state[idx] = amax;
        const float t = __fdiv_rn(peak, fmax);
        const float s = __fdiv_rn(t, pow2_margin);
        state[len] = fmaxf(s, 1e-12f);
    }
}

hipError_t launch_ring_finalize(float* state, int32_t len, int32_t idx, int fmt,
                                float pow2_margin, const float* amax, hipStream_t stream) {
    hipLaunchKernelGGL(ring_finalize_kernel, dim3(1), dim3(kWave), 0, stream, state, len, idx,
                       fmt ? 57344.0f : 448.0f, pow2_margin, amax);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bias gradient: db[j] = bf16(sum_i g[i][j]).  Pass 1: each lane sums 8
// adjacent columns over a chunk of rows into fp32 partials; pass 2 adds the
// partials of each column in chunk order (deterministic) and rounds once.
// ---------------------------------------------------------------------------
constexpr int kColThreads = 256;

// Rows per chunk: 32, grown so that the chunk count fits gridDim.y.
static int64_t colsum_rows(int64_t m) {
    int64_t r = 32;
    while ((m + r - 1) / r > 65535) r *= 2;
    return r;
}
static int64_t colsum_chunks(int64_t m) { return (m + colsum_rows(m) - 1) / colsum_rows(m); }

size_t colsum_workspace(int64_t m, int64_t n) {
    return (size_t)colsum_chunks(m) * (size_t)n * sizeof(float);
}

__global__ __launch_bounds__(kColThreads) void colsum_partial_kernel(const uint16_t* g,
                                                                     int64_t m, int64_t n,
                                                                     int64_t rows, int vec,
                                                                     float* part) {
    const int64_t chunk = blockIdx.y;
    const int64_t r0 = chunk * rows;
    const int64_t r1 = r0 + rows < m ? r0 + rows : m;
    if (vec) {
        const int64_t c0 = ((int64_t)blockIdx.x * kColThreads + threadIdx.x) * 8;
        if (c0 >= n) return;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int64_t r = r0; r < r1; ++r) {
            const uint4 v = *reinterpret_cast<const uint4*>(g + r * n + c0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] += bf16_lo(w[j]);
                acc[2 * j + 1] += bf16_hi(w[j]);
            }
        }
        float4* dst = reinterpret_cast<float4*>(part + chunk * n + c0);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        const int64_t c = (int64_t)blockIdx.x * kColThreads + threadIdx.x;
        if (c >= n) return;
        float acc = 0.0f;
        for (int64_t r = r0; r < r1; ++r) acc += bf16_to_f32(g[r * n + c]);
        part[chunk * n + c] = acc;
    }
}

__global__ __launch_bounds__(kColThreads) void colsum_final_kernel(const float* part,
                                                                   int64_t chunks, int64_t n,
                                                                   uint16_t* db) {
    const int64_t c = (int64_t)blockIdx.x * kColThreads + threadIdx.x;
    if (c >= n) return;
    float acc = 0.0f;
    for (int64_t q = 0; q < chunks; ++q) acc += part[q * n + c];
    db[c] = f32_to_bf16(acc);
}

hipError_t launch_colsum(const uint16_t* g, int64_t m, int64_t n, uint16_t* db, void* ws,
                         hipStream_t stream) {
    float* part = static_cast<float*>(ws);
    const int64_t chunks = colsum_chunks(m);
    const int vec = (n % 8 == 0) && ((reinterpret_cast<uintptr_t>(g) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(part) & 15) == 0);
    const int64_t cols_per_block = vec ? (int64_t)kColThreads * 8 : kColThreads;
    const dim3 grid1((unsigned)((n + cols_per_block - 1) / cols_per_block), (unsigned)chunks);
    hipLaunchKernelGGL(colsum_partial_kernel, grid1, dim3(kColThreads), 0, stream, g, m, n,
                       colsum_rows(m), vec, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid2((unsigned)((n + kColThreads - 1) / kColThreads));
    hipLaunchKernelGGL(colsum_final_kernel, grid2, dim3(kColThreads), 0, stream, part, chunks, n,
                       db);
    return hipGetLastError();
}

}  // namespace fp8lin
