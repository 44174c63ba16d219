// fp8 GEMM for short A (m <= 64 rows), both operands k-contiguous (NT):
// out[b][i][j] = bf16(sum_k A[i][k] B[j][k] * fp32(sa*sb) + bias[j]).
//
// At m = 64 the product is bound by reading B once from HBM (120 flop per
// byte at 64 x 8192 x 2048), so this kernel is shaped for the load path,
// not for MFMA reuse:
//
//  * One workgroup of 8 waves owns all m rows x 32 columns of the output;
//    the column blocks are spread so that each XCD streams a contiguous slab
//    of B.  Every workgroup also reads all of A (from L2), so per CU the
//    load path carries A + 32 rows of B.
//  * Operands go global -> LDS with buffer_load_dwordx4 ... lds in chunks
//    of 512 k.  Each instruction fetches two whole 512-byte row segments
//    (4 whole 128-byte lines per row), which is what the load path needs to
//    run at full rate: the MFMA register layout itself puts 32 different
//    rows in every load instruction and runs at a quarter of that.
//  * Three chunks are in flight per workgroup (144 KB of LDS).  Within a
//    chunk each wave multiplies one 32-row group of A by B over its share
//    of the chunk's 64-k steps (k is split across the waves), so every
//    wave keeps a partial 32 x 32 tile.
//  * The partial tiles are summed through LDS in a fixed order, then
//    scaled, biased and rounded once to bf16 -- or, with the extended
//    epilogue, biased by fp8 codes times their step and / or written as fp8
//    codes of the value times the reciprocal of the output step.

#include "common.hpp"
#include "gemm_skinny.hpp"

namespace fp8lin {

namespace {

constexpr int kCols = 32;          // output columns per workgroup
constexpr int kWaves = 8;
constexpr int kChunk = 512;        // k bytes per chunk (= 8 MFMA steps, one per wave)
constexpr int kRing = 3;           // chunks in flight
constexpr int kRedStride = 36;     // floats per row of a partial tile in LDS
constexpr uint32_t kOOB = 0x80000000u;  // beyond the buffer range -> zeros

struct SkinnyParams {
    const uint8_t* a;
    const uint8_t* b;
    const float* sa;
    const float* sb;
    const void* bias;         // bf16 [n], or fp8 codes [n] when bias_scale is set
    const float* bias_scale;  // extended epilogue only
    void* out;                // bf16, or fp8 codes of format out_q when out_q >= 0
    int out_q;
    const float* out_scale;
    int64_t m, n, k, lda, ldb, stride_a, stride_b;
    int tiles_n;
    int xcd_remap;
};

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor in SGPRs (uniform base, largest record count so
// that kOOB offsets read zero).
__device__ __forceinline__ v4i rsrc_of(const uint8_t* base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = 0x7fffffff;
    r[3] = 0x00020000;
    return r;
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes go to LDS at M0 + 16*l.
// Inline asm keeps the compiler from tracking (and conservatively waiting
// on) these LDS writes; the waits are explicit (wait_vmcnt).  No output
// register; the s_nop covers the M0-write-to-LDS-DMA hazard.
__device__ __forceinline__ void dma16(const v4i& rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}

// The same with the non-temporal hint: B (the weight) is streamed once per
// call, while A is re-read by every workgroup and stays cached.  Measured
// on 64 x 8192 x 2048 with cold weights: 6.8 against 7.3 us.
__device__ __forceinline__ void dma16_nt(const v4i& rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int FMT>
__device__ __forceinline__ v16f mfma32(const v8i& x, const v8i& y, v16f acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, FMT, FMT, 0, 0, 0, 0);
}

// MT = 32-row groups of A (1 when m <= 32, else 2); EXT = extended epilogue.
template <int FMT, int MT, bool EXT>
__global__ __launch_bounds__(kWaves * 64, 1) void gemm_skinny_kernel(SkinnyParams p) {
    // A chunk is [32*MT A rows + 32 B rows][512 B]; the 16-byte pieces of row
    // r are stored at piece index c ^ (r % 16), so the 16 rows a
    // ds_read_b128 phase touches fall in 16 different bank groups.
    constexpr int kRowsA = 32 * MT, kRows = kRowsA + 32;
    constexpr int kChunkBytes = kRows * kChunk;
    constexpr int kInstr = kRows / 2;  // 1 KB DMA instructions (2 rows) per chunk
    static_assert(kInstr % kWaves == 0, "instructions per wave");
    constexpr int kPer = kInstr / kWaves;
    static_assert(kPer * (kRing - 1) < 64, "vmcnt range");
    constexpr int kRedBytes = (kWaves / MT) * kRowsA * kRedStride * 4;
    static_assert(kRedBytes <= kRing * kChunkBytes, "reduction fits the ring");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * kChunkBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int bid = blockIdx.x;
    if (p.xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const int bz = blockIdx.y;
    const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane(bid) * kCols;

    // The epilogue's scale and this thread's 4 bias values are fetched now,
    // so their latency hides under the main loop instead of adding to it.
    const float sc = (*p.sa) * (*p.sb);
    const int c4 = 4 * (threadIdx.x % (kCols / 4));  // epilogue columns of this thread
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float rq = 0.0f;  // reciprocal of the fp8 output's step
    if (p.bias) {
        if (EXT && p.bias_scale) {
            const float bs = *p.bias_scale;
            const uint8_t* bp = static_cast<const uint8_t*>(p.bias);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (n0 + c4 + c < p.n) bias[c] = dec8<FMT, 0>(bp[n0 + c4 + c]) * bs;
        } else {
            const uint16_t* bp = static_cast<const uint16_t*>(p.bias);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (n0 + c4 + c < p.n) bias[c] = bf16_to_f32(bp[n0 + c4 + c]);
        }
    }
    if (EXT && p.out_q >= 0) rq = __fdiv_rn(1.0f, *p.out_scale);

    const v4i ra = rsrc_of(p.a + (int64_t)bz * p.stride_a);
    const v4i rb = rsrc_of(p.b + (int64_t)bz * p.stride_b + n0 * p.ldb);
    const int kdim = (int)p.k;

    // DMA lane layout: instruction i of a chunk covers rows 2i, 2i+1; lane l
    // takes row 2i + l/32 and piece slot l%32, fetching piece slot ^ (row%16).
    const int half = lane >> 5, slot = lane & 31;
    auto issue = [&](int ring_slot, int chunk) {
        const int k0 = chunk * kChunk;
        uint8_t* base = smem + ring_slot * kChunkBytes;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = wave + j * kWaves;  // uniform
            const int row = 2 * i + half;
            const int kk = k0 + 16 * (slot ^ (row & 15));
            const bool is_a = 2 * i < kRowsA;  // uniform: both rows in A or in B
            const int r = is_a ? row : row - kRowsA;
            const bool ok = kk < kdim && (is_a ? r < p.m : n0 + r < p.n);
            const uint32_t off = ok ? (uint32_t)r * (uint32_t)(is_a ? p.lda : p.ldb) + kk : kOOB;
            const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)(base + 1024 * i));
            if (is_a)
                dma16(ra, la, off);
            else
                dma16_nt(rb, la, off);
        }
    };

    // Work of a wave within a chunk: A row group g = w % MT and the MT
    // consecutive 64-k steps starting at (w / MT) * MT, so every output
    // element collects 8 / MT partial sums.  Fragment of step j: lane l
    // takes row l%32 of its group and pieces 4j + 2*(l/32) + {0,1}.
    constexpr int kParts = kWaves / MT;
    const int grp = wave % MT, part = wave / MT;
    const int r32 = lane & 31;
    uint32_t flo[MT], fhi[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int c0 = 4 * (part * MT + j) + 2 * half;
        flo[j] = (uint32_t)(r32 * kChunk + 16 * (c0 ^ (r32 & 15)));
        fhi[j] = (uint32_t)(r32 * kChunk + 16 * ((c0 + 1) ^ (r32 & 15)));
    }
    auto frag = [&](const uint8_t* rows, int j) {
        const v4i x = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
            (lds_void*)(rows + flo[j]));
        const v4i y = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
            (lds_void*)(rows + fhi[j]));
        v8i v;
        v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
        v[4] = y[0]; v[5] = y[1]; v[6] = y[2]; v[7] = y[3];
        return v;
    };

    v16f acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;

    // Chunks past the end are not loaded; the waits count only what was
    // issued (chunk c and at most kRing-1 after it).
    const int nch = (kdim + kChunk - 1) / kChunk;
#pragma unroll
    for (int c = 0; c < kRing; ++c)
        if (c < nch) issue(c, c);
    for (int c0c = 0; c0c < nch; c0c += kRing) {
#pragma unroll
        for (int q = 0; q < kRing; ++q) {
            const int c = c0c + q;
            if (c >= nch) break;
            // own loads of chunk c landed; after the barrier everyone's have
            const int ahead = nch - 1 - c;
            static_assert(kRing == 3, "wait cases");
            if (ahead >= 2) wait_vmcnt<2 * kPer>();
            else if (ahead == 1) wait_vmcnt<kPer>();
            else wait_vmcnt<0>();
            barrier();
            const uint8_t* base = smem + q * kChunkBytes;
            v8i fa[MT], fb[MT];
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                fa[j] = frag(base + 32 * grp * kChunk, j);
                fb[j] = frag(base + kRowsA * kChunk, j);
            }
#pragma unroll
            for (int j = 0; j < MT; ++j) acc = mfma32<FMT>(fb[j], fa[j], acc);
            // every wave's reads of this slot are done before it is refilled
            __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
            barrier();
            if (c + kRing < nch) issue(q, c + kRing);
        }
    }
    barrier();

    // Partial tile of this wave -> LDS (over the ring).  acc[e] is row
    // 32*grp + lane%32, column 8*(e/4) + 4*(lane/32) + e%4 of the block.
    float* red = reinterpret_cast<float*>(smem);
    float* mine = red + part * (kRowsA * kRedStride);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v4f v;
        v[0] = acc[4 * q]; v[1] = acc[4 * q + 1]; v[2] = acc[4 * q + 2]; v[3] = acc[4 * q + 3];
        *reinterpret_cast<v4f*>(mine + (32 * grp + r32) * kRedStride + 8 * q + 4 * half) = v;
    }
    __syncthreads();

    // Sum the partials in a fixed order, scale, add bias, round once.
    uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)bz * p.m * p.n;
    uint8_t* out8 = static_cast<uint8_t*>(p.out) + (int64_t)bz * p.m * p.n;
    constexpr int kOut = kRowsA * kCols / 4;  // 4-column groups of the tile
    for (int t = threadIdx.x; t < kOut; t += kWaves * 64) {
        const int row = t / (kCols / 4);  // column group c4: t % 8 == threadIdx.x % 8
        if (row >= p.m) continue;
        v4f s = *reinterpret_cast<const v4f*>(red + row * kRedStride + c4);
#pragma unroll
        for (int w = 1; w < kParts; ++w)
            s += *reinterpret_cast<const v4f*>(red + w * (kRowsA * kRedStride) +
                                               row * kRedStride + c4);
        const int64_t gn = n0 + c4;
        if (EXT && p.out_q >= 0) {
            const uint32_t w = cvt4_rt(p.out_q, fmaf(s[0], sc, bias[0]) * rq,
                                       fmaf(s[1], sc, bias[1]) * rq, fmaf(s[2], sc, bias[2]) * rq,
                                       fmaf(s[3], sc, bias[3]) * rq);
            uint8_t* dst = out8 + (int64_t)row * p.n + gn;
            if (gn + 3 < p.n && ((reinterpret_cast<uintptr_t>(dst) & 3) == 0)) {
                *reinterpret_cast<uint32_t*>(dst) = w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (gn + c < p.n) dst[c] = (uint8_t)(w >> (8 * c));
            }
            continue;
        }
        const uint32_t w0 = f32x2_to_bf16x2(fmaf(s[0], sc, bias[0]), fmaf(s[1], sc, bias[1]));
        const uint32_t w1 = f32x2_to_bf16x2(fmaf(s[2], sc, bias[2]), fmaf(s[3], sc, bias[3]));
        uint16_t* dst = out + (int64_t)row * p.n + gn;
        if (gn + 3 < p.n && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        } else {
            const uint16_t h[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1,
                                   (uint16_t)(w1 >> 16)};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (gn + c < p.n) dst[c] = h[c];
        }
    }
}

}  // namespace

bool gemm_skinny_supported(const GemmLaunch& g) {
    if (g.trans_a != 0 || g.trans_b == 0) return false;  // NT only
    if (g.m < 1 || g.m > 64 || g.n < 1 || g.k < 1) return false;
    if ((reinterpret_cast<uintptr_t>(g.a) & 15) || (reinterpret_cast<uintptr_t>(g.b) & 15))
        return false;
    if ((g.lda % 16) || (g.ldb % 16) || (g.k % 16)) return false;
    if (g.batch > 1 && ((g.stride_a % 16) || (g.stride_b % 16))) return false;
    const double lim = 2147483647.0;
    if ((double)g.m * (double)g.lda >= lim || (double)g.n * (double)g.ldb >= lim) return false;
    if ((g.n + kCols - 1) / kCols >= (1 << 30) || g.batch > 65535) return false;
    return true;
}

hipError_t launch_gemm_skinny(const GemmLaunch& g, hipStream_t stream) {
    SkinnyParams p{};
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
    p.tiles_n = (int)((g.n + kCols - 1) / kCols);
    p.xcd_remap = (p.tiles_n % 8) == 0;
    const dim3 grid((unsigned)p.tiles_n, (unsigned)g.batch);
    const dim3 block(kWaves * 64);
    const int sel = g.fmt * 4 + (g.m <= 32 ? 0 : 2) + (g.ext() ? 1 : 0);
    switch (sel) {
    case 0: hipLaunchKernelGGL((gemm_skinny_kernel<0, 1, false>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<0, 1, true>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<0, 2, false>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((gemm_skinny_kernel<0, 2, true>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((gemm_skinny_kernel<1, 1, false>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((gemm_skinny_kernel<1, 1, true>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((gemm_skinny_kernel<1, 2, false>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((gemm_skinny_kernel<1, 2, true>), grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
}

}  // namespace fp8lin
