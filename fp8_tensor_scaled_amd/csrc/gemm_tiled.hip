// LDS-tiled fp8 GEMM on CDNA4 MFMA (v_mfma_f32_16x16x128_f8f6f4).
//
// Computes out[b][i][j] = bf16(sum_k A[i][k] B[k][j] * fp32(sa*sb) + bias[j])
// for the four storage layouts of the operands (AstrAI compare view
// 3e57cc8...main: csrc/kernels/fp8/common.h layout tags, the removed
// linear_backward_fp8 binding's NN dX and TN dW products, and
// gemm/epilogue.cuh for the bias / single-rounding epilogue).  The pages'
// NVIDIA mainloop (cp.async rings, ldmatrix, byte-permute transposes) is
// not followed; this is a gfx950 design:
//
//  * A workgroup of 4 waves (2x2) owns a BM x BN output tile; each wave owns
//    (BM/2) x (BN/2) and keeps its fp32 accumulators in registers.
//  * Operand tiles of 128 k are staged through LDS, double-buffered, with one
//    barrier per k-step: the next k-step's global loads are issued before
//    the MFMAs of the current one and written to the other buffer after.
//  * A k-contiguous operand ("K-major": A stored [M][K], B stored [N][K]) is
//    kept as [rows][128 B] with its 16-byte chunks XOR-swizzled by row, and
//    read as two ds_read_b128 per fragment.
//  * An m/n-contiguous operand ("MN-major": A stored [K][M], B stored
//    [K][N]) is kept as [128 k][R bytes] with 16-byte chunks XOR-swizzled by
//    k, and read with ds_read_b64_tr_b8, which transposes 8x8-byte blocks
//    across lanes so each lane receives 8 consecutive k of one row: the
//    NN / TN layouts need no separate transpose pass.
//  * The MFMA is issued with the B fragment as its first operand, so each
//    lane ends with 4 consecutive output columns of one row (8-byte bf16
//    stores, 4-wide bias loads).
//  * Workgroup ids are remapped so that each XCD (consecutive ids go to the 8
//    XCDs in turn) owns a contiguous, grouped range of output tiles: tiles
//    that share A row panels and B column panels share an L2.

#include "common.hpp"
#include "gemm_tiled.hpp"

namespace fp8lin {

constexpr int kTThreads = 256;
constexpr int kBK = 128;

struct TiledParams {
    const uint8_t* a;
    const uint8_t* b;
    const float* sa;
    const float* sb;
    const uint16_t* bias;
    uint16_t* out;
    int64_t m, n, k, lda, ldb, stride_a, stride_b;
    int64_t tiles_m, tiles_n, tiles_per_batch;
    int64_t group_m;
    int vec_out;  // out rows 8-byte aligned and n % 4 == 0
    int xcd_remap;
};

// Chunk swizzle of a K-major tile row r (8 chunks of 16 B per 128-byte row).
__device__ __forceinline__ int swz_kmajor(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Chunk swizzle of an MN-major tile row k (R / 16 chunks per row).
template <int R>
__device__ __forceinline__ int swz_mnmajor(int k) {
    if constexpr (R >= 256) return (k & 7) | (((k >> 5) & 1) << 3);
    else if constexpr (R == 128) return (k & 7) ^ ((k >> 5) & 1);
    else return (k >> 1) & 3;
}

template <bool MN, int R>
struct TileIO {
    static_assert(R % 32 == 0 && R >= 64 && R <= 256, "tile rows");
    static constexpr int kPasses = R / 32;                   // 16-byte loads per thread
    static constexpr int kChunksPerRowMN = R / 16;           // MN-major
    static constexpr int kRowsPerPassMN = kTThreads / kChunksPerRowMN;

    // Global -> registers for the k-step starting at k0.  `rows` is the
    // operand's extent along m (A) or n (B); out-of-range chunks are zero.
    __device__ static void load(uint4 (&r)[kPasses], const uint8_t* base, int64_t ld,
                                int64_t row0, int64_t rows, int64_t k0, int64_t kdim, int tid) {
#pragma unroll
        for (int q = 0; q < kPasses; ++q) {
            bool ok;
            const uint8_t* src;
            if constexpr (!MN) {
                const int row = q * 32 + tid / 8;
                const int c = tid % 8;
                const int64_t gr = row0 + row, gk = k0 + 16 * c;
                ok = gr < rows && gk < kdim;
                src = base + gr * ld + gk;
            } else {
                const int kr = q * kRowsPerPassMN + tid / kChunksPerRowMN;
                const int cm = tid % kChunksPerRowMN;
                const int64_t gk = k0 + kr, gm = row0 + 16 * cm;
                ok = gk < kdim && gm < rows;
                src = base + gk * ld + gm;
            }
            r[q] = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        }
    }

    __device__ static void store(uint8_t* lds, const uint4 (&r)[kPasses], int tid) {
#pragma unroll
        for (int q = 0; q < kPasses; ++q) {
            int off;
            if constexpr (!MN) {
                const int row = q * 32 + tid / 8;
                const int c = tid % 8;
                off = row * kBK + ((c ^ swz_kmajor(row)) << 4);
            } else {
                const int kr = q * kRowsPerPassMN + tid / kChunksPerRowMN;
                const int cm = tid % kChunksPerRowMN;
                off = kr * R + ((cm ^ swz_mnmajor<R>(kr)) << 4);
            }
            *reinterpret_cast<uint4*>(lds + off) = r[q];
        }
    }

    // MFMA operand for the 16 tile rows starting at rf: lane l gets row
    // rf + l%16 and k = 32*(l/16) .. +31 of this k-step.
    __device__ static v8i frag(const uint8_t* lds, int rf, int lane) {
        v8i v;
        if constexpr (!MN) {
            const int row = rf + (lane & 15);
            const int c0 = 2 * (lane >> 4);
            const int sw = swz_kmajor(row);
            const uint4 lo = *reinterpret_cast<const uint4*>(lds + row * kBK + ((c0 ^ sw) << 4));
            const uint4 hi =
                *reinterpret_cast<const uint4*>(lds + row * kBK + (((c0 + 1) ^ sw) << 4));
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        } else {
            // ds_read_b64_tr_b8: within each 16-lane group, lane p names the
            // 8 bytes at (k = kb + p/2, m = rf + 8*(p%2)); lane l receives the
            // bytes of m = rf + l for k = kb .. kb+7.
            const int g = lane >> 4, p = lane & 15;
            const int cm = rf >> 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int kr = 32 * g + 8 * q + (p >> 1);
                const int off = kr * R + ((cm ^ swz_mnmajor<R>(kr)) << 4) + 8 * (p & 1);
                const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(lds + off));
                v[2 * q] = t[0];
                v[2 * q + 1] = t[1];
            }
        }
        return v;
    }
};

template <int FMT, bool AMN, bool BMN, int BM, int BN>
__global__ __launch_bounds__(kTThreads, 1) void gemm_tiled_kernel(TiledParams p) {
    constexpr int kStage = (BM + BN) * kBK;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
    using IOA = TileIO<AMN, BM>;
    using IOB = TileIO<BMN, BN>;
    constexpr int FM = BM / 32;  // 16-row fragments per wave along m
    constexpr int FN = BN / 32;  // along n

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Tile of this workgroup.
    int64_t bid = blockIdx.x;
    const int64_t G = gridDim.x;
    if (p.xcd_remap) bid = (bid & 7) * (G >> 3) + (bid >> 3);
    const int64_t bz = bid / p.tiles_per_batch;
    const int64_t t = bid - bz * p.tiles_per_batch;
    const int64_t per_group = p.group_m * p.tiles_n;
    const int64_t first_m = (t / per_group) * p.group_m;
    const int64_t gsz = p.tiles_m - first_m < p.group_m ? p.tiles_m - first_m : p.group_m;
    const int64_t r = t - (t / per_group) * per_group;
    const int64_t tm = first_m + r % gsz;
    const int64_t tn = r / gsz;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    const uint8_t* A = p.a + bz * p.stride_a;
    const uint8_t* B = p.b + bz * p.stride_b;

    uint4 ra[IOA::kPasses], rb[IOB::kPasses];
    IOA::load(ra, A, p.lda, m0, p.m, 0, p.k, tid);
    IOB::load(rb, B, p.ldb, n0, p.n, 0, p.k, tid);
    IOA::store(smem, ra, tid);
    IOB::store(smem + BM * kBK, rb, tid);
    __syncthreads();

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t nk = (p.k + kBK - 1) / kBK;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) {
            IOA::load(ra, A, p.lda, m0, p.m, (kt + 1) * kBK, p.k, tid);
            IOB::load(rb, B, p.ldb, n0, p.n, (kt + 1) * kBK, p.k, tid);
        }
        const uint8_t* la = smem + cur * kStage;
        const uint8_t* lb = la + BM * kBK;
        v8i af[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = IOA::frag(la, wm * (BM / 2) + 16 * i, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const v8i bf = IOB::frag(lb, wn * (BN / 2) + 16 * j, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i][j] = mfma16x16x128<FMT>(bf, af[i], acc[i][j]);
        }
        if (more) {
            uint8_t* nxt = smem + (cur ^ 1) * kStage;
            IOA::store(nxt, ra, tid);
            IOB::store(nxt + BM * kBK, rb, tid);
        }
        __syncthreads();
    }

    // Epilogue: lane holds rows m0 + wm*BM/2 + 16i + lane%16, columns
    // n0 + wn*BN/2 + 16j + 4*(lane/16) + 0..3.
    const float s = (*p.sa) * (*p.sb);
    uint16_t* out = p.out + bz * p.m * p.n;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t gn = n0 + wn * (BN / 2) + 16 * j + 4 * (lane >> 4);
        float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (p.bias) {
            if (p.vec_out && gn + 3 < p.n) {
                const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + gn);
                bias[0] = bf16_lo(bb.x); bias[1] = bf16_hi(bb.x);
                bias[2] = bf16_lo(bb.y); bias[3] = bf16_hi(bb.y);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (gn + q < p.n) bias[q] = bf16_to_f32(p.bias[gn + q]);
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t gm = m0 + wm * (BM / 2) + 16 * i + (lane & 15);
            if (gm >= p.m) continue;
            uint16_t h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16(fmaf(acc[i][j][q], s, bias[q]));
            uint16_t* dst = out + gm * p.n + gn;
            if (p.vec_out && gn + 3 < p.n) {
                *reinterpret_cast<uint2*>(dst) =
                    make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                               (uint32_t)h[2] | ((uint32_t)h[3] << 16));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (gn + q < p.n) dst[q] = h[q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: support test, tile choice, launch.
// ---------------------------------------------------------------------------
static bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

bool gemm_tiled_supported(const GemmLaunch& g) {
    if (!aligned16(g.a) || !aligned16(g.b)) return false;
    if ((g.lda % 16) || (g.ldb % 16)) return false;
    if (g.batch > 1 && ((g.stride_a % 16) || (g.stride_b % 16))) return false;
    const bool a_mn = g.trans_a != 0, b_mn = g.trans_b == 0;
    if ((!a_mn || !b_mn) && (g.k % 16)) return false;  // k-contiguous operand
    if (a_mn && (g.m % 16)) return false;
    if (b_mn && (g.n % 16)) return false;
    return true;
}

template <int FMT, bool AMN, bool BMN, int BM, int BN>
static hipError_t launch_cfg(const GemmLaunch& g, hipStream_t stream) {
    TiledParams p{};
    p.a = g.a;
    p.b = g.b;
    p.sa = g.scale_a;
    p.sb = g.scale_b;
    p.bias = g.bias;
    p.out = g.out;
    p.m = g.m;
    p.n = g.n;
    p.k = g.k;
    p.lda = g.lda;
    p.ldb = g.ldb;
    p.stride_a = g.batch > 1 ? g.stride_a : 0;
    p.stride_b = g.batch > 1 ? g.stride_b : 0;
    p.tiles_m = (g.m + BM - 1) / BM;
    p.tiles_n = (g.n + BN - 1) / BN;
    p.tiles_per_batch = p.tiles_m * p.tiles_n;
    p.group_m = 4;
    p.vec_out = ((reinterpret_cast<uintptr_t>(g.out) & 7) == 0) && (g.n % 4 == 0) &&
                (g.bias == nullptr || (reinterpret_cast<uintptr_t>(g.bias) & 7) == 0);
    const int64_t total = p.tiles_per_batch * g.batch;
    p.xcd_remap = (total % 8) == 0;
    hipLaunchKernelGGL((gemm_tiled_kernel<FMT, AMN, BMN, BM, BN>), dim3((unsigned)total),
                       dim3(kTThreads), 0, stream, p);
    return hipGetLastError();
}

template <int FMT, bool AMN, bool BMN>
static hipError_t launch_layout(const GemmLaunch& g, hipStream_t stream) {
    // Pick the largest tile that still gives every CU at least one tile.
    const int64_t t256 = ((g.m + 255) / 256) * ((g.n + 255) / 256) * g.batch;
    const int64_t t128 = ((g.m + 127) / 128) * ((g.n + 127) / 128) * g.batch;
    if (t256 >= 256) return launch_cfg<FMT, AMN, BMN, 256, 256>(g, stream);
    if (t128 >= 256 || g.m > 64) return launch_cfg<FMT, AMN, BMN, 128, 128>(g, stream);
    return launch_cfg<FMT, AMN, BMN, 64, 64>(g, stream);
}

template <int FMT>
static hipError_t launch_fmt(const GemmLaunch& g, hipStream_t stream) {
    const bool a_mn = g.trans_a != 0, b_mn = g.trans_b == 0;
    if (!a_mn && !b_mn) return launch_layout<FMT, false, false>(g, stream);
    if (!a_mn && b_mn) return launch_layout<FMT, false, true>(g, stream);
    if (a_mn && !b_mn) return launch_layout<FMT, true, false>(g, stream);
    return launch_layout<FMT, true, true>(g, stream);
}

hipError_t launch_gemm_tiled(const GemmLaunch& g, hipStream_t stream) {
    return g.fmt == 0 ? launch_fmt<0>(g, stream) : launch_fmt<1>(g, stream);
}

}  // namespace fp8lin
