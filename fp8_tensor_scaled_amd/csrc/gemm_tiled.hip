// LDS-tiled fp8 GEMM on CDNA4 MFMA (v_mfma_f32_32x32x64_f8f6f4).
//
// Computes out[b][i][j] = bf16(sum_k A[i][k] B[k][j] * fp32(sa*sb) + bias[j])
// (or, with the extended epilogue, an fp8 bias and / or fp8 output codes)
// for the four storage layouts of the operands (AstrAI compare view
// 3e57cc8...main: csrc/kernels/fp8/common.h layout tags, the removed
// linear_backward_fp8 binding's NN dX and TN dW products, and
// gemm/epilogue.cuh for the bias / single-rounding epilogue).  The pages'
// NVIDIA mainloop (cp.async rings, ldmatrix, byte-permute transposes) is
// not followed; this is a gfx950 design:
//
//  * A workgroup of WM x WN waves owns a BM x BN output tile; each wave owns
//    (BM/WM) x (BN/WN) as 32x32 MFMA tiles with fp32 accumulators in
//    registers.
//  * A stage holds 128 k of both operand tiles; the MFMAs take it in two
//    substeps of 64 k.  Operand tiles go global -> LDS with
//    buffer_load_dwordx4 ... lds (no register staging): each instruction
//    writes 1 KB of LDS in lane order, and each lane picks the 16 global
//    bytes that belong at its LDS slot, which is how the XOR swizzle is
//    applied.  128 k per stage makes every row segment a load touches a
//    whole 128-byte line: half-line segments measured at half the load
//    throughput on this part.  Out-of-range chunks (matrix tails, stages past
//    the end of k) use an offset beyond the buffer range and arrive as zeros.
//  * STAGES LDS buffers form a ring.  In the second substep of stage t each
//    wave waits for its own loads of stage t+1 (vmcnt) and for its LDS reads
//    of stage t; a raw s_barrier then makes everyone's loads visible and
//    frees buffer t, which receives stage t+STAGES.  The loop is unrolled by
//    STAGES so that every LDS offset is a compile-time constant.
//  * A k-contiguous operand ("K-major": A stored [M][K], B stored [N][K]) is
//    kept as [rows][128 B] and read with two ds_read_b128 per fragment; an
//    m/n-contiguous operand ("MN-major": A stored [K][M], B stored [K][N])
//    is kept as [128 k][R bytes] and read with ds_read_b64_tr_b8, which
//    transposes 8x8-byte blocks across lanes so each lane receives 8
//    consecutive k of one row: NN / TN need no transpose pass.  The
//    swizzles make both read patterns conflict-free on gfx950's 64-bank LDS
//    (16 lanes per cycle for 16-byte reads).
//  * The MFMA takes the B fragment as its first operand, so each lane ends
//    with runs of 4 consecutive output columns of one row.
//  * Workgroup ids are remapped so that each XCD (consecutive ids go to the 8
//    XCDs in turn) owns a contiguous, grouped range of output tiles: tiles
//    that share A row panels and B column panels share an L2.

#include <type_traits>

#include "common.hpp"
#include "gemm_tiled.hpp"

namespace fp8lin {

constexpr int kSub = 64;  // k per MFMA substep
typedef __attribute__((address_space(3))) void lds_void;

struct TiledParams {
    const uint8_t* a;
    const uint8_t* b;
    const float* sa;
    const float* sb;
    const void* bias;         // bf16 [n], or fp8 codes [n] when bias_scale is set
    const float* bias_scale;  // extended epilogue only
    void* out;                // bf16, or fp8 codes when out_q >= 0
    int out_q;                // extended epilogue only: -1 bf16, 0 E4M3, 1 E5M2
    const float* out_scale;
    int64_t m, n, k, lda, ldb, stride_a, stride_b;
    int tiles_m, tiles_n, tiles_per_batch;
    int group_m;
    int vec_out;    // 4-element output stores: out aligned for them and n % 4 == 0
    int vec_out16;  // output rows in whole 16-byte chunks, 16-byte aligned (LDS-staged)
    int vec_bias;   // 4-element bias loads: bias aligned for them (or no bias)
    int xcd_remap;
};

// vmcnt-only wait (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] at [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// lgkmcnt(0) only (LDS reads of this wave complete).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Chunk swizzle of a K-major tile row r (BK/16 chunks of 16 B per row).  A
// ds_read_b128 phase reads one chunk column of 16 consecutive rows.
// 128-byte rows: rows 2i and 2i+1 differ in the bank half and (r/2) % 8
// spreads the 8 row pairs over the 8 chunk positions.  64-byte rows: 4 rows
// share a 256-byte bank line, (r/2) % 4 and r/8 spread the rest.  Either way
// the 16 reads hit 16 distinct bank groups.  Only bits 1..3 of r are used.
template <int BK>
__device__ __forceinline__ int swz_kmajor(int r) {
    if constexpr (BK == 128) return (r >> 1) & 7;
    else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

// Chunk swizzle of an MN-major tile row k (R / 16 chunks per row): even
// values, so the two 16-lane groups of a transposed-read phase (adjacent
// chunks, same rows) never share a bank group.  Depends on k % 8 only
// through the bits used, so rows k and k + 8q share it.
template <int R>
__device__ __forceinline__ int swz_mnmajor(int k) {
    if constexpr (R >= 256) return (k & 7) << 1;
    else if constexpr (R == 128) return ((k >> 1) & 3) << 1;
    else return ((k >> 2) & 1) << 1;
}

constexpr uint32_t kOOB = 0x80000000u;  // beyond every buffer range -> zeros

// Buffer descriptor (raw, 4 dwords): base address, no stride, the largest
// record count (offsets past it, such as kOOB, read as zero), and the
// default data format.  The base is uniform; readfirstlane says so to the
// compiler, so the descriptor lives in SGPRs.
__device__ __forceinline__ v4i make_rsrc(const void* base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = 0x7fffffff;
    r[3] = 0x00020000;
    return r;
}

// One buffer_load_dwordx4 ... lds: lane l fetches 16 bytes at descriptor base
// + voff and the hardware writes them to LDS at M0 + 16*l.  Written as
// inline asm so that the compiler does not track these LDS writes: its own
// tracking merges them at the k-loop back edge and then waits for every load
// in flight before the next fragment read, which drains the prefetch ring.
// The ring's waits are explicit here (wait_vmcnt), and nothing else in the
// k loop uses the vector memory counter.  The instruction has no output
// register; the s_nop covers the M0-write-to-LDS-DMA hazard.
__device__ __forceinline__ void dma16(const v4i& rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p);
}

template <bool MN, int R, int NW, int BK>
struct Operand {
    static_assert(R == 64 || R == 128 || R == 256, "tile rows");
    static_assert(BK == 64 || BK == 128, "stage depth");
    static constexpr int kInstr = R * BK / 1024;  // 1 KB DMA instructions per stage
    static_assert(kInstr % NW == 0, "instructions per wave");
    static constexpr int kPerWave = kInstr / NW;

    // Lane layout of DMA instruction j of this wave: the tile row (K-major:
    // 1024/BK rows x BK bytes per instruction) or k row (MN-major: 1024/R
    // rows x R bytes) and the 16-byte chunk it fetches.
    __device__ static void slot(int j, int wave, int lane, int& row, int& chunk) {
        const int i = wave + j * NW;
        if constexpr (!MN) {
            constexpr int kLanesPerRow = BK / 16;
            row = (64 / kLanesPerRow) * i + lane / kLanesPerRow;
            chunk = (lane % kLanesPerRow) ^ swz_kmajor<BK>(row);
        } else {
            constexpr int kRowsPer = 1024 / R;
            constexpr int kChunks = R / 16;
            row = kRowsPer * i + lane / kChunks;
            chunk = (lane % kChunks) ^ swz_mnmajor<R>(row);
        }
    }

    // Instruction j of a wave covers the rows of instruction 0 shifted by
    // j*NW instructions; the swizzle of those rows is the same (the shift is
    // a multiple of 16 rows for K-major, of 8 k rows for MN-major), so the
    // offset of instruction j is that of instruction 0 plus a uniform stride.
    static constexpr int kRowStep = NW * (MN ? 1024 / R : 1024 / BK);  // rows per j
    static_assert(NW % 2 == 0, "row shift keeps the swizzle");

    // Per-lane byte offset of instruction 0 at k = 0.  MN-major: kOOB when
    // the lane's 16 columns lie outside the matrix (the same for every j).
    // `rows_left` = extent of the operand along m (A) or n (B) from this
    // tile's origin.
    __device__ static uint32_t init(uint32_t ld, int64_t rows_left, int wave, int lane) {
        int row, c;
        slot(0, wave, lane, row, c);
        if constexpr (!MN) return (uint32_t)row * ld + 16 * c;
        else return 16 * c < rows_left ? (uint32_t)row * ld + 16 * c : kOOB;
    }

    // Issue this wave's DMA loads of the stage starting at k0 into `lds`.
    // All offsets are 32-bit (the host only takes this path when every
    // operand slice is addressable that way; kOOB plus any in-range offset
    // stays below 2^32 and beyond the range).  `full_rows`: every tile row
    // exists (uniform), else K-major rows past the edge read zeros.
    __device__ static void issue(const v4i& rs, uint8_t* lds, uint32_t base, uint32_t ld, int k0,
                                 int kdim, bool full_rows, int64_t rows_left, int wave, int lane) {
        const uint32_t delta = MN ? (uint32_t)k0 * ld : (uint32_t)k0;
        const uint32_t jstride = (uint32_t)kRowStep * ld;
        const bool full = k0 + BK <= kdim;  // uniform: no k tail in this stage
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            uint32_t off = base + delta + j * jstride;
            if (!full || (!MN && !full_rows)) {
                int row, c;
                slot(j, wave, lane, row, c);
                const int gk = MN ? k0 + row : k0 + 16 * c;
                if (gk >= kdim) off = kOOB;
                if (!MN && row >= rows_left) off = kOOB;
            }
            dma16(rs, lds_addr(lds + 1024 * (wave + j * NW)), off);
        }
    }

    // Offset of this lane for DMA instruction j of the stage at k0 (kOOB past
    // the matrix), and the LDS address instruction j writes.
    __device__ static uint32_t off_of(uint32_t base, uint32_t ld, int k0, int kdim,
                                      bool full_rows, int64_t rows_left, int j, int wave,
                                      int lane) {
        const uint32_t delta = MN ? (uint32_t)k0 * ld : (uint32_t)k0;
        uint32_t off = base + delta + j * ((uint32_t)kRowStep * ld);
        if (!(k0 + BK <= kdim) || (!MN && !full_rows)) {
            int row, c;
            slot(j, wave, lane, row, c);
            const int gk = MN ? k0 + row : k0 + 16 * c;
            if (gk >= kdim) off = kOOB;
            if (!MN && row >= rows_left) off = kOOB;
        }
        return off;
    }
    __device__ static uint32_t lds_of(uint8_t* lds, int j, int wave) {
        return lds_addr(lds + 1024 * (wave + j * NW));
    }

    // Fragment addressing.  The MFMA operand of the 32 tile rows starting at
    // rf, substep h, gives lane l row rf + l%32 and k = 64h + 32*(l/32) ..
    // +31 of the stage.  The lane-dependent part of each address is computed
    // once (frag_off); the rest is a compile-time constant or a fixed XOR.
    //
    // K-major: rf is a multiple of 32, so the swizzle depends on the lane
    // only and rf adds rf*128.  The 16-byte pieces wanted are chunks
    // 4h + 2*(l/32) + e (e = 0, 1); their bits are disjoint, so the swizzled
    // chunk is (2*(l/32) ^ swizzle) ^ 4h ^ e, i.e. the substep and the half
    // flip bits 6 and 4 of the lane's offset.
    // MN-major (ds_read_b64_tr_b8): within each 16-lane group, lane p names
    // the 8 bytes at (k = kb + 8q + p/2, m = mb + 8*(p%2)) and lane p of the
    // group receives m = mb + p for k = kb+8q .. +7 (q = 0..3), with kb =
    // 64h + 32*(group/2).  The swizzle of row k depends on p only, so h and
    // q add (64h + 8q)*R; the chunk (mb/16) ^ swizzle stays per fragment.
    __device__ static uint32_t frag_off(int rf, int lane) {
        if constexpr (!MN) {
            const int row = lane & 31;  // rf*128 is added as a constant
            const int c = (2 * (lane >> 5)) ^ swz_kmajor<BK>(row);
            (void)rf;
            return (uint32_t)(row * BK + (c << 4));
        } else {
            const int g = lane >> 4, p = lane & 15;
            const int mb = rf + 16 * (g & 1);
            const int kr = 32 * (g >> 1) + (p >> 1);
            return (uint32_t)(kr * R + (((mb >> 4) ^ swz_mnmajor<R>(kr)) << 4) + 8 * (p & 1));
        }
    }

    // Reads the substep-H fragment: `lds` = stage start (K-major: plus
    // rf*BK), `off` = frag_off(rf, lane).
    template <int H>
    __device__ static v8i frag(const uint8_t* lds, uint32_t off) {
        v8i v;
        if constexpr (!MN) {
            const v4i lo = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
                (lds_void*)(lds + (off ^ (64u * H))));
            const v4i hi = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
                (lds_void*)(lds + (off ^ (64u * H + 16u))));
            v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
            v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(lds + off + (kSub * H + 8 * q) * R));
                v[2 * q] = t[0];
                v[2 * q + 1] = t[1];
            }
        }
        return v;
    }
};

// Order of the DMA instructions of one refill.  A refill is one stage
// (P = 1: A's instructions, then B's) or a pair of 64-k stages X, Y (P = 2).
// In a pair, a k-contiguous operand alternates its X and Y instructions, so
// the two 64-byte halves of every line it reads go out back to back; an
// m/n-contiguous operand (whole lines either way) issues all of its X
// instructions and then all of its Y instructions, after the alternating
// ones.  Loads complete in issue order, so what may still be in flight once
// X has landed is exactly the refill's instructions after the last X one
// (pair_tail_x).
struct DmaSlot {
    int op;  // 0: A, 1: B
    int j;   // instruction of that operand's stage
    int h;   // 0: X (or the single stage), 1: Y
};

template <int NA, int NB, bool IA, bool IB, int P>
__host__ __device__ constexpr DmaSlot dma_slot(int x) {
    if (P == 1) return x < NA ? DmaSlot{0, x, 0} : DmaSlot{1, x - NA, 0};
    const int ia = IA ? 2 * NA : 0, ib = IB ? 2 * NB : 0;
    if (x < ia) return DmaSlot{0, x / 2, x % 2};
    x -= ia;
    if (x < ib) return DmaSlot{1, x / 2, x % 2};
    x -= ib;
    constexpr int ba = IA ? 0 : NA, bb = IB ? 0 : NB;  // blocked instructions per stage
    if constexpr (ba + bb == 0) return DmaSlot{-1, -1, -1};  // x out of range
    const int h = x / (ba + bb);
    x -= h * (ba + bb);
    return x < ba ? DmaSlot{0, x, h} : DmaSlot{1, x - ba, h};
}

template <int NA, int NB, bool IA, bool IB>
constexpr int pair_tail_x() {
    const int blocked = (IA ? 0 : NA) + (IB ? 0 : NB);
    return blocked > 0 ? blocked : 1;
}

// Compile-time check of a pair order: every (operand, instruction, stage)
// issued exactly once, and exactly pair_tail_x instructions after the last
// X one.
template <int NA, int NB, bool IA, bool IB>
constexpr bool pair_order_ok() {
    static_assert(NA <= 8 && NB <= 8, "checker bounds");
    int seen[2][8][2] = {};
    int last_x = -1;
    const int n = 2 * (NA + NB);
    for (int x = 0; x < n; ++x) {
        const DmaSlot d = dma_slot<NA, NB, IA, IB, 2>(x);
        if (d.op < 0 || d.op > 1 || d.h < 0 || d.h > 1 || d.j < 0 || d.j >= (d.op ? NB : NA))
            return false;
        ++seen[d.op][d.j][d.h];
        if (d.h == 0) last_x = x;
    }
    for (int op = 0; op < 2; ++op)
        for (int j = 0; j < (op ? NB : NA); ++j)
            if (seen[op][j][0] != 1 || seen[op][j][1] != 1) return false;
    return n - 1 - last_x == pair_tail_x<NA, NB, IA, IB>();
}
static_assert(pair_order_ok<2, 2, true, true>() && pair_order_ok<2, 2, true, false>() &&
                  pair_order_ok<2, 2, false, true>() && pair_order_ok<2, 2, false, false>() &&
                  pair_order_ok<1, 3, true, false>() && pair_order_ok<3, 1, false, true>(),
              "pair refill order");

template <int FMT>
__device__ __forceinline__ v16f mfma32x32x64(const v8i& x, const v8i& y, v16f acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, FMT, FMT, 0, 0, 0, 0);
}

// LDS bytes of a configuration's ring (also its epilogue staging area).
template <int BM, int BN, int BK, int STAGES>
constexpr int tiled_lds_bytes() {
    return STAGES * (BM + BN) * BK;
}

// A held-back fold carried by a GEMM launch: waves 0 and 1 of its extra
// workgroup fold one ring each.
__device__ __forceinline__ void fold_waves(const FoldJob& fold) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
    if (wave == 0) fold_ring_lines(fold.r[0]);
    else if (wave == 1 && fold.n > 1) fold_ring_lines(fold.r[1]);
}

// One output tile: workgroup `bid` of a grid of G workgroups over problem p,
// with `smem` the workgroup's LDS ring of tiled_lds_bytes<...>() bytes.
// Four bias values of columns gn .. gn+3 (zero past n) for the extended
// epilogue: bf16, or fp8 codes of FMT times their step bs.
template <int FMT>
__device__ __forceinline__ void ext_bias4(const TiledParams& p, float bs, int64_t gn,
                                          float b[4]) {
    b[0] = b[1] = b[2] = b[3] = 0.0f;
    if (!p.bias || gn >= p.n) return;
    const bool whole = p.vec_bias && gn + 3 < p.n;
    if (p.bias_scale) {
        const uint8_t* bp = static_cast<const uint8_t*>(p.bias) + gn;
        if (whole) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(bp);
            b[0] = dec8<FMT, 0>(w) * bs; b[1] = dec8<FMT, 1>(w) * bs;
            b[2] = dec8<FMT, 2>(w) * bs; b[3] = dec8<FMT, 3>(w) * bs;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (gn + c < p.n) b[c] = dec8<FMT, 0>(bp[c]) * bs;
        }
    } else {
        const uint16_t* bp = static_cast<const uint16_t*>(p.bias) + gn;
        if (whole) {
            const uint2 bb = *reinterpret_cast<const uint2*>(bp);
            b[0] = bf16_lo(bb.x); b[1] = bf16_hi(bb.x);
            b[2] = bf16_lo(bb.y); b[3] = bf16_hi(bb.y);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (gn + c < p.n) b[c] = bf16_to_f32(bp[c]);
        }
    }
}

// EXT selects the extended epilogue (fp8 bias and / or fp8 output, chosen at
// run time); without it the epilogue is the plain bf16 one.
template <int FMT, bool AMN, bool BMN, int BM, int BN, int WM, int WN, int BK, int STAGES,
          bool EXT = false>
__device__ __forceinline__ void gemm_tile(const TiledParams& p, int bid, const int G,
                                          uint8_t* smem) {
    constexpr int NW = WM * WN;
    constexpr int kSubs = BK / kSub;  // MFMA substeps per stage
    static_assert((STAGES * kSubs) % 2 == 0, "fragment slots alternate with the unrolled steps");
    static_assert(kSubs == 2 || (STAGES >= 4 && STAGES % 2 == 0), "64-k stages refill in pairs");
    constexpr int kStageA = BM * BK, kStageB = BN * BK;
    constexpr int kStage = kStageA + kStageB;
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
    static_assert(FM >= 1 && FN >= 1, "wave tile");
    using OA = Operand<AMN, BM, NW, BK>;
    using OB = Operand<BMN, BN, NW, BK>;
    constexpr int kLoads = OA::kPerWave + OB::kPerWave;  // DMA loads per wave per stage
    static_assert(STAGES >= 2 && kLoads * (STAGES - 1) < 64, "vmcnt range");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wm = wave / WN, wn = wave % WN;

    // Tile of this workgroup (32-bit, uniform: tile counts fit easily).
    if (p.xcd_remap) bid = (bid & 7) * (G >> 3) + (bid >> 3);
    const int bz = bid / p.tiles_per_batch;
    const int t = bid - bz * p.tiles_per_batch;
    const int per_group = p.group_m * p.tiles_n;
    const int first_m = (t / per_group) * p.group_m;
    const int gsz = p.tiles_m - first_m < p.group_m ? p.tiles_m - first_m : p.group_m;
    const int r = t - (t / per_group) * per_group;
    const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((first_m + r % gsz) * BM);
    const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((r / gsz) * BN);

    // The epilogue's scale, fetched now so its latency hides under the loop.
    const float sc = (*p.sa) * (*p.sb);
    float ext_bs = 0.0f, ext_rq = 0.0f;  // bias step, output step's reciprocal
    if constexpr (EXT) {
        if (p.bias_scale) ext_bs = *p.bias_scale;
        if (p.out_q >= 0) ext_rq = __fdiv_rn(1.0f, *p.out_scale);
    }

    // Buffer descriptors based at this tile's first row / column.
    const uint8_t* A = p.a + (int64_t)bz * p.stride_a + (AMN ? m0 : m0 * p.lda);
    const uint8_t* B = p.b + (int64_t)bz * p.stride_b + (BMN ? n0 : n0 * p.ldb);
    const v4i ra = make_rsrc(A);
    const v4i rb = make_rsrc(B);
    const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
    const int kdim = (int)p.k;
    const int64_t arows = p.m - m0, brows = p.n - n0;
    const bool afull = arows >= BM, bfull = brows >= BN;
    const uint32_t abase = OA::init(lda, arows, wave, lane);
    const uint32_t bbase = OB::init(ldb, brows, wave, lane);

    auto issue = [&](int stage, int kstage) {
        uint8_t* s = smem + stage * kStage;
        OA::issue(ra, s, abase, lda, kstage * BK, kdim, afull, arows, wave, lane);
        OB::issue(rb, s + kStageA, bbase, ldb, kstage * BK, kdim, bfull, brows, wave, lane);
    };

    // Fragments are read one substep ahead: while substep u's MFMAs run, the
    // fragments of u+1 are already coming in from LDS, so the MFMA pipe does
    // not idle behind LDS latency.  Substeps alternate between two register
    // slots.
    v8i af[2][FM], bf[2][FN];
    // Per-lane fragment offsets within a stage (see Operand::frag_off).
    uint32_t aoff[FM], boff[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) aoff[i] = OA::frag_off(AMN ? wm * TM + 32 * i : 0, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) boff[j] = OB::frag_off(BMN ? wn * TN + 32 * j : 0, lane);
    // K-major fragments add the wave's first tile row as a byte offset.
    constexpr int kRowA = AMN ? 0 : BK, kRowB = BMN ? 0 : BK;
    const uint32_t arow = (uint32_t)(wm * TM * kRowA);
    const uint32_t brow = (uint32_t)(wn * TN * kRowB);
    // read_frags(slot, substep, buffer)
    auto read_frags = [&](auto slotc, auto hc, int buf) {
        constexpr int SL = decltype(slotc)::value, H = decltype(hc)::value;
        const uint8_t* la = smem + buf * kStage + arow;
        const uint8_t* lb = smem + buf * kStage + kStageA + brow;
#pragma unroll
        for (int i = 0; i < FM; ++i) af[SL][i] = OA::template frag<H>(la + 32 * i * kRowA, aoff[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[SL][j] = OB::template frag<H>(lb + 32 * j * kRowB, boff[j]);
    };
    // The empty asm statements keep the compiler from moving LDS accesses
    // across the raw barriers.
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // The DMA instructions of one refill (a stage, or a pair of 64-k stages
    // in the order dma_slot gives): offsets and LDS addresses are computed
    // right after the barrier, the instructions themselves are spread
    // between the MFMAs.  Issued in one burst, 8 waves x 8 instructions fill
    // the texture addresser's queue and the waves at its back stall before
    // their first MFMA.
    constexpr int kPairs = kSubs == 1 ? 2 : 1;
    constexpr int kND = (OA::kPerWave + OB::kPerWave) * kPairs;
    constexpr int kPA = OA::kPerWave, kPB = OB::kPerWave;
    constexpr bool kIA = !AMN, kIB = !BMN;  // k-contiguous: alternate X / Y
    uint32_t doff[kND], dlds[kND];
    auto plan_refill = [&](int s0, int s1, int kstage) {
#pragma unroll
        for (int x = 0; x < kND; ++x) {
            const DmaSlot d = dma_slot<kPA, kPB, kIA, kIB, kPairs>(x);
            uint8_t* dst = smem + (d.h ? s1 : s0) * kStage;
            if (d.op == 0) {
                doff[x] = OA::off_of(abase, lda, (kstage + d.h) * BK, kdim, afull, arows, d.j,
                                     wave, lane);
                dlds[x] = OA::lds_of(dst, d.j, wave);
            } else {
                doff[x] = OB::off_of(bbase, ldb, (kstage + d.h) * BK, kdim, bfull, brows, d.j,
                                     wave, lane);
                dlds[x] = OB::lds_of(dst + kStageA, d.j, wave);
            }
        }
    };
    auto issue_planned = [&](int x) {
        dma16(dma_slot<kPA, kPB, kIA, kIB, kPairs>(x).op == 0 ? ra : rb, dlds[x], doff[x]);
    };
    // Pairs: loads that may be in flight when the first stage of a pair has
    // landed (the pair's instructions after its last X one).
    constexpr int kTailX = pair_tail_x<kPA, kPB, kIA, kIB>();

    // One substep: the MFMAs of register slot SL; between them, in this
    // order, the fragment reads of the next substep (slot NSL, substep NH of
    // buffer nbuf) and, when `refill`, the planned DMA instructions.  The
    // sched_barriers keep that interleave exactly as written.
    constexpr int kMF = FM * FN;
    constexpr int kFR = FM + FN;
    constexpr int kFRPer = (kFR + kMF - 1) / kMF;
    // With three or more stages a refill has more than a stage of slack, so
    // its DMA instructions go out over two substeps: the first kH in the
    // substep after the barrier, the rest in the next stage's first
    // substep (still before the next barrier, so every wait below counts
    // whole refills).  Half the instructions per MFMA keep the texture
    // addresser's queue from filling (training-shape GEMMs 3-7 % faster).
    constexpr bool kSplit = kSubs == 2 && STAGES >= 3;
    constexpr int kH = (kND + 1) / 2;
    auto substep = [&](auto slc, auto nslc, auto nhc, int nbuf, auto partc) {
        constexpr int SL = decltype(slc)::value, NSL = decltype(nslc)::value;
        constexpr int NH = decltype(nhc)::value;
        // planned DMA instructions issued here: 0 none, 1 [0, kH),
        // 2 [kH, kND), 3 all
        constexpr int P = decltype(partc)::value;
        constexpr int x0 = P == 2 ? kH : 0;
        constexpr int x1 = P == 1 ? kH : kND;
        constexpr int nD = P == 0 ? 0 : x1 - x0;
        constexpr int kDPer = (nD + kMF - 1) / kMF;
        const uint8_t* la = smem + nbuf * kStage + arow;
        const uint8_t* lb = smem + nbuf * kStage + kStageA + brow;
#pragma unroll
        for (int m = 0; m < kMF; ++m) {
            const int i = m % FM, j = m / FM;
            acc[i][j] = mfma32x32x64<FMT>(bf[SL][j], af[SL][i], acc[i][j]);
#pragma unroll
            for (int q = 0; q < kFRPer; ++q) {
                const int f = m * kFRPer + q;
                if (f < FM) af[NSL][f] = OA::template frag<NH>(la + 32 * f * kRowA, aoff[f]);
                else if (f < kFR)
                    bf[NSL][f - FM] =
                        OB::template frag<NH>(lb + 32 * (f - FM) * kRowB, boff[f - FM]);
            }
            if constexpr (P != 0) {
#pragma unroll
                for (int q = 0; q < kDPer; ++q) {
                    const int x = x0 + m * kDPer + q;
                    if (x < x1) issue_planned(x);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using PNone = std::integral_constant<int, 0>;
    using PAll = std::integral_constant<int, 3>;
    using PFirst = std::integral_constant<int, kSplit ? 1 : 3>;
    using PSecond = std::integral_constant<int, kSplit ? 2 : 0>;

    // Prologue: every buffer starts loading; stage 0's first fragments are
    // read.  Pairs go out in the loop's refill order; stage 0 is the X of
    // the first pair, so the rest of that pair's tail and the later pairs
    // may still be in flight.
    if constexpr (kSubs == 1) {
#pragma unroll
        for (int s = 0; s < STAGES; s += 2) {
            plan_refill(s, s + 1, s);
#pragma unroll
            for (int x = 0; x < kND; ++x) issue_planned(x);
        }
        wait_vmcnt<kTailX + kLoads * (STAGES - 2)>();
    } else {
        if constexpr (kSplit) {
            // the last stage's second half goes out in stage 0's first
            // substep, as a refill's would
#pragma unroll
            for (int s = 0; s < STAGES - 1; ++s) issue(s, s);
            plan_refill(STAGES - 1, STAGES - 1, STAGES - 1);
#pragma unroll
            for (int x = 0; x < kH; ++x) issue_planned(x);
            wait_vmcnt<kLoads * (STAGES - 2) + kH>();
        } else {
#pragma unroll
            for (int s = 0; s < STAGES; ++s) issue(s, s);
            wait_vmcnt<kLoads * (STAGES - 1)>();
        }
    }
    barrier();
    read_frags(I0{}, I0{}, 0);

    // One stage = kSubs substeps.  Every substep but the last reads the next
    // substep of the same buffer.  The last one first waits for its own
    // loads of stage st+1 and its reads of this stage; after the barrier
    // that holds for every wave, so st+1 can be read and this buffer
    // refilled with st+STAGES.
    const int nk = (kdim + BK - 1) / BK;
    for (int t0 = 0; t0 < nk; t0 += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
            const int st = t0 + s;
            if (st >= nk) break;
            if constexpr (kSubs == 2) {
                // substep 0 uses slot 0, substep 1 slot 1
                substep(I0{}, I1{}, I1{}, s, PSecond{});
                wait_vmcnt<kLoads * (STAGES - 2)>();
                wait_lgkmcnt0();
                barrier();
                plan_refill(s, s, st + STAGES);
                substep(I1{}, I0{}, I0{}, (s + 1) % STAGES, PFirst{});
            } else {
                // 64-k stages are refilled in pairs: at every odd step the
                // slots of this step and the one before take steps
                // st+STAGES-1 and st+STAGES, so pairs are (even, odd) steps.
                // Loads that may be in flight when the awaited step st+1 has
                // landed: odd st (st+1 is a pair's X): the tail of its pair
                // after the last X instruction plus the later pairs; even st
                // (st+1 is a Y): the later pairs only.
                if (s & 1) wait_vmcnt<kTailX + kLoads * (STAGES - 4)>();
                else wait_vmcnt<kLoads * (STAGES - 2)>();
                wait_lgkmcnt0();
                barrier();
                if (s & 1) {
                    plan_refill(s - 1, s, st + STAGES - 1);
                    substep(I1{}, I0{}, I0{}, (s + 1) % STAGES, PAll{});
                } else {
                    substep(I0{}, I1{}, I0{}, (s + 1) % STAGES, PNone{});
                }
            }
        }
    }
    wait_vmcnt<0>();  // drain the (out-of-range) prefetches before exit

    // Epilogue: acc[i][j][e] is row m0 + wm*TM + 32i + lane%32, column
    // n0 + wn*TN + 32j + 8*(e/4) + 4*(lane/32) + e%4.
    if constexpr (EXT) {
        // Output element of OB bytes: 2 (bf16) or 1 (fp8 code of format
        // out_q).  The same two store forms as the plain epilogue below.
        auto store = [&](auto ob_tag) __attribute__((always_inline)) {
            constexpr int OB = decltype(ob_tag)::value;
            uint8_t* outb = static_cast<uint8_t*>(p.out) + (int64_t)bz * p.m * p.n * OB;
            // four consecutive outputs -> their packed bytes (8 or 4)
            auto pack = [&](float v0, float v1, float v2, float v3) __attribute__((always_inline)) {
                if constexpr (OB == 2) {
                    v2i pk;
                    pk[0] = (int)f32x2_to_bf16x2(v0, v1);
                    pk[1] = (int)f32x2_to_bf16x2(v2, v3);
                    return pk;
                } else {
                    return cvt4_rt(p.out_q, v0 * ext_rq, v1 * ext_rq, v2 * ext_rq, v3 * ext_rq);
                }
            };
            if (p.vec_out16) {
                constexpr int kRowBytes = TN * OB;
                constexpr int kChunks = kRowBytes / 16;
                constexpr int kRowsPerPass = 64 / kChunks;
                constexpr int kRegion = TM * kRowBytes;
                static_assert(NW * kRegion <= STAGES * kStage, "epilogue staging fits");
                barrier();  // every wave is done with the operand buffers
                uint8_t* wl = smem + wave * kRegion;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int cl = 32 * j + 8 * q + 4 * (lane >> 5);
                        float bias[4];
                        ext_bias4<FMT>(p, ext_bs, n0 + wn * TN + cl, bias);
#pragma unroll
                        for (int i = 0; i < FM; ++i) {
                            const int r = 32 * i + (lane & 31);
                            const int byte = cl * OB;
                            const int chunk = (byte >> 4) ^ (r % kChunks);
                            const auto v = pack(fmaf(acc[i][j][4 * q + 0], sc, bias[0]),
                                                fmaf(acc[i][j][4 * q + 1], sc, bias[1]),
                                                fmaf(acc[i][j][4 * q + 2], sc, bias[2]),
                                                fmaf(acc[i][j][4 * q + 3], sc, bias[3]));
                            *reinterpret_cast<__attribute__((address_space(3)))
                                              std::remove_const_t<decltype(v)>*>(
                                (lds_void*)(wl + r * kRowBytes + chunk * 16 + (byte & 15))) = v;
                        }
                    }
                }
                const int cc = lane % kChunks;
                const int64_t gn = n0 + wn * TN + (16 / OB) * cc;
#pragma unroll
                for (int ps = 0; ps < TM / kRowsPerPass; ++ps) {
                    const int r = ps * kRowsPerPass + lane / kChunks;
                    const v4i v = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
                        (lds_void*)(wl + r * kRowBytes + ((cc ^ (r % kChunks)) << 4)));
                    const int64_t gm = m0 + wm * TM + r;
                    if (gm < p.m && gn < p.n)
                        *reinterpret_cast<v4i*>(outb + (gm * p.n + gn) * OB) = v;
                }
                return;
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t gn = n0 + wn * TN + 32 * j + 8 * q + 4 * (lane >> 5);
                    float bias[4];
                    ext_bias4<FMT>(p, ext_bs, gn, bias);
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const int64_t gm = m0 + wm * TM + 32 * i + (lane & 31);
                        if (gm >= p.m || gn >= p.n) continue;
                        const auto v = pack(fmaf(acc[i][j][4 * q + 0], sc, bias[0]),
                                            fmaf(acc[i][j][4 * q + 1], sc, bias[1]),
                                            fmaf(acc[i][j][4 * q + 2], sc, bias[2]),
                                            fmaf(acc[i][j][4 * q + 3], sc, bias[3]));
                        uint8_t* dst = outb + (gm * p.n + gn) * OB;
                        if (p.vec_out && gn + 3 < p.n) {
                            *reinterpret_cast<std::remove_const_t<decltype(v)>*>(dst) = v;
                        } else {
                            uint8_t bytes[4 * OB];
                            __builtin_memcpy(bytes, &v, 4 * OB);
                            for (int c = 0; c < 4 && gn + c < p.n; ++c)
                                __builtin_memcpy(dst + c * OB, bytes + c * OB, OB);
                        }
                    }
                }
            }
        };
        if (p.out_q < 0)
            store(std::integral_constant<int, 2>{});
        else
            store(std::integral_constant<int, 1>{});
        return;
    }
    uint16_t* out = static_cast<uint16_t*>(p.out) + bz * p.m * p.n;
    const uint16_t* bias_p = static_cast<const uint16_t*>(p.bias);
    if (p.vec_out16) {
        // Through LDS: each wave rounds its tile to bf16 into its own LDS
        // region (16-byte chunks XOR-swizzled by row), then writes whole
        // 16-byte chunks, 8 lanes per row, so every store instruction fills
        // complete 128-byte lines instead of scattering 8-byte pieces.
        constexpr int kRowBytes = TN * 2;
        constexpr int kChunks = kRowBytes / 16;
        constexpr int kRowsPerPass = 64 / kChunks;
        constexpr int kRegion = TM * kRowBytes;  // one wave's staging bytes
        static_assert(NW * kRegion <= STAGES * kStage, "epilogue staging fits the stage buffers");
        barrier();  // every wave is done with the operand buffers
        uint8_t* wl = smem + wave * kRegion;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cl = 32 * j + 8 * q + 4 * (lane >> 5);  // column in the wave tile
                const int64_t gn = n0 + wn * TN + cl;
                float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (bias_p && gn < p.n) {
                    const uint2 bb = *reinterpret_cast<const uint2*>(bias_p + gn);
                    bias[0] = bf16_lo(bb.x); bias[1] = bf16_hi(bb.x);
                    bias[2] = bf16_lo(bb.y); bias[3] = bf16_hi(bb.y);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = 32 * i + (lane & 31);
                    const int chunk = (cl >> 3) ^ (r % kChunks);
                    v2i pk;
                    pk[0] = (int)f32x2_to_bf16x2(fmaf(acc[i][j][4 * q + 0], sc, bias[0]),
                                                 fmaf(acc[i][j][4 * q + 1], sc, bias[1]));
                    pk[1] = (int)f32x2_to_bf16x2(fmaf(acc[i][j][4 * q + 2], sc, bias[2]),
                                                 fmaf(acc[i][j][4 * q + 3], sc, bias[3]));
                    *reinterpret_cast<__attribute__((address_space(3))) v2i*>(
                        (lds_void*)(wl + r * kRowBytes + chunk * 16 + 8 * (lane >> 5))) = pk;
                }
            }
        }
        const int cc = lane % kChunks;  // this lane's 16-byte chunk of a row
        const int64_t gn = n0 + wn * TN + 8 * cc;
#pragma unroll
        for (int ps = 0; ps < TM / kRowsPerPass; ++ps) {
            const int r = ps * kRowsPerPass + lane / kChunks;
            const v4i v = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(
                (lds_void*)(wl + r * kRowBytes + ((cc ^ (r % kChunks)) << 4)));
            const int64_t gm = m0 + wm * TM + r;
            if (gm < p.m && gn < p.n) *reinterpret_cast<v4i*>(out + gm * p.n + gn) = v;
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t gn = n0 + wn * TN + 32 * j + 8 * q + 4 * (lane >> 5);
            float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (bias_p) {
                if (p.vec_out && gn + 3 < p.n) {
                    const uint2 bb = *reinterpret_cast<const uint2*>(bias_p + gn);
                    bias[0] = bf16_lo(bb.x); bias[1] = bf16_hi(bb.x);
                    bias[2] = bf16_lo(bb.y); bias[3] = bf16_hi(bb.y);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (gn + c < p.n) bias[c] = bf16_to_f32(bias_p[gn + c]);
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int64_t gm = m0 + wm * TM + 32 * i + (lane & 31);
                if (gm >= p.m) continue;
                const uint32_t w0 = f32x2_to_bf16x2(fmaf(acc[i][j][4 * q + 0], sc, bias[0]),
                                                    fmaf(acc[i][j][4 * q + 1], sc, bias[1]));
                const uint32_t w1 = f32x2_to_bf16x2(fmaf(acc[i][j][4 * q + 2], sc, bias[2]),
                                                    fmaf(acc[i][j][4 * q + 3], sc, bias[3]));
                uint16_t* dst = out + gm * p.n + gn;
                if (p.vec_out && gn + 3 < p.n) {
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
    }
}

// FOLD: the grid's last workgroup runs a held-back ring fold instead of a
// tile.  Only the plain NT kernels that the linear forward launches are
// built with it; every other kernel is the same code with or without the
// job argument (a branch ahead of the tile code costs the 256 x 256 tiles a
// register at their limit).
template <int FMT, bool AMN, bool BMN, int BM, int BN, int WM, int WN, int BK, int STAGES,
          bool EXT, bool FOLD>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_tiled_kernel(TiledParams p, FoldJob fold) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[tiled_lds_bytes<BM, BN, BK, STAGES>()];
    if constexpr (FOLD) {
        // (this form of the test keeps the 256 x 256 tiles free of spills)
        const int tiles = (int)gridDim.x - 1;
        if ((int)blockIdx.x == tiles) {  // the last workgroup, dispatched after
            fold_waves(fold);            // every tile: the held-back fold(s)
            return;
        }
        gemm_tile<FMT, AMN, BMN, BM, BN, WM, WN, BK, STAGES, EXT>(p, blockIdx.x, tiles, smem);
    } else {
        gemm_tile<FMT, AMN, BMN, BM, BN, WM, WN, BK, STAGES, EXT>(p, blockIdx.x, gridDim.x, smem);
    }
}

// Two independent problems in one launch (the linear backward's dX, NN, and
// dW, TN), both on one tile configuration: workgroups [0, n0) take problem
// 0's tiles and the rest problem 1's.  One workgroup fits a CU, so problem
// 1's tiles start on CUs as problem 0's finish: their prologue loads overlap
// problem 0's output stores, and there is one launch boundary instead of
// two.  When problem 0's tiles are the longer ones (dX walks the layer's N,
// dW its M), the CUs that finish a short tile early take the next one, so
// the two problems balance over the machine.  Workgroups past n0 + n1 run
// the bias gradient's last pass (`cf`, a quarter of the workgroup's lanes in
// columns each): the highest ids are dispatched last, so they take CUs as
// the first tiles finish, in place of a launch of their own.  A held-back
// ring fold (`fold`) takes one more workgroup, id fold_at, ahead of the
// tiles and workgroups after it.  Stream order makes the partials and the
// group lines (written by earlier launches) visible to them.
// A tile configuration as a type: BM x BN tile, WM x WN waves, BK k per
// stage, ST stages.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int ST_>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, ST = ST_;
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int kLds = tiled_lds_bytes<BM, BN, BK, ST>();
};
using ShapeBig = TileShape<256, 256, 2, 4, 128, 2>;
using ShapeWide = TileShape<128, 256, 2, 4, 128, 3>;
using ShapeTall = TileShape<256, 128, 4, 2, 128, 3>;
using ShapeMid = TileShape<128, 128, 4, 2, 128, 4>;
using ShapeMidNN = TileShape<128, 128, 2, 4, 128, 4>;  // the NN problem (dX) on 128 x 128

template <int FMT, class S0, class S1>
__global__ __launch_bounds__(S0::kThreads, 1) void gemm_tiled_pair_kernel(TiledParams p0,
                                                                          TiledParams p1, int n0,
                                                                          int n1,
                                                                          ColsumFinalJob cf,
                                                                          FoldJob fold,
                                                                          int fold_at) {
    static_assert(S0::kThreads == S1::kThreads, "one workgroup size");
    constexpr int T = S0::kThreads;
    constexpr int kLds = S0::kLds > S1::kLds ? S0::kLds : S1::kLds;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
    static_assert(kLds >= T * 4, "column-sum scratch fits");
    if (fold.n > 0 && (int)blockIdx.x == fold_at) {
        fold_waves(fold);
        return;
    }
    const int b = (int)blockIdx.x - (fold.n > 0 && (int)blockIdx.x > fold_at ? 1 : 0);
    if (b < n0)
        gemm_tile<FMT, false, true, S0::BM, S0::BN, S0::WM, S0::WN, S0::BK, S0::ST>(p0, b, n0,
                                                                                  smem);
    else if (b < n0 + n1)
        gemm_tile<FMT, true, true, S1::BM, S1::BN, S1::WM, S1::WN, S1::BK, S1::ST>(p1, b - n0,
                                                                                 n1, smem);
    else
        colsum_final_cols<T>(cf.part, cf.chunks, cf.n, (int64_t)(b - n0 - n1) * (T / 4), cf.db,
                             reinterpret_cast<float*>(smem));
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
    // 32-bit buffer offsets within one batch slice
    const double lim = 2147483647.0;
    if ((double)(a_mn ? g.k : g.m) * (double)g.lda >= lim) return false;
    if ((double)(b_mn ? g.k : g.n) * (double)g.ldb >= lim) return false;
    // 32-bit tile ids (64 x 64 is the smallest tile)
    if ((double)((g.m + 63) / 64) * (double)((g.n + 63) / 64) * (double)g.batch >= lim) return false;
    return true;
}

template <int BM, int BN>
static TiledParams tiled_params(const GemmLaunch& g) {
    TiledParams p{};
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
    p.tiles_m = (int)((g.m + BM - 1) / BM);
    p.tiles_n = (int)((g.n + BN - 1) / BN);
    p.tiles_per_batch = p.tiles_m * p.tiles_n;
    p.group_m = 4;
    const uintptr_t ob = reinterpret_cast<uintptr_t>(g.out), bb = reinterpret_cast<uintptr_t>(g.bias);
    if (!g.ext()) {
        const bool bias8 = g.bias == nullptr || (bb & 7) == 0;
        p.vec_out = ((ob & 7) == 0) && (g.n % 4 == 0) && bias8;
        p.vec_out16 = ((ob & 15) == 0) && (g.n % 8 == 0) && bias8;
        p.vec_bias = bias8;
    } else {
        const int osz = g.out_q < 0 ? 2 : 1;  // output bytes per element
        p.vec_out = ((ob & (4 * osz - 1)) == 0) && (g.n % 4 == 0);
        p.vec_out16 = ((ob & 15) == 0) && ((g.n * osz) % 16 == 0);
        p.vec_bias = g.bias == nullptr || (bb & (g.bias_scale ? 3 : 7)) == 0;
    }
    const int64_t total = p.tiles_per_batch * g.batch;
    p.xcd_remap = (total % 8) == 0;
    return p;
}

template <int FMT, bool AMN, bool BMN, int BM, int BN, int WM, int WN, int BK, int ST>
static hipError_t launch_cfg(const GemmLaunch& g, hipStream_t stream, const FoldJob& fold) {
    const TiledParams p = tiled_params<BM, BN>(g);
    const int64_t total = (int64_t)p.tiles_per_batch * g.batch;
    const dim3 block(WM * WN * 64);
    if constexpr (!AMN && !BMN) {  // NT: the linear forward's GEMM may carry a fold
        if (fold.n > 0) {
            if (g.ext()) return hipErrorInvalidValue;  // callers check gemm_tiled_carries_fold
            hipLaunchKernelGGL((gemm_tiled_kernel<FMT, AMN, BMN, BM, BN, WM, WN, BK, ST, false, true>),
                               dim3((unsigned)(total + 1)), block, 0, stream, p, fold);
            return hipGetLastError();
        }
    } else {
        if (fold.n > 0) return hipErrorInvalidValue;
    }
    if (g.ext())
        hipLaunchKernelGGL((gemm_tiled_kernel<FMT, AMN, BMN, BM, BN, WM, WN, BK, ST, true, false>),
                           dim3((unsigned)total), block, 0, stream, p, fold);
    else
        hipLaunchKernelGGL((gemm_tiled_kernel<FMT, AMN, BMN, BM, BN, WM, WN, BK, ST, false, false>),
                           dim3((unsigned)total), block, 0, stream, p, fold);
    return hipGetLastError();
}

bool gemm_tiled_carries_fold(const GemmLaunch& g) {
    return gemm_tiled_supported(g) && g.trans_a == 0 && g.trans_b != 0 && !g.ext();
}

static int64_t tiles_of(const GemmLaunch& g, int bm, int bn) {
    return ((g.m + bm - 1) / bm) * ((g.n + bn - 1) / bn) * g.batch;
}

// Tile configuration by output-tile count.  Every configuration runs one
// workgroup per CU (its LDS ring takes most of the 160 KB), so the tiles go
// in rounds of 256 (one per CU), each round as long as one tile: the
// launch costs rounds x tile time.  A larger tile reads fewer operand bytes
// per flop, but fewer of them leave CUs idle or a last round nearly empty.
// The configurations, with the tile time in units of a 256 x 256 tile's
// (per-unit-area cost measured on MI355X over k = 272 .. 4112, graph
// bursts, every configuration forced in turn on the same operands):
//   kBig    256 x 256, 8 waves of 128 x 64                   1000
//   kWide   128 x 256, 8 waves of  64 x 64   (1.35 per area)  675
//   kTall   256 x 128, 8 waves of  64 x 64   (1.35 per area)  675
//   kMid    128 x 128, 8 waves of  32 x 64   (1.9 per area)   475  (NN: 64 x 32)
//   kSmall   64 x  64, 4 waves of  32 x 32   m <= 64 below 256 tiles of 128 x 128
// The cheapest wins; ties go to the larger tile, and between 128 x 256 and
// 256 x 128 to the one whose long side lies along the longer output side.
// Measured (us): 2048 x 4096 x 1024 NT 13.9 wide (big 18.0, mid 15.1);
// 2048 x 1024 x 4096 NN 16.4 mid (wide 25.7); 4096 x 1024 x 2048 TN 12.3 mid
// (wide 15.8); 4112 x 1040 x 2064 TN 18.8 wide against 25.6 for 297 mid
// tiles in two rounds; 3000 x 3000 x 2048 NT 28.6 big (144 tiles, one
// round) against 31.2 wide (288 tiles, two rounds); 4096^3 57 big (wide
// 69, mid 77).  For NN, B is n-contiguous and goes through the transposing
// LDS read (about 180 B/clk per CU against 250 for ds_read_b128), so kMid
// arranges its waves 2 x 4 there: each B fragment is read by two waves
// instead of four (per 64-k substep 16 KB of transposing reads and 32 KB of
// plain ones, instead of 32 and 16); 2048 x 1024 x 4096 NN 16.37 against
// 16.50, 1024 x 1024 x 8192 NN 27.5 against 27.9, the training step's
// paired dX + dW 19.54 against 19.74.  All configurations sum every
// output's k range in the same order, so the choice never changes a result
// bit.
enum TileCfg { kBig, kWide, kTall, kMid, kSmall };

static TileCfg tile_cfg(const GemmLaunch& g) {
    if (g.m <= 64 && tiles_of(g, 128, 128) < 256) return kSmall;
    struct Opt {
        TileCfg c;
        int bm, bn;
        int64_t w;  // tile time, 1/1000 of a 256 x 256 tile's
    };
    const Opt wide{kWide, 128, 256, 675}, tall{kTall, 256, 128, 675};
    const Opt order[4] = {{kBig, 256, 256, 1000}, g.n >= g.m ? wide : tall,
                          g.n >= g.m ? tall : wide, {kMid, 128, 128, 475}};
    TileCfg best = kBig;
    int64_t best_cost = -1;
    for (const Opt& o : order) {
        const int64_t cost = (tiles_of(g, o.bm, o.bn) + 255) / 256 * o.w;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = o.c;
        }
    }
    return best;
}

template <int FMT, bool AMN, bool BMN>
static hipError_t launch_layout(const GemmLaunch& g, hipStream_t stream, const FoldJob& fold) {
    // 256 x 256 tiles take 128-k stages, double-buffered, in every layout:
    // a k-contiguous row segment is then a whole 128-byte line, and for NN /
    // TN they measured as fast as four 64-k stages refilled in pairs alone
    // (54.5 / 53.0 against 54.6 / 53.5 us at 4096^3) and 2.5 us faster in
    // the backward pair (103.4 against 106.1 us).  The 64-k stage code
    // (kSubs == 1, refills in pairs) is kept for configurations that want a
    // deeper ring of smaller stages; none of the shipped ones does.
    switch (tile_cfg(g)) {
        case kBig: return launch_cfg<FMT, AMN, BMN, 256, 256, 2, 4, 128, 2>(g, stream, fold);
        case kWide: return launch_cfg<FMT, AMN, BMN, 128, 256, 2, 4, 128, 3>(g, stream, fold);
        case kTall: return launch_cfg<FMT, AMN, BMN, 256, 128, 4, 2, 128, 3>(g, stream, fold);
        case kMid:
            if constexpr (!AMN && BMN) return launch_cfg<FMT, AMN, BMN, 128, 128, 2, 4, 128, 4>(g, stream, fold);
            else return launch_cfg<FMT, AMN, BMN, 128, 128, 4, 2, 128, 4>(g, stream, fold);
        case kSmall: break;
    }
    return launch_cfg<FMT, AMN, BMN, 64, 64, 2, 2, 128, 4>(g, stream, fold);
}

template <int FMT>
static hipError_t launch_fmt(const GemmLaunch& g, hipStream_t stream, const FoldJob& fold) {
    const bool a_mn = g.trans_a != 0, b_mn = g.trans_b == 0;
    if (!a_mn && !b_mn) return launch_layout<FMT, false, false>(g, stream, fold);
    if (!a_mn && b_mn) return launch_layout<FMT, false, true>(g, stream, fold);
    if (a_mn && !b_mn) return launch_layout<FMT, true, false>(g, stream, fold);
    return launch_layout<FMT, true, true>(g, stream, fold);
}

hipError_t launch_gemm_tiled(const GemmLaunch& g, hipStream_t stream, const FoldJob& fold) {
    return g.fmt == 0 ? launch_fmt<0>(g, stream, fold) : launch_fmt<1>(g, stream, fold);
}

// Paired configurations.  Both problems on 256 x 256 tiles when each fills
// the CUs with them.  Otherwise the tiles are sized so that one tile of
// either problem is about the same work: the problem with the longer k
// (the backward's dX walks the layer's N, dW its M) takes 128 x 128 tiles
// and the other, when its k is a third to two thirds of that, tiles twice
// that area (256 x 128 when its m >= n, else 128 x 256); and the two must
// give at least one tile per CU.  Then the CUs finish together instead of
// some taking two short tiles while others run one long tile (training
// step at 2048 x 4096 x 1024: dX 2048 x 1024 x 4096 + dW 4096 x 1024 x 2048).
struct PairCfg {
    TileCfg c0 = kSmall, c1 = kSmall;  // kSmall: no paired launch
};

static int cfg_bm(TileCfg c) { return c == kBig || c == kTall ? 256 : 128; }
static int cfg_bn(TileCfg c) { return c == kBig || c == kWide ? 256 : 128; }

static PairCfg pair_cfg(const GemmLaunch& g0, const GemmLaunch& g1) {
    PairCfg r;
    if (tiles_of(g0, 256, 256) >= 256 && tiles_of(g1, 256, 256) >= 256) {
        r.c0 = r.c1 = kBig;
        return r;
    }
    auto larger = [](const GemmLaunch& g) { return g.m >= g.n ? kTall : kWide; };
    r.c0 = r.c1 = kMid;
    if (2 * g1.k <= g0.k * 4 / 3 && 2 * g1.k >= g0.k * 2 / 3) r.c1 = larger(g1);  // k1 ~ k0/2
    else if (2 * g0.k <= g1.k * 4 / 3 && 2 * g0.k >= g1.k * 2 / 3) r.c0 = larger(g0);
    if (tiles_of(g0, cfg_bm(r.c0), cfg_bn(r.c0)) + tiles_of(g1, cfg_bm(r.c1), cfg_bn(r.c1)) < 256)
        r.c0 = r.c1 = kSmall;
    return r;
}

static int64_t pair_tiles(const GemmLaunch& g0, const GemmLaunch& g1, const PairCfg& c) {
    return tiles_of(g0, cfg_bm(c.c0), cfg_bn(c.c0)) + tiles_of(g1, cfg_bm(c.c1), cfg_bn(c.c1));
}

bool gemm_tiled_pair_supported(const GemmLaunch& g0, const GemmLaunch& g1) {
    if (!gemm_tiled_supported(g0) || !gemm_tiled_supported(g1) || g0.fmt != g1.fmt) return false;
    if (g0.ext() || g1.ext()) return false;  // the paired kernel has the plain epilogue
    // problem 0 NN (A k-contiguous, B n-contiguous), problem 1 TN (both
    // m/n-contiguous)
    if (g0.trans_a != 0 || g0.trans_b != 0 || g1.trans_a != 1 || g1.trans_b != 0) return false;
    const PairCfg c = pair_cfg(g0, g1);
    if (c.c0 == kSmall) return false;
    return (double)pair_tiles(g0, g1, c) < 2147483647.0;
}

bool gemm_tiled_pair_carries(const GemmLaunch& g0, const GemmLaunch& g1,
                             const ColsumFinalJob& cf) {
    const int64_t extra = (cf.n + 127) / 128;
    return cf.db && cf.n >= 1 &&
           (double)pair_tiles(g0, g1, pair_cfg(g0, g1)) + (double)extra < 2147483647.0;
}

template <class S0, class S1>
static hipError_t launch_pair_cfg(const GemmLaunch& g0, const GemmLaunch& g1,
                                  hipStream_t stream, const ColsumFinalJob* cf,
                                  const FoldJob& fold) {
    TiledParams p0 = tiled_params<S0::BM, S0::BN>(g0);
    TiledParams p1 = tiled_params<S1::BM, S1::BN>(g1);
    const int n0 = (int)tiles_of(g0, S0::BM, S0::BN), n1 = (int)tiles_of(g1, S1::BM, S1::BN);
    // problem 1's local ids line up with the XCDs only if n0 is a multiple of 8
    p1.xcd_remap = p1.xcd_remap && (n0 % 8) == 0;
    ColsumFinalJob job;
    int extra = 0;
    constexpr int kCols = S0::kThreads / 4;  // bias-gradient columns per extra workgroup
    if (cf && cf->db) {  // callers check gemm_tiled_pair_carries first
        job = *cf;
        extra = (int)((cf->n + kCols - 1) / kCols);
    }
    // A held-back fold goes to the first CU that frees up: right after
    // problem 0's tiles when those alone fill the 256 CUs (the CU that
    // folds then takes one of problem 1's tiles a moment later, while others
    // still run problem 0), else right after all the tiles.
    const int fold_at = n0 >= 256 ? n0 : n0 + n1;
    const dim3 grid((unsigned)(n0 + n1 + extra + (fold.n > 0 ? 1 : 0)));
    const dim3 block(S0::kThreads);
    if (g0.fmt == 0)
        hipLaunchKernelGGL((gemm_tiled_pair_kernel<0, S0, S1>), grid, block, 0, stream, p0, p1, n0,
                           n1, job, fold, fold_at);
    else
        hipLaunchKernelGGL((gemm_tiled_pair_kernel<1, S0, S1>), grid, block, 0, stream, p0, p1, n0,
                           n1, job, fold, fold_at);
    return hipGetLastError();
}

hipError_t launch_gemm_tiled_pair(const GemmLaunch& g0, const GemmLaunch& g1,
                                  hipStream_t stream, const ColsumFinalJob* cf,
                                  const FoldJob& fold) {
    const PairCfg c = pair_cfg(g0, g1);
    if (c.c0 == kBig) return launch_pair_cfg<ShapeBig, ShapeBig>(g0, g1, stream, cf, fold);
    if (c.c0 == kMid && c.c1 == kTall) return launch_pair_cfg<ShapeMidNN, ShapeTall>(g0, g1, stream, cf, fold);
    if (c.c0 == kMid && c.c1 == kWide) return launch_pair_cfg<ShapeMidNN, ShapeWide>(g0, g1, stream, cf, fold);
    if (c.c0 == kTall) return launch_pair_cfg<ShapeTall, ShapeMid>(g0, g1, stream, cf, fold);
    if (c.c0 == kWide) return launch_pair_cfg<ShapeWide, ShapeMid>(g0, g1, stream, cf, fold);
    return launch_pair_cfg<ShapeMidNN, ShapeMid>(g0, g1, stream, cf, fold);
}

}  // namespace fp8lin
