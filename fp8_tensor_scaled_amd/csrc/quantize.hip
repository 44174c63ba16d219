// bf16 -> fp8 quantize with fused amax and the delayed-scaling ring fold,
// the standalone ring finalize, and the bias-gradient column sum.
//
// Method (AstrAI compare view 3e57cc8...main, csrc/kernels/fp8/quantize.cuh:
// fp8_quantize_kernel and publish_amax; astrai/extension/fp8.py:
// FP8Recipe.scale_from_history and _ScaleRing): each element is multiplied
// by the reciprocal of the step and converted with round-to-nearest-even and
// saturation; the running max of |x| is taken over the raw inputs; every
// workgroup contributes its max through atomics, and the workgroup that
// finishes last records the amax in the history slot, publishes the next
// step from the window's max and re-arms its scratch slots, so the delayed
// update costs no extra launch.
//
// gfx950 design:
//  * HBM streaming (quantize_kernel, quantize_two_kernel): workgroups of 256
//    data lanes and one publisher wave, two per CU (at most 512), sweeping
//    the tensor in rounds: in a
//    round the grid's lanes take consecutive 16-element chunks, each lane
//    keeping four chunks (four 32-byte loads) in flight and storing 16 codes
//    per chunk with one 16-byte store.  From 2^25 elements, one chunk per
//    lane per round and up to 1024 workgroups (four per CU).  An input read once is loaded
//    non-temporally, so it neither displaces lines the next kernel reads
//    nor, when cold, loses anything; the library's measure-then-cast
//    sequences and fp32 inputs use ordinary loads.  The codes' stores are
//    ordinary (they feed the GEMM that follows).  Conversions are
//    v_cvt_pk_{fp8,bf8}_f32 after a med3 clamp to +-max (satfinite).
//  * The fold's cost is its atomics: same-address atomics serialize at the
//    coherence point (about 11 ns each, measured), and a returning atomic
//    waits for every store its wave issued before it.  So the maxima meet
//    in two levels (16 groups, then the ring's words), each workgroup
//    publishes in its last round after the loads and before the stores, from
//    a wave with no stores of its own (the publisher; in the 1024-lane
//    kernels, wave 0), and the window is read at kernel start so the last
//    workgroup does not wait for it.  The single-lane
//    atomics are kept as written (the build turns off the compiler's atomic
//    optimizer, whose wave-wide form would wait for the result at once).
//  * The fused column-sum, transposed and small-tensor kernels keep
//    1024-lane workgroups (one per CU).
//  * The fold uses relaxed agent-scope atomics only.  Release/acquire at
//    agent scope write back / invalidate the per-XCD L2s and cost tens of ns
//    per workgroup when every workgroup issues them; instead each level
//    takes its counter only after its max has returned (the returned value
//    feeds the increment), so by the time a counter completes every max it
//    covers has been performed at the device coherence point, where the
//    following atomic reads see it.  The fp8 outputs need no ordering
//    against the fold (kernel boundaries publish them).

#include "common.hpp"
#include "internal.hpp"

namespace fp8lin {

constexpr int kQuantThreads = 1024;  // fused / transposed / small-tensor kernels
constexpr int kQuantWaves = kQuantThreads / kWave;
constexpr int kVecElems = 16;  // bf16 elements per lane per unrolled slot
constexpr int kUnroll = 4;     // slots in flight per lane
// The streaming quantize: workgroups of 256 lanes, two per CU.
constexpr int kQT = 256;
constexpr int kQGridMax = 512;
// From 2^25 elements: one slot per lane per round and up to 1024
// workgroups (four per CU), the shape the bare 2:1 stream runs fastest in
// there (8192^2 with fold 41.0 against 44.1 us; below it the narrower,
// deeper shape wins: 4096^2 13.9 against 14.0, 2048 x 4096 9.6 against 9.8).
constexpr int kUnrollLarge = 1;
constexpr int kQGridMaxLarge = 1024;
constexpr int64_t kLargeNumel = int64_t(1) << 25;

struct QuantParams {
    const void* x;        // elements of the kernel's input type
    int64_t numel;
    const float* scale;
    uint8_t* out;
    uint8_t* out2;        // second format's codes (dual quantize), or null
    float* hist;          // ring window (null: no fold)
    float* scale_out;     // ring scale slot
    uint32_t* amax_slot;  // ring scratch: running amax bits
    uint32_t* done;       // ring scratch: finished-workgroup counter
    uint32_t* groups;     // ring scratch: kRingGroups x (max, counter) lines
    int32_t len;
    int32_t idx;
    float fmax;
    float pow2_margin;
    float* scale_used;
    float* amax_out;  // optional max |x| output: written by the fold, or (no
                      // ring) an atomic max over workgroups after an arming launch
    int vec;    // 1: x and out are 16-byte aligned
    int nt;     // 1: non-temporal input loads (vector path, 2-byte inputs)
    int defer;  // 1: with a ring, only the group lines' maxima (held-back fold)
};

// Last-workgroup fold (one wave): hist[idx] = amax;
// scale = max(peak / fmax / 2^margin, 1e-12).  `win` = this lane's share of
// the window's other slots, loaded at kernel start (only the fold writes the
// window, and the previous launch's fold finished before this kernel began).
__device__ __forceinline__ void fold_ring(const QuantParams& p, float s_read, float win) {
    const int lane = threadIdx.x % kWave;
    float amax = 0.0f;
    if (lane == 0)
        amax = __uint_as_float(
            __hip_atomic_load(p.amax_slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    amax = __shfl(amax, 0, kWave);
    float w = win;
    for (int i = lane + kWave; i < p.len; i += kWave)  // windows longer than a wave
        if (i != p.idx) w = fmaxf(w, p.hist[i]);
    const float peak = fmaxf(wave_max(w), amax);
    if (lane == 0) {
        p.hist[p.idx] = amax;
        if (p.amax_out) *p.amax_out = amax;
        const float t = __fdiv_rn(peak, p.fmax);
        const float s = __fdiv_rn(t, p.pow2_margin);
        *p.scale_out = fmaxf(s, 1e-12f);
        if (p.scale_used) *p.scale_used = s_read;
        __hip_atomic_store(p.amax_slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Workgroup max of v, published by thread PUB in two levels: workgroup b is
// in group b % G (G = min(workgroups, kRingGroups)); it takes the group's
// atomic max and then, once that has been performed (the increment depends
// on the returned value), the group's counter.  The group's last workgroup
// reads the group max, re-arms the group's line, and does the same on the
// ring's amax / done words.  Same-address atomics serialize (about 11 ns
// each, measured), so 16 x 16 contenders cost far less than 256 on one
// word.  Returns, at thread PUB, nblocks - 1 if this workgroup drew the last
// top-level ticket (it folds), else ~0u.  The whole chain runs before the
// caller's last stores, which go out while it is in flight.  With p.defer
// (a held-back fold) the workgroup only takes the max into line b % 16 and
// returns ~0u: nothing waits on it.  Every thread of the workgroup must
// call it once.
template <int T = kQuantThreads, int PUB = 0>
__device__ __forceinline__ uint32_t publish_amax(const QuantParams& p, float v, uint32_t nblocks,
                                                 uint32_t b) {
    constexpr int kW = T / kWave;
    __shared__ float slots[kW];
    v = wave_max(v);
    if ((threadIdx.x % kWave) == 0) slots[threadIdx.x / kWave] = v;
    __syncthreads();
    uint32_t ticket = ~0u;
    if (threadIdx.x == PUB) {
        v = slots[0];
#pragma unroll
        for (int w = 1; w < kW; ++w) v = fmaxf(v, slots[w]);
        if (p.defer) {
            __hip_atomic_fetch_max(p.groups + kRingGroupWords * (b % kRingGroups),
                                   __float_as_uint(v), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            return ticket;
        }
        const uint32_t ng = nblocks < kRingGroups ? nblocks : kRingGroups;
        const uint32_t g = b % ng;
        const uint32_t members = (nblocks - g + ng - 1) / ng;
        uint32_t* line = p.groups + kRingGroupWords * g;
        // |x| maxima are never all-ones bits; the comparisons make each
        // increment wait for the max before it to have been performed.
        const uint32_t old = __hip_atomic_fetch_max(line, __float_as_uint(v), __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t gt = __hip_atomic_fetch_add(line + 1, old == ~0u ? 2u : 1u,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (gt == members - 1) {
            const uint32_t gm = __hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(line + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t o2 = __hip_atomic_fetch_max(p.amax_slot, gm, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t t = __hip_atomic_fetch_add(p.done, o2 == ~0u ? 2u : 1u,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (t == ng - 1) ticket = nblocks - 1;
        }
    }
    return ticket;
}

// Without a ring: the workgroup max goes into *amax_out (armed to +0 by the
// launch before) by one atomic max; non-negative floats order as their bits.
// Every thread of the workgroup must call it once.
template <int T, int PUB = 0>
__device__ __forceinline__ void publish_amax_out(const QuantParams& p, float v) {
    constexpr int kW = T / kWave;
    __shared__ float slots[kW];
    v = wave_max(v);
    if ((threadIdx.x % kWave) == 0) slots[threadIdx.x / kWave] = v;
    __syncthreads();
    if (threadIdx.x == PUB) {
        v = slots[0];
#pragma unroll
        for (int w = 1; w < kW; ++w) v = fmaxf(v, slots[w]);
        __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(p.amax_out), __float_as_uint(v),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void arm_amax_kernel(float* amax_out) { *amax_out = 0.0f; }

// The workgroup that drew the last ticket folds, on the wave of thread PUB.
template <int PUB = 0>
__device__ __forceinline__ void finish_fold(const QuantParams& p, uint32_t ticket, float s_read,
                                            float win, uint32_t nblocks) {
    if (threadIdx.x / kWave != PUB / kWave) return;
    const int last = threadIdx.x == PUB && ticket == nblocks - 1u;
    if (__shfl(last, 0, kWave)) fold_ring(p, s_read, win);
}

// Input element types.  A 16-element chunk is kLoads 16-byte loads; unpack
// widens it to fp32 exactly ([CMP] quantize.cuh quant_in_traits: bf16,
// fp16 and fp32 inputs), `one` reads a single element.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int IN>
struct In;
template <>
struct In<kInBf16> {
    static constexpr int kLoads = 2;
    __device__ static float one(const void* x, int64_t e) {
        return bf16_to_f32(static_cast<const uint16_t*>(x)[e]);
    }
    __device__ static void unpack(const uint4* r, float f[16]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[8 * i + 2 * j] = bf16_lo(w[j]);
                f[8 * i + 2 * j + 1] = bf16_hi(w[j]);
            }
        }
    }
};
template <>
struct In<kInF16> {
    static constexpr int kLoads = 2;
    __device__ static float one(const void* x, int64_t e) {
        return (float)static_cast<const _Float16*>(x)[e];
    }
    __device__ static void unpack(const uint4* r, float f[16]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x2_t v = __builtin_convertvector(__builtin_bit_cast(f16x2_t, w[j]),
                                                          f32x2_t);
                f[8 * i + 2 * j] = v[0];
                f[8 * i + 2 * j + 1] = v[1];
            }
        }
    }
};
template <>
struct In<kInF32> {
    static constexpr int kLoads = 4;
    __device__ static float one(const void* x, int64_t e) {
        return static_cast<const float*>(x)[e];
    }
    __device__ static void unpack(const uint4* r, float f[16]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[4 * i] = __uint_as_float(r[i].x);
            f[4 * i + 1] = __uint_as_float(r[i].y);
            f[4 * i + 2] = __uint_as_float(r[i].z);
            f[4 * i + 3] = __uint_as_float(r[i].w);
        }
    }
};

template <int IN>
__device__ __forceinline__ float absmax16(const uint4* r, float amax) {
    float f[16];
    In<IN>::unpack(r, f);
#pragma unroll
    for (int j = 0; j < 16; j += 2) amax = fmaxf(amax, fmaxf(fabsf(f[j]), fabsf(f[j + 1])));
    return amax;
}

// 16 codes of x * m into dst; FMT2 >= 0: the same scaled values in the
// second format into dst2 (one read of x feeds both encodings).
template <int IN, int FMT, int FMT2>
__device__ __forceinline__ void encode16(const uint4* r, float m, uint4* dst, uint4* dst2) {
    float f[16];
    In<IN>::unpack(r, f);
#pragma unroll
    for (int j = 0; j < 16; ++j) f[j] *= m;
    uint4 o;
    o.x = cvt4<FMT>(f[0], f[1], f[2], f[3]);
    o.y = cvt4<FMT>(f[4], f[5], f[6], f[7]);
    o.z = cvt4<FMT>(f[8], f[9], f[10], f[11]);
    o.w = cvt4<FMT>(f[12], f[13], f[14], f[15]);
    *dst = o;
    if constexpr (FMT2 >= 0) {
        uint4 o2;
        o2.x = cvt4<FMT2>(f[0], f[1], f[2], f[3]);
        o2.y = cvt4<FMT2>(f[4], f[5], f[6], f[7]);
        o2.z = cvt4<FMT2>(f[8], f[9], f[10], f[11]);
        o2.w = cvt4<FMT2>(f[12], f[13], f[14], f[15]);
        *dst2 = o2;
    }
}

// A workgroup is kQT data lanes plus one publisher wave.  Vector path (x,
// out, out2 16-byte aligned): the grid sweeps the 16-element chunks in
// rounds; in round rd, slot u, workgroup b's lanes take the kQT consecutive
// chunks ((rd * U + u) * nb + b) * kQT + lane, so at any time the
// whole grid streams one narrow window of the tensor (measured faster than a
// contiguous range per workgroup: 37 against 40.6 us for the bare read-2 /
// write-1 stream at 8192 x 8192).  A round's loads all go out before any of
// its data is used (round 0's before the step's reciprocal is taken, so the
// wait for the step overlaps them), and the non-temporal choice is made
// once, outside the loop, so the waits count the loads one by one.  The
// numel % 16 leftover elements go to workgroup 0.  With a ring, the data
// waves hand their max to the publisher wave at one barrier in their last
// round, before their stores; the publisher runs the fold's atomics while
// the data waves store (a data wave that ran them would hold its own stores
// back for the whole chain: 1 us more per launch, measured at every size).
// Scalar path (unaligned bases): grid-stride elements, then the publish.
// Workgroup b of the nb that process p (the whole grid, or one tensor's
// share of a two-tensor launch).
template <int IN, int FMT, int FMT2, bool MEASURE_ONLY, int U = kUnroll>
__device__ __forceinline__ void quantize_body(const QuantParams& p, const uint32_t b,
                                              const uint32_t nb) {
    constexpr int kL = In<IN>::kLoads;
    float m = 0.0f, s_read = 0.0f;
    if constexpr (!MEASURE_ONLY) s_read = *p.scale;
    const int t = threadIdx.x;
    if (t >= kQT) {
        // The publisher wave: no data of its own; it takes the workgroup's
        // max at the publish barrier and runs the atomics (and the fold), so
        // that no data wave waits for them before its stores.
        if (p.hist) {
            const int wl = t - kQT;
            const float win = (!p.defer && wl < p.len && wl != p.idx) ? p.hist[wl] : 0.0f;
            const uint32_t tk = publish_amax<kQT + kWave, kQT>(p, 0.0f, nb, b);
            finish_fold<kQT>(p, tk, s_read, win, nb);  // no ticket when deferred
        } else if (p.amax_out) {
            publish_amax_out<kQT + kWave, kQT>(p, 0.0f);
        }
        return;
    }
    float amax = 0.0f;
    if (p.vec) {
        const int64_t nvec = p.numel / kVecElems;
        // the numel % 16 leftover elements (workgroup 0)
        auto leftover = [&]() __attribute__((always_inline)) {
            if (b != 0) return;
            const int64_t e = nvec * kVecElems + t;
            if (e < p.numel) {
                const float f = In<IN>::one(p.x, e);
                amax = fmaxf(amax, fabsf(f));
                if constexpr (!MEASURE_ONLY) {
                    p.out[e] = cvt1<FMT>(f * m);
                    if constexpr (FMT2 >= 0) p.out2[e] = cvt1<FMT2>(f * m);
                }
            }
        };
        const uint4* xv = reinterpret_cast<const uint4*>(p.x);
        uint4* ov = reinterpret_cast<uint4*>(p.out);
        uint4* ov2 = reinterpret_cast<uint4*>(p.out2);
        const int64_t slot = (int64_t)nb * kQT;   // chunks per slot of a round
        const int64_t round = slot * U;     // chunks per round
        const int64_t nr = (nvec + round - 1) / round;  // uniform
        const int64_t mine = (int64_t)b * kQT + t;
        // An input read once is loaded non-temporally (p.nt): it then skips
        // the MALL, neither displacing lines the next kernel reads nor, when
        // cold, losing anything.  An input that a measure pass just read is
        // cached, and fp32 inputs measured slower with the hint: ordinary
        // loads.  Loads are unconditional (a chunk past the end re-reads
        // chunk 0 and is ignored).
        auto sweep = [&](auto nt_tag) __attribute__((always_inline)) {
            uint4 r[U][kL];
            auto issue = [&](int64_t rd) __attribute__((always_inline)) {
                const int64_t c0 = rd * round + mine;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t c = c0 + u * slot;
                    const int64_t cl = c < nvec ? c : 0;
#pragma unroll
                    for (int i = 0; i < kL; ++i) {
                        if constexpr (decltype(nt_tag)::value) {
                            const v4i v = __builtin_nontemporal_load(
                                reinterpret_cast<const v4i*>(xv + kL * cl + i));
                            r[u][i] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2],
                                                 (uint32_t)v[3]);
                        } else {
                            r[u][i] = xv[kL * cl + i];
                        }
                    }
                }
                // every load of the round goes out before any of its data is used
                __builtin_amdgcn_sched_barrier(0);
            };
            auto process = [&](int64_t rd) __attribute__((always_inline)) {
                const int64_t c0 = rd * round + mine;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (c0 + u * slot < nvec) amax = absmax16<IN>(r[u], amax);
                if (p.hist && rd == nr - 1) publish_amax<kQT + kWave, kQT>(p, amax, nb, b);
                if constexpr (!MEASURE_ONLY) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int64_t c = c0 + u * slot;
                        if (c < nvec) encode16<IN, FMT, FMT2>(r[u], m, ov + c, ov2 + c);
                    }
                }
            };
            // Round 0's loads go out before the step's reciprocal is taken,
            // so the wait for the step overlaps them.
            issue(0);
            if constexpr (!MEASURE_ONLY) m = __fdiv_rn(1.0f, s_read);
            leftover();
            process(0);
            for (int64_t rd = 1; rd < nr; ++rd) {
                issue(rd);
                process(rd);
            }
        };
        if (nr == 0) {
            if constexpr (!MEASURE_ONLY) m = __fdiv_rn(1.0f, s_read);
            leftover();
            if (p.hist) publish_amax<kQT + kWave, kQT>(p, amax, nb, b);
        } else if (IN != kInF32 && p.nt) {
            sweep(std::true_type{});
        } else {
            sweep(std::false_type{});
        }
    } else {
        if constexpr (!MEASURE_ONLY) m = __fdiv_rn(1.0f, s_read);
        const int64_t stride = (int64_t)nb * kQT;
        for (int64_t e = (int64_t)b * kQT + t; e < p.numel; e += stride) {
            const float f = In<IN>::one(p.x, e);
            amax = fmaxf(amax, fabsf(f));
            if constexpr (!MEASURE_ONLY) {
                p.out[e] = cvt1<FMT>(f * m);
                if constexpr (FMT2 >= 0) p.out2[e] = cvt1<FMT2>(f * m);
            }
        }
        if (p.hist) publish_amax<kQT + kWave, kQT>(p, amax, nb, b);
    }
    if (!p.hist || p.defer) {
        if constexpr (!MEASURE_ONLY) {
            if (p.scale_used && b == 0 && t == 0) *p.scale_used = s_read;
        }
    }
    if (!p.hist && p.amax_out) publish_amax_out<kQT + kWave, kQT>(p, amax);
}

template <int IN, int FMT, int FMT2, bool MEASURE_ONLY, int U>
__global__ __launch_bounds__(kQT + kWave) void quantize_kernel(QuantParams p) {
    quantize_body<IN, FMT, FMT2, MEASURE_ONLY, U>(p, blockIdx.x, gridDim.x);
}

// Two bf16 tensors in one launch (the forward's x and w): workgroups
// [0, nb0) quantize p0, the rest p1, each with its own fold; one launch and
// one latency chain (first loads, fold, last stores) instead of two.  U as
// in quantize_kernel, chosen from the two tensors' total size.
template <int FMT, int FMT2, int U>
__global__ __launch_bounds__(kQT + kWave) void quantize_two_kernel(QuantParams p0,
                                                                     QuantParams p1,
                                                                     uint32_t nb0) {
    if (blockIdx.x < nb0)
        quantize_body<kInBf16, FMT, FMT2, false, U>(p0, blockIdx.x, nb0);
    else
        quantize_body<kInBf16, FMT, FMT2, false, U>(p1, blockIdx.x - nb0, gridDim.x - nb0);
}

static int quant_grid(int64_t numel, int vec, bool large = false) {
    const int64_t per_block = (int64_t)kQT * (vec ? kVecElems : 1);
    int64_t blocks = (numel + per_block - 1) / per_block;
    const int64_t cap = large ? kQGridMaxLarge : kQGridMax;  // four / two per CU
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

template <int IN, int U>
static void launch_quantize_in(const QuantLaunch& q, const QuantParams& p, dim3 grid,
                               hipStream_t stream) {
    const dim3 block(kQT + kWave);
    const bool measure = q.out == nullptr;
    const int dual = q.out2 ? q.fmt2 : -1;
#define FP8_Q(F, F2, M) \
    hipLaunchKernelGGL((quantize_kernel<IN, F, F2, M, U>), grid, block, 0, stream, p)
    if (measure) {
        if (q.fmt == 0) FP8_Q(0, -1, true);
        else FP8_Q(1, -1, true);
    } else if (dual < 0) {
        if (q.fmt == 0) FP8_Q(0, -1, false);
        else FP8_Q(1, -1, false);
    } else if constexpr (IN == kInBf16) {  // the dual-format pass takes bf16 only
        if (q.fmt == 0) {
            if (dual == 0) FP8_Q(0, 0, false);
            else FP8_Q(0, 1, false);
        } else {
            if (dual == 0) FP8_Q(1, 0, false);
            else FP8_Q(1, 1, false);
        }
    }
#undef FP8_Q
}

static QuantParams quant_params(const QuantLaunch& q) {
    QuantParams p{};
    p.x = q.x;
    p.numel = q.numel;
    p.scale = q.scale;
    p.out = q.out;
    p.out2 = q.out2;
    if (q.ring_state) {
        p.hist = q.ring_state;
        p.scale_out = q.ring_state + q.ring_len;
        p.amax_slot = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 2);
        p.done = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 3);
        p.groups = reinterpret_cast<uint32_t*>(q.ring_state + ring_groups_offset(q.ring_len));
        p.len = q.ring_len;
        p.idx = q.ring_idx;
    }
    p.fmax = q.fmt ? 57344.0f : 448.0f;
    p.pow2_margin = q.pow2_margin;
    p.scale_used = q.scale_used;
    p.amax_out = q.amax_out;
    p.nt = q.cached_input ? 0 : 1;
    p.defer = q.defer_fold && q.ring_state ? 1 : 0;
    const uintptr_t al = reinterpret_cast<uintptr_t>(q.x) | reinterpret_cast<uintptr_t>(q.out) |
                         reinterpret_cast<uintptr_t>(q.out2);
    p.vec = (al & 15) == 0;
    return p;
}

hipError_t launch_quantize(const QuantLaunch& q, hipStream_t stream) {
    if (q.out2 && q.in_type != kInBf16) return hipErrorInvalidValue;
    const QuantParams p = quant_params(q);
    const bool large = p.vec && q.numel >= kLargeNumel;
    const dim3 grid(quant_grid(q.numel, p.vec, large));
    if (q.amax_out && !q.ring_state)
        hipLaunchKernelGGL(arm_amax_kernel, dim3(1), dim3(1), 0, stream, q.amax_out);
    if (large) {
        if (q.in_type == kInF16) launch_quantize_in<kInF16, kUnrollLarge>(q, p, grid, stream);
        else if (q.in_type == kInF32) launch_quantize_in<kInF32, kUnrollLarge>(q, p, grid, stream);
        else launch_quantize_in<kInBf16, kUnrollLarge>(q, p, grid, stream);
    } else {
        if (q.in_type == kInF16) launch_quantize_in<kInF16, kUnroll>(q, p, grid, stream);
        else if (q.in_type == kInF32) launch_quantize_in<kInF32, kUnroll>(q, p, grid, stream);
        else launch_quantize_in<kInBf16, kUnroll>(q, p, grid, stream);
    }
    return hipGetLastError();
}

bool quantize_two_supported(const QuantLaunch& q0, const QuantLaunch& q1) {
    auto ok = [](const QuantLaunch& q) {
        return q.in_type == kInBf16 && q.out && !q.amax_out && q.numel > 0;
    };
    return ok(q0) && ok(q1) && q0.fmt == q1.fmt && (q0.out2 ? q0.fmt2 : -1) ==
                                                       (q1.out2 ? q1.fmt2 : -1);
}

hipError_t launch_quantize_two(const QuantLaunch& q0, const QuantLaunch& q1,
                               hipStream_t stream) {
    if (!quantize_two_supported(q0, q1)) return hipErrorInvalidValue;
    const QuantParams p0 = quant_params(q0), p1 = quant_params(q1);
    // Both tensors aligned for the vector path: the large-tensor shape of
    // quantize_kernel (one slot per lane per round, a cap of four workgroups
    // per CU) at every size.  With two code stores per chunk it measured
    // faster here also below 2^25 elements (x [2048, 1024] + w [4096, 1024]:
    // the forward call 24.2 against 25.1 us), and the same at 2 x 2^24.
    const bool large = p0.vec && p1.vec;
    const int64_t cap = large ? kQGridMaxLarge : kQGridMax;
    // Each tensor's own grid, scaled down to the single launch's cap in all,
    // split in proportion to the tensors' sizes.
    int64_t b0 = quant_grid(q0.numel, p0.vec, large), b1 = quant_grid(q1.numel, p1.vec, large);
    if (b0 + b1 > cap) {
        const double f0 = (double)q0.numel / ((double)q0.numel + (double)q1.numel);
        b0 = (int64_t)(cap * f0 + 0.5);
        b0 = b0 < 1 ? 1 : (b0 > cap - 1 ? cap - 1 : b0);
        b1 = cap - b0;
    }
    const dim3 grid((unsigned)(b0 + b1)), block(kQT + kWave);
    const int dual = q0.out2 ? q0.fmt2 : -1;
#define FP8_Q2(F, F2)                                                                         \
    do {                                                                                      \
        if (large)                                                                            \
            hipLaunchKernelGGL((quantize_two_kernel<F, F2, kUnrollLarge>), grid, block, 0,     \
                               stream, p0, p1, (uint32_t)b0);                                 \
        else                                                                                  \
            hipLaunchKernelGGL((quantize_two_kernel<F, F2, kUnroll>), grid, block, 0, stream,  \
                               p0, p1, (uint32_t)b0);                                         \
    } while (0)
    if (q0.fmt == 0) {
        if (dual < 0) FP8_Q2(0, -1);
        else if (dual == 0) FP8_Q2(0, 0);
        else FP8_Q2(0, 1);
    } else {
        if (dual < 0) FP8_Q2(1, -1);
        else if (dual == 0) FP8_Q2(1, 0);
        else FP8_Q2(1, 1);
    }
#undef FP8_Q2
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dynamic (current-amax) quantize of small tensors in one launch: workgroup b
// takes job b, measures max |x| over its whole tensor, derives the step as a
// measure pass folding into a length-1 window does (max(amax / fmax /
// 2^margin, 1e-12), two IEEE divisions), writes it out and casts the tensor
// with the fp32 reciprocal of that step.  The second read comes from L2.
// For small tensors the three launch-bound passes (measure, fold, cast)
// become one launch for x and w together.
// ---------------------------------------------------------------------------
struct SmallDynParams {
    SmallDynamicJob job[2];
    float fmax;
    float pow2_margin;
};

template <int FMT>
__global__ __launch_bounds__(kQuantThreads) void quantize_small_dynamic_kernel(SmallDynParams p) {
    const SmallDynamicJob j = p.job[blockIdx.x];
    const int t = threadIdx.x;
    const bool vec =
        ((reinterpret_cast<uintptr_t>(j.x) | reinterpret_cast<uintptr_t>(j.out)) & 15) == 0;
    const int64_t nvec = vec ? j.numel / kVecElems : 0;
    const uint4* xv = reinterpret_cast<const uint4*>(j.x);
    float amax = 0.0f;
    for (int64_t c = t; c < nvec; c += kQuantThreads) {
        const uint4 r[2] = {xv[2 * c], xv[2 * c + 1]};
        amax = absmax16<kInBf16>(r, amax);
    }
    for (int64_t e = nvec * kVecElems + t; e < j.numel; e += kQuantThreads)
        amax = fmaxf(amax, fabsf(bf16_to_f32(j.x[e])));
    __shared__ float slots[kQuantWaves];
    amax = wave_max(amax);
    if (t % kWave == 0) slots[t / kWave] = amax;
    __syncthreads();
    float peak = slots[0];
#pragma unroll
    for (int w = 1; w < kQuantWaves; ++w) peak = fmaxf(peak, slots[w]);
    const float s = fmaxf(__fdiv_rn(__fdiv_rn(peak, p.fmax), p.pow2_margin), 1e-12f);
    const float m = __fdiv_rn(1.0f, s);
    if (t == 0 && j.scale_out) *j.scale_out = s;
    uint4* ov = reinterpret_cast<uint4*>(j.out);
    for (int64_t c = t; c < nvec; c += kQuantThreads) {
        const uint4 r[2] = {xv[2 * c], xv[2 * c + 1]};
        encode16<kInBf16, FMT, -1>(r, m, ov + c, nullptr);
    }
    for (int64_t e = nvec * kVecElems + t; e < j.numel; e += kQuantThreads)
        j.out[e] = cvt1<FMT>(bf16_to_f32(j.x[e]) * m);
}

hipError_t launch_quantize_small_dynamic(const SmallDynamicJob* jobs, int njobs, int fmt,
                                         float pow2_margin, hipStream_t stream) {
    if (njobs < 1 || njobs > 2) return hipErrorInvalidValue;
    SmallDynParams p{};
    for (int i = 0; i < njobs; ++i) {
        if (jobs[i].numel > kSmallDynamicNumel) return hipErrorInvalidValue;
        p.job[i] = jobs[i];
    }
    p.fmax = fmt ? 57344.0f : 448.0f;
    p.pow2_margin = pow2_margin;
    if (fmt == 0)
        hipLaunchKernelGGL(quantize_small_dynamic_kernel<0>, dim3(njobs), dim3(kQuantThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL(quantize_small_dynamic_kernel<1>, dim3(njobs), dim3(kQuantThreads), 0,
                           stream, p);
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

// A held-back fold as a launch of its own: one workgroup, a wave per ring.
__global__ __launch_bounds__(2 * kWave) void fold_job_kernel(FoldJob j) {
    const int wave = threadIdx.x / kWave;
    if (wave == 0) fold_ring_lines(j.r[0]);
    else if (j.n > 1) fold_ring_lines(j.r[1]);
}

void fold_job_add(FoldJob& j, const QuantLaunch& q) {
    if (j.n >= 2 || !q.ring_state) return;
    RingFold& r = j.r[j.n++];
    r.state = q.ring_state;
    r.len = q.ring_len;
    r.idx = q.ring_idx;
    r.fmax = q.fmt ? 57344.0f : 448.0f;
    r.pow2_margin = q.pow2_margin;
}

hipError_t launch_fold_job(const FoldJob& j, hipStream_t stream) {
    if (j.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fold_job_kernel, dim3(1), dim3(2 * kWave), 0, stream, j);
    return hipGetLastError();
}

hipError_t launch_ring_finalize(float* state, int32_t len, int32_t idx, int fmt,
                                float pow2_margin, const float* amax, hipStream_t stream) {
    hipLaunchKernelGGL(ring_finalize_kernel, dim3(1), dim3(kWave), 0, stream, state, len, idx,
                       fmt ? 57344.0f : 448.0f, pow2_margin, amax);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bias gradient: db[j] = bf16(sum_i g[i][j]), fp32 sums in a fixed order,
// optionally fused with the quantize of g (one read of g for both).
//
// Pass 1 (vector path, n % 8 == 0, 16-byte aligned rows): a workgroup of
// 1024 lanes covers 256 columns x one chunk of rows; its lanes are 32 column
// groups (8 columns = one 16-byte load) x 32 row phases, each lane summing
// every 32nd row of the chunk in row order with 8 loads in flight; the 32
// phases are then added in LDS in phase order and the chunk's 256 column
// sums written as partials.  When fused, the same lanes also encode the 8
// values of each row they read (8 codes, one 8-byte store), take the max of
// |x| and fold it like the quantize kernel (published in the last round
// before that round's stores).  Chunks are sized for about one
// workgroup per CU (the fold's atomics stay few).
// Pass 2: 64 columns per workgroup, 4 lanes per column each adding a
// quarter of the chunk partials, combined in a fixed order, one rounding.
// The scalar path (other shapes) sums a column per lane over the same
// chunks, so both paths of a given shape always give the same bits.
// ---------------------------------------------------------------------------
constexpr int kColThreads = 256;    // pass 2 and the scalar pass 1
constexpr int kQCThreads = 1024;    // vector pass 1
constexpr int kQCPhases = kQCThreads / 32;  // row phases (32 column groups each)
static_assert(kQCThreads == kQuantThreads, "the fold's per-wave slots");

// Rows per chunk: about 256 workgroups over the matrix, a multiple of the
// phase count, at most 65535 chunks.
static int64_t colsum_rows(int64_t m, int64_t n) {
    const int64_t colblocks = (n + 255) / 256;
    int64_t chunks = 256 / colblocks;
    if (chunks < 1) chunks = 1;
    int64_t rows = (m + chunks - 1) / chunks;
    rows = (rows + kQCPhases - 1) / kQCPhases * kQCPhases;
    while ((m + rows - 1) / rows > 65535) rows *= 2;
    return rows;
}
static int64_t colsum_chunks(int64_t m, int64_t n) {
    const int64_t r = colsum_rows(m, n);
    return (m + r - 1) / r;
}

size_t colsum_workspace(int64_t m, int64_t n) {
    return (size_t)colsum_chunks(m, n) * (size_t)n * sizeof(float);
}

struct QCParams {
    QuantParams q;       // quantize + fold (x = g, out = g8); unused when !QUANT
    const uint16_t* g;
    int64_t m, n, rows;
    float* part;         // [chunks][n] partial column sums
};

template <int FMT, bool QUANT>
__global__ __launch_bounds__(kQCThreads) void quantize_colsum_kernel(QCParams p) {
    float mul = 0.0f, s_read = 0.0f;
    if constexpr (QUANT) s_read = *p.q.scale;
    const int wl = threadIdx.x;
    const float win = (QUANT && p.q.hist && !p.q.defer && wl < p.q.len && wl < kWave &&
                       wl != p.q.idx)
                          ? p.q.hist[wl] : 0.0f;
    const int cg = threadIdx.x % 32;   // column group
    const int ph = threadIdx.x / 32;   // row phase
    const int64_t chunk = blockIdx.y;
    const int64_t r0 = chunk * p.rows;
    const int64_t r1 = r0 + p.rows < p.m ? r0 + p.rows : p.m;
    const int64_t c0 = (int64_t)blockIdx.x * 256 + cg * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float amax = 0.0f;
    uint32_t ticket = ~0u;  // publish_amax's result (thread 0)
    // Rounds of 8 rows per lane (8 loads in flight); the round count is
    // uniform over the workgroup, rows past the chunk read as zeros and
    // store nothing.  Column sums and |x| take the rows in order; with a
    // ring, the max is published in the last round before its stores.
    constexpr int kRows = 8;
    const int64_t nr = (r1 - r0 + kRows * kQCPhases - 1) / (kRows * kQCPhases);
    const bool colok = c0 < p.n;
    for (int64_t rd = 0; rd < nr; ++rd) {
        const int64_t rb = r0 + rd * (kRows * kQCPhases) + ph;
        uint4 v[kRows];
        // Unconditional loads (rows past the chunk re-read its first row
        // and are ignored; so are column groups past n, which read column 0)
        // keep their waits counted one by one.
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            const int64_t r = rb + u * kQCPhases;
            const int64_t rl = r < r1 ? r : r0;
            v[u] = *reinterpret_cast<const uint4*>(p.g + rl * p.n + (colok ? c0 : 0));
        }
        // the round's loads all go out first; the step's reciprocal is
        // taken after round 0's, so the wait for the step overlaps them
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QUANT) {
            if (rd == 0) mul = __fdiv_rn(1.0f, s_read);
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            if (!(colok && rb + u * kQCPhases < r1)) continue;  // adds nothing (keeps -0)
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
                acc[2 * j] += lo;
                acc[2 * j + 1] += hi;
                if constexpr (QUANT) amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
            }
        }
        if constexpr (QUANT) {
            if (p.q.hist && rd == nr - 1) ticket = publish_amax(p.q, amax, gridDim.x * gridDim.y,
                                                    blockIdx.y * gridDim.x + blockIdx.x);
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const int64_t r = rb + u * kQCPhases;
                if (colok && r < r1) {
                    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    float f[8];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f[2 * j] = bf16_lo(w[j]) * mul;
                        f[2 * j + 1] = bf16_hi(w[j]) * mul;
                    }
                    uint2 o;
                    o.x = cvt4<FMT>(f[0], f[1], f[2], f[3]);
                    o.y = cvt4<FMT>(f[4], f[5], f[6], f[7]);
                    *reinterpret_cast<uint2*>(p.q.out + r * p.n + c0) = o;
                }
            }
        }
    }
    if constexpr (QUANT) {
        if (p.q.hist && nr == 0) ticket = publish_amax(p.q, amax, gridDim.x * gridDim.y,
                                                    blockIdx.y * gridDim.x + blockIdx.x);
    }
    __shared__ float red[kQCPhases][256 + 4];
#pragma unroll
    for (int j = 0; j < 8; ++j) red[ph][cg * 8 + j] = acc[j];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int col = threadIdx.x;
        const int64_t gc = (int64_t)blockIdx.x * 256 + col;
        if (gc < p.n) {
            float sum = red[0][col];
#pragma unroll
            for (int q = 1; q < kQCPhases; ++q) sum += red[q][col];
            p.part[chunk * p.n + gc] = sum;
        }
    }
    if constexpr (QUANT) {
        if (p.q.hist && !p.q.defer) {
            finish_fold(p.q, ticket, s_read, win, gridDim.x * gridDim.y);
        } else if (p.q.scale_used && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
            *p.q.scale_used = s_read;
        }
    }
}

// Scalar pass 1: one column per lane over a chunk, rows in order.
__global__ __launch_bounds__(kColThreads) void colsum_partial_kernel(const uint16_t* g,
                                                                     int64_t m, int64_t n,
                                                                     int64_t rows, float* part) {
    const int64_t chunk = blockIdx.y;
    const int64_t r0 = chunk * rows;
    const int64_t r1 = r0 + rows < m ? r0 + rows : m;
    const int64_t c = (int64_t)blockIdx.x * kColThreads + threadIdx.x;
    if (c >= n) return;
    float acc = 0.0f;
    for (int64_t r = r0; r < r1; ++r) acc += bf16_to_f32(g[r * n + c]);
    part[chunk * n + c] = acc;
}

__global__ __launch_bounds__(kColThreads) void colsum_final_kernel(const float* part,
                                                                   int64_t chunks, int64_t n,
                                                                   uint16_t* db) {
    __shared__ float red[kColThreads];
    colsum_final_cols<kColThreads>(part, chunks, n, (int64_t)blockIdx.x * (kColThreads / 4), db,
                                   red);
}

static bool colsum_vec(const uint16_t* g, int64_t n) {
    return (n % 8 == 0) && ((reinterpret_cast<uintptr_t>(g) & 15) == 0);
}

hipError_t launch_colsum_final_job(const ColsumFinalJob& j, hipStream_t stream) {
    constexpr int kCols = kColThreads / 4;
    const dim3 grid2((unsigned)((j.n + kCols - 1) / kCols));
    hipLaunchKernelGGL(colsum_final_kernel, grid2, dim3(kColThreads), 0, stream, j.part, j.chunks,
                       j.n, j.db);
    return hipGetLastError();
}

static hipError_t launch_colsum_final(float* part, int64_t m, int64_t n, uint16_t* db,
                                      hipStream_t stream) {
    ColsumFinalJob j;
    j.part = part;
    j.chunks = colsum_chunks(m, n);
    j.n = n;
    j.db = db;
    return launch_colsum_final_job(j, stream);
}

hipError_t launch_colsum(const uint16_t* g, int64_t m, int64_t n, uint16_t* db, void* ws,
                         hipStream_t stream) {
    float* part = static_cast<float*>(ws);
    const int64_t rows = colsum_rows(m, n);
    const int64_t chunks = colsum_chunks(m, n);
    if (colsum_vec(g, n)) {
        QCParams p{};
        p.g = g;
        p.m = m;
        p.n = n;
        p.rows = rows;
        p.part = part;
        const dim3 grid1((unsigned)((n + 255) / 256), (unsigned)chunks);
        hipLaunchKernelGGL((quantize_colsum_kernel<0, false>), grid1, dim3(kQCThreads), 0, stream,
                           p);
    } else {
        const dim3 grid1((unsigned)((n + kColThreads - 1) / kColThreads), (unsigned)chunks);
        hipLaunchKernelGGL(colsum_partial_kernel, grid1, dim3(kColThreads), 0, stream, g, m, n,
                           rows, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_colsum_final(part, m, n, db, stream);
}

hipError_t launch_quantize_colsum(const QuantLaunch& q, int64_t m, int64_t n, uint16_t* db,
                                  void* ws, hipStream_t stream, ColsumFinalJob* defer) {
    if (defer) *defer = ColsumFinalJob{};
    const uint16_t* gx = static_cast<const uint16_t*>(q.x);
    const bool vec = colsum_vec(gx, n) && q.out &&
                     (reinterpret_cast<uintptr_t>(q.out) & 15) == 0 && !q.out2;
    if (!vec) {
        hipError_t e = launch_quantize(q, stream);
        if (e != hipSuccess) return e;
        return launch_colsum(gx, m, n, db, ws, stream);
    }
    QCParams p{};
    p.q.x = q.x;
    p.q.numel = m * n;
    p.q.scale = q.scale;
    p.q.out = q.out;
    if (q.ring_state) {
        p.q.hist = q.ring_state;
        p.q.scale_out = q.ring_state + q.ring_len;
        p.q.amax_slot = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 2);
        p.q.done = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 3);
        p.q.groups = reinterpret_cast<uint32_t*>(q.ring_state + ring_groups_offset(q.ring_len));
        p.q.len = q.ring_len;
        p.q.idx = q.ring_idx;
    }
    p.q.fmax = q.fmt ? 57344.0f : 448.0f;
    p.q.pow2_margin = q.pow2_margin;
    p.q.scale_used = q.scale_used;
    p.q.defer = q.defer_fold && q.ring_state ? 1 : 0;
    p.g = gx;
    p.m = m;
    p.n = n;
    p.rows = colsum_rows(m, n);
    p.part = static_cast<float*>(ws);
    const dim3 grid1((unsigned)((n + 255) / 256), (unsigned)colsum_chunks(m, n));
    if (q.fmt == 0)
        hipLaunchKernelGGL((quantize_colsum_kernel<0, true>), grid1, dim3(kQCThreads), 0, stream,
                           p);
    else
        hipLaunchKernelGGL((quantize_colsum_kernel<1, true>), grid1, dim3(kQCThreads), 0, stream,
                           p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (defer) {  // the caller's next launch carries the last pass
        defer->part = p.part;
        defer->chunks = colsum_chunks(m, n);
        defer->n = n;
        defer->db = db;
        return hipSuccess;
    }
    return launch_colsum_final(p.part, m, n, db, stream);
}

// ---------------------------------------------------------------------------
// Transposed / dual-orientation quantize ([CMP] quantize.cuh,
// fp8_quantize_tiled_kernel with the Transposed and Dual layouts; fp8.py
// _LinearFp8.backward feeds its NT GEMMs with them): bf16 x [rows][cols] ->
// out_t [cols][rows], the codes of x transposed, and with `out` the
// row-major codes too, from one read of x; amax and fold as the quantize.
//
// 128 x 128 tiles walked in grid-stride order by workgroups of 1024 lanes
// (up to 1024 workgroups, two resident per CU).
// A tile is read in 2 passes of 64 rows x 16 lanes x 16 bytes (whole
// 256-byte row segments); each lane converts its 8 values, stores the
// row-major codes directly (8 bytes, DUAL) and scatters them into an LDS
// tile [128 columns][128 rows] (pitch 144 bytes); after a barrier every
// lane writes 16 bytes of one out_t row, 8 lanes a whole 128-byte line.
// Other shapes (cols % 8, rows % 16, unaligned bases) take a per-element
// path.
// ---------------------------------------------------------------------------
constexpr int kTT = 128;           // tile edge
constexpr int kTPitch = kTT + 16;  // LDS bytes per tile column

struct QTParams {
    QuantParams q;   // x (bf16), out (row-major codes, nullable), scale, ring
    uint8_t* out_t;  // [cols][rows]
    int64_t rows, cols;
    int vec;
};

template <int FMT, bool DUAL>
__global__ __launch_bounds__(kQuantThreads) void quantize_t_kernel(QTParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTT * kTPitch];
    const float s_read = *p.q.scale;
    const float m = __fdiv_rn(1.0f, s_read);
    const int t = threadIdx.x;
    const float win =
        (p.q.hist && t < p.q.len && t < kWave && t != p.q.idx) ? p.q.hist[t] : 0.0f;
    float amax = 0.0f;
    const uint16_t* x = static_cast<const uint16_t*>(p.q.x);
    if (p.vec) {
        const int64_t tcols = (p.cols + kTT - 1) / kTT;
        const int64_t ntiles = ((p.rows + kTT - 1) / kTT) * tcols;
        const int lr = t / 16, lc = (t % 16) * 8;  // load: row within a pass, first column
        const int sc = t / 8, sr = (t % 8) * 16;   // store: tile column, first row
        for (int64_t id = blockIdx.x; id < ntiles; id += gridDim.x) {
            const int64_t r0 = (id / tcols) * kTT, c0 = (id % tcols) * kTT;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                const int rr = pass * 64 + lr;
                const int64_t r = r0 + rr, c = c0 + lc;
                if (r < p.rows && c < p.cols) {
                    const uint4 v = *reinterpret_cast<const uint4*>(x + r * p.cols + c);
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                    float f[8];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f[2 * j] = bf16_lo(w[j]);
                        f[2 * j + 1] = bf16_hi(w[j]);
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
                    uint2 o;
                    o.x = cvt4<FMT>(f[0] * m, f[1] * m, f[2] * m, f[3] * m);
                    o.y = cvt4<FMT>(f[4] * m, f[5] * m, f[6] * m, f[7] * m);
                    if constexpr (DUAL) *reinterpret_cast<uint2*>(p.q.out + r * p.cols + c) = o;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        tile[(lc + j) * kTPitch + rr] =
                            (uint8_t)(((j < 4 ? o.x : o.y) >> (8 * (j % 4))) & 0xff);
                }
            }
            __syncthreads();
            const int64_t c = c0 + sc, r = r0 + sr;
            if (c < p.cols && r < p.rows)
                *reinterpret_cast<uint4*>(p.out_t + c * p.rows + r) =
                    *reinterpret_cast<const uint4*>(tile + sc * kTPitch + sr);
            __syncthreads();  // the next tile rewrites the LDS tile
        }
    } else {
        const int64_t n = p.rows * p.cols;
        const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
        for (int64_t e = (int64_t)blockIdx.x * kQuantThreads + t; e < n; e += stride) {
            const int64_t r = e / p.cols, c = e - r * p.cols;
            const float f = bf16_to_f32(x[e]);
            amax = fmaxf(amax, fabsf(f));
            const uint8_t code = cvt1<FMT>(f * m);
            if constexpr (DUAL) p.q.out[e] = code;
            p.out_t[c * p.rows + r] = code;
        }
    }
    if (p.q.hist) {
        const uint32_t ticket = publish_amax(p.q, amax, gridDim.x, blockIdx.x);
        finish_fold(p.q, ticket, s_read, win, gridDim.x);
    } else if (p.q.scale_used && blockIdx.x == 0 && t == 0) {
        *p.q.scale_used = s_read;
    }
}

hipError_t launch_quantize_t(const QuantLaunch& q, int64_t rows, int64_t cols, uint8_t* out_t,
                             hipStream_t stream) {
    if (q.defer_fold) return hipErrorInvalidValue;  // folds itself only
    QTParams p{};
    p.q.x = q.x;
    p.q.numel = rows * cols;
    p.q.scale = q.scale;
    p.q.out = q.out;
    if (q.ring_state) {
        p.q.hist = q.ring_state;
        p.q.scale_out = q.ring_state + q.ring_len;
        p.q.amax_slot = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 2);
        p.q.done = reinterpret_cast<uint32_t*>(q.ring_state + q.ring_len + 3);
        p.q.groups = reinterpret_cast<uint32_t*>(q.ring_state + ring_groups_offset(q.ring_len));
        p.q.len = q.ring_len;
        p.q.idx = q.ring_idx;
    }
    p.q.fmax = q.fmt ? 57344.0f : 448.0f;
    p.q.pow2_margin = q.pow2_margin;
    p.q.scale_used = q.scale_used;
    p.out_t = out_t;
    p.rows = rows;
    p.cols = cols;
    const uintptr_t ax = reinterpret_cast<uintptr_t>(q.x);
    const uintptr_t ao = reinterpret_cast<uintptr_t>(q.out);
    const uintptr_t at = reinterpret_cast<uintptr_t>(out_t);
    p.vec = (cols % 8 == 0) && (rows % 16 == 0) && (ax % 16 == 0) && (ao % 8 == 0) &&
            (at % 16 == 0);
    int64_t blocks = p.vec ? ((rows + kTT - 1) / kTT) * ((cols + kTT - 1) / kTT)
                           : (rows * cols + kQuantThreads - 1) / kQuantThreads;
    // Up to 1024 workgroups (18 KB of LDS each: two resident per CU), so a
    // CU overlaps one workgroup's loads with another's transposition and
    // stores: dual pass at 8192^2 75.8 against 89.9 us with one workgroup
    // per CU walking four tiles in turn, 24.7 against 26.9 us at 4096^2.
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(kQuantThreads);
    const bool dual = q.out != nullptr;
    if (q.fmt == 0) {
        if (dual) hipLaunchKernelGGL((quantize_t_kernel<0, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((quantize_t_kernel<0, false>), grid, block, 0, stream, p);
    } else {
        if (dual) hipLaunchKernelGGL((quantize_t_kernel<1, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((quantize_t_kernel<1, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fp8lin
