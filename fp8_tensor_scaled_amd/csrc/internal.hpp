// Host-side declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8lin {

// Ring state layout (fp32 words): [hist len | scale | legacy | amax | done],
// then, from the next 128-byte boundary, kRingGroups lines of 32 words whose
// first two words are a group's running max and counter (the quantize
// fold's first level; left at zero by every fold).
constexpr int kRingGroups = 16;
constexpr int kRingGroupWords = 32;
constexpr int64_t ring_groups_offset(int32_t len) { return ((int64_t)len + 4 + 31) / 32 * 32; }
constexpr int64_t ring_state_words(int32_t len) {
    return ring_groups_offset(len) + (int64_t)kRingGroups * kRingGroupWords;
}

// Everything a quantize launch needs (plain values, no ownership).
// Quantize input element types (each widens exactly to fp32).
enum InType : int { kInBf16 = 0, kInF16 = 1, kInF32 = 2 };

struct QuantLaunch {
    const void* x = nullptr;  // numel elements of type in_type
    int in_type = kInBf16;
    int64_t numel = 0;
    int fmt = 0;
    const float* scale = nullptr;  // step s (device); m = 1/s
    uint8_t* out = nullptr;        // null: measure only
    uint8_t* out2 = nullptr;       // optional second encoding (format fmt2)
    int fmt2 = -1;
    float* ring_state = nullptr;   // null: no fold
    int32_t ring_len = 0;
    int32_t ring_idx = 0;
    float pow2_margin = 1.0f;
    float* scale_used = nullptr;
    float* amax_out = nullptr;     // optional: receives max |x| (fp32)
    // The input was just read and sits in the caches (a measure pass then
    // the cast): ordinary loads.  Otherwise 2-byte inputs are loaded
    // non-temporally, which skips the MALL for data read once.
    bool cached_input = false;
    // With a ring: hold the fold back (FoldJob below); the kernel then
    // writes the step snapshot to scale_used itself.  Not with amax_out.
    bool defer_fold = false;
};
hipError_t launch_quantize(const QuantLaunch& q, hipStream_t stream);

// A ring fold held back from quantize launches made with defer_fold: their
// workgroups only take the atomic max of their |x| maxima into the ring's
// group lines (no counters, no dependent round trips), and the fold --
// hist[idx] = the largest line, the next step from the window's peak, the
// lines back to zero -- runs later in stream order: as one extra workgroup
// of the GEMM launch that follows (which reads the step snapshot, never the
// ring), or as a launch of its own.  It leaves the ring state the
// quantize's own fold leaves, bit for bit.
struct RingFold {
    float* state = nullptr;  // ring state words (layout above)
    int32_t len = 0, idx = 0;
    float fmax = 448.0f;
    float pow2_margin = 1.0f;
};
struct FoldJob {
    RingFold r[2];
    int n = 0;  // rings held, 0..2
};
// Appends q's ring (q.ring_state set) to j.
void fold_job_add(FoldJob& j, const QuantLaunch& q);
hipError_t launch_fold_job(const FoldJob& j, hipStream_t stream);

// Two bf16 quantizes with codes (same format, same second format or none, no
// amax_out) in one launch, each with its own fold; results are those of two
// launch_quantize calls.
bool quantize_two_supported(const QuantLaunch& q0, const QuantLaunch& q1);
hipError_t launch_quantize_two(const QuantLaunch& q0, const QuantLaunch& q1, hipStream_t stream);

// Dynamic (current-amax) quantize of up to two small bf16 tensors in one
// launch, one workgroup each: measure max |x|, derive the step, cast.  The
// codes and steps equal those of a measure-only pass into a length-1 ring
// followed by the cast with its step.  For numel <= kSmallDynamicNumel: the
// dynamic forward at M = N = K = n took 7.8 / 11.7 / 26.0 us this way against
// 17.2 / 18.5 / 19.4 us through the general path's launches at 2^14 / 2^16 /
// 2^18 elements per tensor, so the paths cross near 2^17.
constexpr int64_t kSmallDynamicNumel = int64_t(1) << 17;
struct SmallDynamicJob {
    const uint16_t* x = nullptr;
    int64_t numel = 0;
    uint8_t* out = nullptr;
    float* scale_out = nullptr;  // receives the step
};
hipError_t launch_quantize_small_dynamic(const SmallDynamicJob* jobs, int njobs, int fmt,
                                         float pow2_margin, hipStream_t stream);

// Transposed quantize of bf16 q.x [rows][cols] into out_t [cols][rows]; with
// q.out also the row-major codes (one read of x).  Ring, scale, scale_used as
// launch_quantize; q.in_type must be bf16.
hipError_t launch_quantize_t(const QuantLaunch& q, int64_t rows, int64_t cols, uint8_t* out_t,
                             hipStream_t stream);

hipError_t launch_ring_finalize(float* state, int32_t len, int32_t idx, int fmt,
                                float pow2_margin, const float* amax, hipStream_t stream);

// GEMM problem in the C-ABI's terms.
struct GemmLaunch {
    const uint8_t* a = nullptr;
    const uint8_t* b = nullptr;
    int fmt = 0;
    int trans_a = 0, trans_b = 0;
    int64_t m = 0, n = 0, k = 0, lda = 0, ldb = 0;
    int64_t batch = 1, stride_a = 0, stride_b = 0;
    const float* scale_a = nullptr;
    const float* scale_b = nullptr;
    // bias: bf16 [n] when bias_scale is null, else fp8 codes [n] of fmt whose
    // values are code * bias_scale[0]; NULL for none.
    const void* bias = nullptr;
    const float* bias_scale = nullptr;
    // out: bf16 [batch][m][n] (out_q < 0) or fp8 codes of format out_q
    // (0 E4M3, 1 E5M2) of the value times fp32(1 / out_scale[0]).
    void* out = nullptr;
    int out_q = -1;
    const float* out_scale = nullptr;
    // Needs the extended epilogue (fp8 bias or fp8 output).
    bool ext() const { return bias_scale != nullptr || out_q >= 0; }
};
// A held-back fold (nullable; consumed: n is 0 on success) rides along as
// an extra workgroup of the tiled kernels' launch, or runs as a launch of
// its own after the GEMM.
hipError_t launch_gemm(const GemmLaunch& g, hipStream_t stream, FoldJob* fold = nullptr);

// The bias gradient's last pass (chunk partials -> bf16 db) as a job that
// another launch can carry; db == nullptr: no job.
struct ColsumFinalJob {
    const float* part = nullptr;  // [chunks][n]
    int64_t chunks = 0;
    int64_t n = 0;
    uint16_t* db = nullptr;
};
hipError_t launch_colsum_final_job(const ColsumFinalJob& j, hipStream_t stream);

// Two independent GEMMs: one launch when both take the tiled kernels' paired
// form (the linear backward's NN dX and TN dW), else launch_gemm twice in
// order.  Results are bit-identical to the two separate launches.  A job
// `cf` (nullable) rides along as extra workgroups of the paired launch, or
// runs as its own launch after the two; a held-back fold as launch_gemm.
hipError_t launch_gemm_pair(const GemmLaunch& g0, const GemmLaunch& g1, hipStream_t stream,
                            const ColsumFinalJob* cf = nullptr, FoldJob* fold = nullptr);

// Column sum (bias gradient).
size_t colsum_workspace(int64_t m, int64_t n);
hipError_t launch_colsum(const uint16_t* g, int64_t m, int64_t n, uint16_t* db, void* ws,
                         hipStream_t stream);
// Quantize of g [m][n] (q.x = g, q.numel = m*n) fused with its column sum:
// one read of g when the shape allows, else the two launches in sequence;
// the column sums are the bits launch_colsum gives for the same g.  With
// `defer`, the fused form leaves its last pass (partials -> db) to the
// caller in *defer instead of launching it; defer->db stays nullptr when
// nothing was left.
hipError_t launch_quantize_colsum(const QuantLaunch& q, int64_t m, int64_t n, uint16_t* db,
                                  void* ws, hipStream_t stream, ColsumFinalJob* defer = nullptr);

}  // namespace fp8lin
