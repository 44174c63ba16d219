// C ABI of the fp8 linear layer: argument validation, workspace layout and
// the linear-layer orchestration.  Declarations and contracts: fp8lin.h.
//
// Orchestration follows AstrAI compare view 3e57cc8...main,
// astrai/extension/fp8.py: fp8_linear_forward (seed the rings on first use,
// snapshot the scales, quantize with the in-kernel fold, GEMM with the
// snapshots, advance) and _LinearFp8.backward (the gradient ring likewise,
// forward scales reused, operands re-quantized in the backward format).
// Unlike the pages' current backward, which transposes the operands while
// quantizing and runs NT products, dX and dW run directly as NN and TN
// products (the layouts of the pages' removed fused backward binding).

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/fp8lin.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

fp8_status_t fail(fp8_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

fp8_status_t hip_fail(hipError_t e, const char* what) {
    return fail(FP8_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// gfx950 check, cached per device.  Calls may come from several host
// threads: each slot is an atomic (a racing first call only repeats the
// property query and stores the same value).
fp8_status_t check_device() {
    static std::atomic<int> cached[64];  // 0 unknown, 1 ok, 2 unsupported
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev >= 0 && dev < 64 && cached[dev].load(std::memory_order_relaxed) == 1) return FP8_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) cached[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    if (!ok)
        return fail(FP8_EUNSUPPORTED, "device %d is %s; this library is built for gfx950",
                    dev, prop.gcnArchName);
    return FP8_OK;
}

bool fmt_ok(fp8_fmt_t f) { return f == FP8_E4M3 || f == FP8_E5M2; }

fp8_status_t check_ring(const fp8_ring_t* r, const char* name) {
    if (!r) return fail(FP8_EINVAL, "%s: ring is NULL", name);
    if (!r->state) return fail(FP8_EINVAL, "%s: ring state is NULL", name);
    if (r->len < 1 || r->len > 4096)
        return fail(FP8_EINVAL, "%s: ring len %d outside [1, 4096]", name, r->len);
    if (r->idx < 0 || r->idx >= r->len)
        return fail(FP8_EINVAL, "%s: ring idx %d outside [0, %d)", name, r->idx, r->len);
    return FP8_OK;
}

float pow2f(int32_t margin) { return ldexpf(1.0f, margin); }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace layouts.  Control block (zero-once, self-cleaning): three
// length-1 scratch rings, each a whole ring state (its group lines
// included) starting on a 128-byte boundary, then slot 3 (three floats:
// the backward's scales when the caller passes no scales_out).
constexpr int kScratchRingLen = 1;
constexpr size_t kScratchRingBytes = sizeof(float) * fp8lin::ring_state_words(kScratchRingLen);
static_assert(kScratchRingBytes % 128 == 0, "scratch rings must stay 128-byte aligned");
constexpr size_t kCtrl = (3 * kScratchRingBytes + 3 * sizeof(float) + 255) / 256 * 256;
float* scratch_ring(void* ws, int i) {
    return reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + i * kScratchRingBytes);
}

struct FwdLayout {
    size_t x8, w8, total;
};
FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K) {
    FwdLayout l;
    l.x8 = kCtrl;
    l.w8 = align256(l.x8 + (size_t)M * K);
    l.total = align256(l.w8 + (size_t)N * K);
    return l;
}

// Backward: control block, g8, the column-sum partials, then the codes of x
// and w that the call makes itself (not needed when the caller passes them,
// so `base` bytes suffice then).
struct BwdLayout {
    size_t g8, colsum, base, x8, w8, total;
};
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K) {
    BwdLayout l;
    l.g8 = kCtrl;
    l.colsum = align256(l.g8 + (size_t)M * N);
    l.base = align256(l.colsum + fp8lin::colsum_workspace(M, N));
    l.x8 = l.base;
    l.w8 = align256(l.x8 + (size_t)M * K);
    l.total = align256(l.w8 + (size_t)N * K);
    return l;
}

fp8lin::QuantLaunch make_quant(const void* x, int64_t numel, fp8_fmt_t fmt, const float* scale,
                               uint8_t* out, float* ring_state, int32_t len, int32_t idx,
                               int32_t margin, float* scale_used, uint8_t* out2 = nullptr,
                               int fmt2 = -1, int in_type = fp8lin::kInBf16,
                               float* amax_out = nullptr, bool cached_input = false) {
    fp8lin::QuantLaunch q;
    q.x = x;
    q.in_type = in_type;
    q.numel = numel;
    q.fmt = fmt;
    q.scale = scale;
    q.out = out;
    q.out2 = out2;
    q.fmt2 = fmt2;
    q.ring_state = ring_state;
    q.ring_len = len;
    q.ring_idx = idx;
    q.pow2_margin = pow2f(margin);
    q.scale_used = scale_used;
    q.amax_out = amax_out;
    q.cached_input = cached_input;
    return q;
}

fp8_status_t do_quantize(const void* x, int64_t numel, fp8_fmt_t fmt, const float* scale,
                         uint8_t* out, float* ring_state, int32_t len, int32_t idx,
                         int32_t margin, float* scale_used, hipStream_t stream,
                         uint8_t* out2 = nullptr, int fmt2 = -1,
                         int in_type = fp8lin::kInBf16, float* amax_out = nullptr,
                         bool cached_input = false) {
    const fp8lin::QuantLaunch q = make_quant(x, numel, fmt, scale, out, ring_state, len, idx,
                                             margin, scale_used, out2, fmt2, in_type, amax_out,
                                             cached_input);
    hipError_t e = fp8lin::launch_quantize(q, stream);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return FP8_OK;
}

fp8_status_t do_quantize_colsum(const uint16_t* g, int64_t m, int64_t n, fp8_fmt_t fmt,
                                const float* scale, uint8_t* out, float* ring_state,
                                int32_t len, int32_t idx, int32_t margin, float* scale_used,
                                uint16_t* db, void* ws, hipStream_t stream,
                                fp8lin::ColsumFinalJob* defer = nullptr,
                                fp8lin::FoldJob* fold = nullptr) {
    fp8lin::QuantLaunch q;
    q.x = g;
    q.numel = m * n;
    q.fmt = fmt;
    q.scale = scale;
    q.out = out;
    q.ring_state = ring_state;
    q.ring_len = len;
    q.ring_idx = idx;
    q.pow2_margin = pow2f(margin);
    q.scale_used = scale_used;
    if (fold && ring_state) {  // the ring's fold held back for a later launch
        q.defer_fold = true;
        fp8lin::fold_job_add(*fold, q);
    }
    hipError_t e = fp8lin::launch_quantize_colsum(q, m, n, db, ws, stream, defer);
    if (e != hipSuccess) return hip_fail(e, "quantize + colsum launch");
    return FP8_OK;
}

fp8lin::GemmLaunch gemm_of(const uint8_t* a, const uint8_t* b, fp8_fmt_t fmt, int ta, int tb,
                           int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb,
                           const float* sa, const float* sb, const uint16_t* bias,
                           uint16_t* out) {
    fp8lin::GemmLaunch g;
    g.a = a;
    g.b = b;
    g.fmt = fmt;
    g.trans_a = ta;
    g.trans_b = tb;
    g.m = m;
    g.n = n;
    g.k = k;
    g.lda = lda;
    g.ldb = ldb;
    g.batch = 1;
    g.scale_a = sa;
    g.scale_b = sb;
    g.bias = bias;
    g.out = out;
    return g;
}

fp8_status_t do_gemm(const uint8_t* a, const uint8_t* b, fp8_fmt_t fmt, int ta, int tb,
                     int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb,
                     const float* sa, const float* sb, const uint16_t* bias, uint16_t* out,
                     hipStream_t stream, fp8lin::FoldJob* fold = nullptr) {
    hipError_t e = fp8lin::launch_gemm(
        gemm_of(a, b, fmt, ta, tb, m, n, k, lda, ldb, sa, sb, bias, out), stream, fold);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return FP8_OK;
}

fp8_status_t do_gemm_launch(const fp8lin::GemmLaunch& g, hipStream_t stream,
                            fp8lin::FoldJob* fold = nullptr) {
    hipError_t e = fp8lin::launch_gemm(g, stream, fold);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return FP8_OK;
}

fp8_status_t do_gemm_pair(const fp8lin::GemmLaunch& g0, const fp8lin::GemmLaunch& g1,
                          hipStream_t stream, const fp8lin::ColsumFinalJob* cf = nullptr,
                          fp8lin::FoldJob* fold = nullptr) {
    hipError_t e = fp8lin::launch_gemm_pair(g0, g1, stream, cf, fold);
    if (e != hipSuccess) return hip_fail(e, "gemm pair launch");
    return FP8_OK;
}

// fp8_mm's argument checks; fills g on success.
fp8_status_t check_mm(const char* who, const fp8_mm_args_t& x, fp8lin::GemmLaunch& g) {
    if (!fmt_ok(x.fmt)) return fail(FP8_EINVAL, "%s: unsupported fp8 format %d", who, x.fmt);
    if (!x.a || !x.b || !x.out || !x.scale_a || !x.scale_b)
        return fail(FP8_EINVAL, "%s: NULL operand, output or scale", who);
    if ((x.trans_a != 0 && x.trans_a != 1) || (x.trans_b != 0 && x.trans_b != 1))
        return fail(FP8_EINVAL, "%s: trans flags must be 0 or 1", who);
    if (x.m < 1 || x.n < 1 || x.k < 1)
        return fail(FP8_EINVAL, "%s: m, n, k must be >= 1 (got %lld, %lld, %lld)", who,
                    (long long)x.m, (long long)x.n, (long long)x.k);
    if (x.batch < 1 || x.batch > 65535)
        return fail(FP8_EINVAL, "%s: batch %lld outside [1, 65535]", who, (long long)x.batch);
    const int64_t a_cols = x.trans_a ? x.m : x.k, b_cols = x.trans_b ? x.k : x.n;
    if (x.lda < a_cols)
        return fail(FP8_EINVAL, "%s: lda %lld < %lld", who, (long long)x.lda,
                    (long long)a_cols);
    if (x.ldb < b_cols)
        return fail(FP8_EINVAL, "%s: ldb %lld < %lld", who, (long long)x.ldb,
                    (long long)b_cols);
    if (x.batch > 1 && (x.stride_a < 0 || x.stride_b < 0))
        return fail(FP8_EINVAL, "%s: negative batch stride", who);
    if ((double)x.m * (double)x.n * (double)x.batch >= 1099511627776.0)
        return fail(FP8_EINVAL, "%s: output too large", who);
    g = gemm_of(x.a, x.b, x.fmt, x.trans_a, x.trans_b, x.m, x.n, x.k, x.lda, x.ldb, x.scale_a,
                x.scale_b, x.bias, x.out);
    g.batch = x.batch;
    g.stride_a = x.stride_a;
    g.stride_b = x.stride_b;
    return FP8_OK;
}

}  // namespace

extern "C" {

int64_t fp8_ring_state_floats(int32_t len) { return len < 1 ? 0 : fp8lin::ring_state_words(len); }

float fp8_format_max(fp8_fmt_t fmt) {
    return fmt == FP8_E4M3 ? 448.0f : fmt == FP8_E5M2 ? 57344.0f : 0.0f;
}

const char* fp8_last_error(void) { return g_err; }

const char* fp8_version(void) { return "fp8lin 0.1 (gfx950)"; }

static fp8_status_t quantize_entry(const char* who, const void* x, int in_type, int64_t numel,
                                   fp8_fmt_t fmt, const float* scale, uint8_t* out,
                                   float* amax_out, const fp8_ring_t* ring, int32_t margin,
                                   float* scale_used, hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt)) return fail(FP8_EINVAL, "%s: unsupported fp8 format %d", who, fmt);
    if (in_type != FP8_IN_BF16 && in_type != FP8_IN_F16 && in_type != FP8_IN_F32)
        return fail(FP8_EINVAL, "%s: unsupported input type %d", who, in_type);
    if (numel < 0) return fail(FP8_EINVAL, "%s: numel %lld < 0", who, (long long)numel);
    if (numel > 0 && !x) return fail(FP8_EINVAL, "%s: x is NULL", who);
    if (numel == 0 && !ring && !amax_out) return FP8_OK;  // nothing to convert or fold
    if (!out && !ring && !amax_out)
        return fail(FP8_EINVAL, "%s: neither out nor amax_out nor ring given", who);
    if (out && !scale) return fail(FP8_EINVAL, "%s: scale is NULL", who);
    if (ring) {
        fp8_status_t st = check_ring(ring, who);
        if (st) return st;
    }
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "%s: margin %d outside [0, 64]", who, margin);
    if (!out && scale_used)
        return fail(FP8_EINVAL, "%s: scale_used needs a quantizing call", who);
    fp8_status_t st = check_device();
    if (st) return st;
    return do_quantize(x, numel, fmt, out ? scale : nullptr, out, ring ? ring->state : nullptr,
                       ring ? ring->len : 0, ring ? ring->idx : 0, margin, scale_used, stream,
                       nullptr, -1, in_type, amax_out);
}

fp8_status_t fp8_quantize(const uint16_t* x, int64_t numel, fp8_fmt_t fmt, const float* scale,
                          uint8_t* out, float* amax_out, const fp8_ring_t* ring, int32_t margin,
                          float* scale_used, hipStream_t stream) {
    return quantize_entry("fp8_quantize", x, FP8_IN_BF16, numel, fmt, scale, out, amax_out, ring,
                          margin, scale_used, stream);
}

fp8_status_t fp8_quantize_ex(const void* x, fp8_in_t in_type, int64_t numel, fp8_fmt_t fmt,
                             const float* scale, uint8_t* out, float* amax_out,
                             const fp8_ring_t* ring, int32_t margin, float* scale_used,
                             hipStream_t stream) {
    return quantize_entry("fp8_quantize_ex", x, in_type, numel, fmt, scale, out, amax_out, ring,
                          margin, scale_used, stream);
}

fp8_status_t fp8_quantize_t(const uint16_t* x, int64_t rows, int64_t cols, fp8_fmt_t fmt,
                            const float* scale, uint8_t* out, uint8_t* out_t,
                            const fp8_ring_t* ring, int32_t margin, float* scale_used,
                            hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt)) return fail(FP8_EINVAL, "fp8_quantize_t: unsupported fp8 format %d", fmt);
    if (rows < 0 || cols < 0)
        return fail(FP8_EINVAL, "fp8_quantize_t: rows, cols must be >= 0 (got %lld, %lld)",
                    (long long)rows, (long long)cols);
    if ((double)rows * (double)cols >= 9.0e15)
        return fail(FP8_EINVAL, "fp8_quantize_t: too many elements");
    const int64_t n = rows * cols;
    if (n == 0 && !ring) return FP8_OK;
    if (n > 0 && (!x || !out_t)) return fail(FP8_EINVAL, "fp8_quantize_t: x or out_t is NULL");
    if (!scale) return fail(FP8_EINVAL, "fp8_quantize_t: scale is NULL");
    if (ring) {
        fp8_status_t st = check_ring(ring, "fp8_quantize_t");
        if (st) return st;
    }
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_quantize_t: margin %d outside [0, 64]", margin);
    if (out && n > 0) {
        const uintptr_t o0 = (uintptr_t)out, o1 = (uintptr_t)out_t;
        if (o0 < o1 + (uintptr_t)n && o1 < o0 + (uintptr_t)n)
            return fail(FP8_EINVAL, "fp8_quantize_t: out and out_t overlap");
    }
    fp8_status_t st = check_device();
    if (st) return st;
    fp8lin::QuantLaunch q;
    q.x = x;
    q.numel = n;
    q.fmt = fmt;
    q.scale = scale;
    q.out = out;
    q.ring_state = ring ? ring->state : nullptr;
    q.ring_len = ring ? ring->len : 0;
    q.ring_idx = ring ? ring->idx : 0;
    q.pow2_margin = pow2f(margin);
    q.scale_used = scale_used;
    hipError_t e = fp8lin::launch_quantize_t(q, rows, cols, out_t, stream);
    if (e != hipSuccess) return hip_fail(e, "transposed quantize launch");
    return FP8_OK;
}

fp8_status_t fp8_quantize2(const uint16_t* x, int64_t numel, fp8_fmt_t fmt, const float* scale,
                           uint8_t* out, fp8_fmt_t fmt2, uint8_t* out2, const fp8_ring_t* ring,
                           int32_t margin, float* scale_used, hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt)) return fail(FP8_EINVAL, "fp8_quantize2: unsupported fp8 format %d", fmt);
    if (!fmt_ok(fmt2))
        return fail(FP8_EINVAL, "fp8_quantize2: unsupported second fp8 format %d", fmt2);
    if (numel < 0) return fail(FP8_EINVAL, "fp8_quantize2: numel %lld < 0", (long long)numel);
    if (numel > 0 && !x) return fail(FP8_EINVAL, "fp8_quantize2: x is NULL");
    if (numel == 0 && !ring) return FP8_OK;  // nothing to convert, nothing to fold
    if (!out || !out2) return fail(FP8_EINVAL, "fp8_quantize2: out and out2 are required");
    if (!scale) return fail(FP8_EINVAL, "fp8_quantize2: scale is NULL");
    if (ring) {
        fp8_status_t st = check_ring(ring, "fp8_quantize2");
        if (st) return st;
    }
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_quantize2: margin %d outside [0, 64]", margin);
    fp8_status_t st = check_device();
    if (st) return st;
    return do_quantize(x, numel, fmt, scale, out, ring ? ring->state : nullptr,
                       ring ? ring->len : 0, ring ? ring->idx : 0, margin, scale_used, stream,
                       out2, fmt2);
}

fp8_status_t fp8_scale_ring_finalize(const fp8_ring_t* ring, fp8_fmt_t fmt, const float* amax,
                                     int32_t margin, hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt))
        return fail(FP8_EINVAL, "fp8_scale_ring_finalize: unsupported fp8 format %d", fmt);
    fp8_status_t st = check_ring(ring, "fp8_scale_ring_finalize");
    if (st) return st;
    if (!amax) return fail(FP8_EINVAL, "fp8_scale_ring_finalize: amax is NULL");
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_scale_ring_finalize: margin %d outside [0, 64]", margin);
    st = check_device();
    if (st) return st;
    hipError_t e = fp8lin::launch_ring_finalize(ring->state, ring->len, ring->idx, fmt,
                                                pow2f(margin), amax, stream);
    if (e != hipSuccess) return hip_fail(e, "ring finalize launch");
    return FP8_OK;
}

fp8_status_t fp8_mm(const uint8_t* a, const uint8_t* b, fp8_fmt_t fmt, int32_t trans_a,
                    int32_t trans_b, int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb,
                    int64_t batch, int64_t stride_a, int64_t stride_b, const float* scale_a,
                    const float* scale_b, const uint16_t* bias, uint16_t* out,
                    hipStream_t stream) {
    g_err[0] = 0;
    fp8_mm_args_t x{};
    x.a = a;
    x.b = b;
    x.fmt = fmt;
    x.trans_a = trans_a;
    x.trans_b = trans_b;
    x.m = m;
    x.n = n;
    x.k = k;
    x.lda = lda;
    x.ldb = ldb;
    x.batch = batch;
    x.stride_a = stride_a;
    x.stride_b = stride_b;
    x.scale_a = scale_a;
    x.scale_b = scale_b;
    x.bias = bias;
    x.out = out;
    fp8lin::GemmLaunch g;
    fp8_status_t st = check_mm("fp8_mm", x, g);
    if (st) return st;
    if ((st = check_device())) return st;
    hipError_t e = fp8lin::launch_gemm(g, stream);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return FP8_OK;
}

fp8_status_t fp8_mm_ex(const uint8_t* a, const uint8_t* b, fp8_fmt_t fmt, int32_t trans_a,
                       int32_t trans_b, int64_t m, int64_t n, int64_t k, int64_t lda,
                       int64_t ldb, int64_t batch, int64_t stride_a, int64_t stride_b,
                       const float* scale_a, const float* scale_b, const void* bias,
                       const float* bias_scale, fp8_out_t out_type, const float* out_scale,
                       void* out, hipStream_t stream) {
    g_err[0] = 0;
    if (out_type != FP8_OUT_BF16 && out_type != FP8_OUT_E4M3 && out_type != FP8_OUT_E5M2)
        return fail(FP8_EINVAL, "fp8_mm_ex: unsupported output type %d", (int)out_type);
    if (out_type == FP8_OUT_BF16 && out_scale)
        return fail(FP8_EINVAL, "fp8_mm_ex: out_scale given for a bf16 output");
    if (out_type != FP8_OUT_BF16 && !out_scale)
        return fail(FP8_EINVAL, "fp8_mm_ex: an fp8 output needs out_scale");
    if (bias_scale && !bias) return fail(FP8_EINVAL, "fp8_mm_ex: bias_scale without a bias");
    fp8_mm_args_t x{};
    x.a = a;
    x.b = b;
    x.fmt = fmt;
    x.trans_a = trans_a;
    x.trans_b = trans_b;
    x.m = m;
    x.n = n;
    x.k = k;
    x.lda = lda;
    x.ldb = ldb;
    x.batch = batch;
    x.stride_a = stride_a;
    x.stride_b = stride_b;
    x.scale_a = scale_a;
    x.scale_b = scale_b;
    x.bias = static_cast<const uint16_t*>(bias);
    x.out = static_cast<uint16_t*>(out);
    fp8lin::GemmLaunch g;
    fp8_status_t st = check_mm("fp8_mm_ex", x, g);
    if (st) return st;
    g.bias_scale = bias_scale;
    g.out_q = out_type == FP8_OUT_BF16 ? -1 : (out_type == FP8_OUT_E4M3 ? 0 : 1);
    g.out_scale = out_scale;
    if ((st = check_device())) return st;
    hipError_t e = fp8lin::launch_gemm(g, stream);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return FP8_OK;
}

fp8_status_t fp8_mm_pair(const fp8_mm_args_t* p0, const fp8_mm_args_t* p1, hipStream_t stream) {
    g_err[0] = 0;
    if (!p0 || !p1) return fail(FP8_EINVAL, "fp8_mm_pair: NULL argument block");
    fp8lin::GemmLaunch g0, g1;
    fp8_status_t st = check_mm("fp8_mm_pair (problem 0)", *p0, g0);
    if (st) return st;
    if ((st = check_mm("fp8_mm_pair (problem 1)", *p1, g1))) return st;
    const uintptr_t o0 = (uintptr_t)p0->out, o1 = (uintptr_t)p1->out;
    const uintptr_t e0 = o0 + (uintptr_t)(p0->batch * p0->m * p0->n * 2);
    const uintptr_t e1 = o1 + (uintptr_t)(p1->batch * p1->m * p1->n * 2);
    if (o0 < e1 && o1 < e0) return fail(FP8_EINVAL, "fp8_mm_pair: the outputs overlap");
    if ((st = check_device())) return st;
    return do_gemm_pair(g0, g1, stream);
}

size_t fp8_colsum_workspace(int64_t m, int64_t n) {
    if (m < 1 || n < 1) return 0;
    return fp8lin::colsum_workspace(m, n);
}

fp8_status_t fp8_colsum(const uint16_t* g, int64_t m, int64_t n, uint16_t* db, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    if (!g || !db || !workspace) return fail(FP8_EINVAL, "fp8_colsum: NULL pointer");
    if (m < 1 || n < 1) return fail(FP8_EINVAL, "fp8_colsum: m, n must be >= 1");
    if (workspace_bytes < fp8lin::colsum_workspace(m, n))
        return fail(FP8_EINVAL, "fp8_colsum: workspace %zu < %zu bytes", workspace_bytes,
                    fp8lin::colsum_workspace(m, n));
    fp8_status_t st = check_device();
    if (st) return st;
    hipError_t e = fp8lin::launch_colsum(g, m, n, db, workspace, stream);
    if (e != hipSuccess) return hip_fail(e, "colsum launch");
    return FP8_OK;
}

fp8_status_t fp8_quantize_colsum(const uint16_t* g, int64_t m, int64_t n, fp8_fmt_t fmt,
                                 const float* scale, uint8_t* out, const fp8_ring_t* ring,
                                 int32_t margin, float* scale_used, uint16_t* db,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt))
        return fail(FP8_EINVAL, "fp8_quantize_colsum: unsupported fp8 format %d", fmt);
    if (m < 1 || n < 1) return fail(FP8_EINVAL, "fp8_quantize_colsum: m, n must be >= 1");
    if (!g || !out || !db || !scale || !workspace)
        return fail(FP8_EINVAL, "fp8_quantize_colsum: NULL pointer");
    if (workspace_bytes < fp8lin::colsum_workspace(m, n))
        return fail(FP8_EINVAL, "fp8_quantize_colsum: workspace %zu < %zu bytes",
                    workspace_bytes, fp8lin::colsum_workspace(m, n));
    if (ring) {
        fp8_status_t st = check_ring(ring, "fp8_quantize_colsum");
        if (st) return st;
    }
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_quantize_colsum: margin %d outside [0, 64]", margin);
    fp8_status_t st = check_device();
    if (st) return st;
    return do_quantize_colsum(g, m, n, fmt, scale, out, ring ? ring->state : nullptr,
                              ring ? ring->len : 0, ring ? ring->idx : 0, margin, scale_used, db,
                              workspace, stream);
}

}  // extern "C"

namespace {

// Scratch of fp8_quantize_colsum_noalloc: the column-sum partials live in
// this file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` only names the variable; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(1) << 20;  // the partials' maximum
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device, under g_scratch_mu

fp8_status_t scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(FP8_EUNSUPPORTED, "device index %d above 63", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(FP8_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FP8_OK;
}

}  // namespace

extern "C" {

size_t fp8_quantize_colsum_noalloc_max_bytes(void) { return kScratchBytes; }

fp8_status_t fp8_quantize_colsum_noalloc(const uint16_t* g, int64_t m, int64_t n, fp8_fmt_t fmt,
                                         const float* scale, uint8_t* out,
                                         const fp8_ring_t* ring, int32_t margin,
                                         float* scale_used, uint16_t* db, hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt))
        return fail(FP8_EINVAL, "fp8_quantize_colsum_noalloc: unsupported fp8 format %d", fmt);
    if (m < 1 || n < 1) return fail(FP8_EINVAL, "fp8_quantize_colsum_noalloc: m, n must be >= 1");
    if (!g || !out || !db || !scale)
        return fail(FP8_EINVAL, "fp8_quantize_colsum_noalloc: NULL pointer");
    const size_t need = fp8lin::colsum_workspace(m, n);
    if (need > kScratchBytes)
        return fail(FP8_EINVAL,
                    "fp8_quantize_colsum_noalloc: %lld x %lld needs %zu bytes of column-sum "
                    "partials, above the static scratch of %zu bytes; use "
                    "fp8_quantize_colsum with a workspace",
                    (long long)m, (long long)n, need, kScratchBytes);
    if (ring) {
        fp8_status_t st = check_ring(ring, "fp8_quantize_colsum_noalloc");
        if (st) return st;
    }
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_quantize_colsum_noalloc: margin %d outside [0, 64]",
                    margin);
    fp8_status_t st = check_device();
    if (st) return st;
    void* ws = nullptr;
    if ((st = scratch_for_current_device(&ws))) return st;
    return do_quantize_colsum(g, m, n, fmt, scale, out, ring ? ring->state : nullptr,
                              ring ? ring->len : 0, ring ? ring->idx : 0, margin, scale_used, db,
                              ws, stream);
}

size_t fp8_linear_fwd_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    return fwd_layout(M, N, K).total;
}
size_t fp8_linear_fwd_x8_offset(int64_t M, int64_t N, int64_t K) {
    return fwd_layout(M, N, K).x8;
}
size_t fp8_linear_fwd_w8_offset(int64_t M, int64_t N, int64_t K) {
    return fwd_layout(M, N, K).w8;
}

fp8_status_t fp8_linear_fwd(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                            int64_t M, int64_t N, int64_t K, fp8_fmt_t fmt, int32_t dynamic,
                            int32_t margin, fp8_ring_t* ring_x, fp8_ring_t* ring_w,
                            void* workspace, size_t workspace_bytes, float* scales_out,
                            uint16_t* out, fp8_fmt_t fmt_bwd, uint8_t* x8_bwd, uint8_t* w8_bwd,
                            hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt)) return fail(FP8_EINVAL, "fp8_linear_fwd: unsupported fp8 format %d", fmt);
    if (!x || !w || !out || !workspace || !scales_out)
        return fail(FP8_EINVAL, "fp8_linear_fwd: NULL pointer argument");
    if (x8_bwd || w8_bwd) {
        if (dynamic)
            return fail(FP8_EINVAL,
                        "fp8_linear_fwd: backward codes need delayed scaling (the dynamic "
                        "backward measures its own steps)");
        if (!fmt_ok(fmt_bwd))
            return fail(FP8_EINVAL, "fp8_linear_fwd: unsupported backward format %d", fmt_bwd);
    }
    if (M < 1 || N < 1 || K < 1) return fail(FP8_EINVAL, "fp8_linear_fwd: M, N, K must be >= 1");
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_linear_fwd: margin %d outside [0, 64]", margin);
    if (!dynamic) {
        fp8_status_t st = check_ring(ring_x, "fp8_linear_fwd ring_x");
        if (st) return st;
        st = check_ring(ring_w, "fp8_linear_fwd ring_w");
        if (st) return st;
        if (ring_x->state == ring_w->state)
            return fail(FP8_EINVAL, "fp8_linear_fwd: ring_x and ring_w share a state buffer");
    }
    const FwdLayout L = fwd_layout(M, N, K);
    if (workspace_bytes < L.total)
        return fail(FP8_EINVAL, "fp8_linear_fwd: workspace %zu < %zu bytes", workspace_bytes,
                    L.total);
    if ((uintptr_t)workspace & 255)
        return fail(FP8_EINVAL, "fp8_linear_fwd: workspace not 256-byte aligned");
    fp8_status_t st = check_device();
    if (st) return st;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* x8 = ws + L.x8;
    uint8_t* w8 = ws + L.w8;
    float* sx = scales_out;
    float* sw = scales_out + 1;
    fp8lin::FoldJob fold;  // delayed: the rings' folds, held back for the GEMM's launch
    if (dynamic) {
        // Current-amax scaling: measure into a length-1 scratch ring, then
        // quantize with the scale it published.
        float* rx = scratch_ring(workspace, 0);
        float* rw = scratch_ring(workspace, 1);
        if (M * K <= fp8lin::kSmallDynamicNumel && N * K <= fp8lin::kSmallDynamicNumel) {
            // small tensors: measure, step and cast of x and w in one launch
            fp8lin::SmallDynamicJob jobs[2];
            jobs[0].x = x, jobs[0].numel = M * K, jobs[0].out = x8, jobs[0].scale_out = sx;
            jobs[1].x = w, jobs[1].numel = N * K, jobs[1].out = w8, jobs[1].scale_out = sw;
            hipError_t e = fp8lin::launch_quantize_small_dynamic(jobs, 2, fmt, pow2f(margin),
                                                                 stream);
            if (e != hipSuccess) return hip_fail(e, "quantize launch");
        } else {
            // x and w are read twice in a row: ordinary (cached) loads.
            const int in = fp8lin::kInBf16;
            if ((st = do_quantize(x, M * K, fmt, nullptr, nullptr, rx, kScratchRingLen, 0, margin,
                                  nullptr, stream, nullptr, -1, in, nullptr, true)))
                return st;
            if ((st = do_quantize(w, N * K, fmt, nullptr, nullptr, rw, kScratchRingLen, 0, margin,
                                  nullptr, stream, nullptr, -1, in, nullptr, true)))
                return st;
            if ((st = do_quantize(x, M * K, fmt, rx + kScratchRingLen, x8, nullptr, 0, 0, margin,
                                  sx, stream, nullptr, -1, in, nullptr, true)))
                return st;
            if ((st = do_quantize(w, N * K, fmt, rw + kScratchRingLen, w8, nullptr, 0, 0, margin,
                                  sw, stream, nullptr, -1, in, nullptr, true)))
                return st;
        }
    } else {
        if (!ring_w->initialized) {
            if ((st = do_quantize(w, N * K, fmt, nullptr, nullptr, ring_w->state, ring_w->len,
                                  ring_w->idx, margin, nullptr, stream)))
                return st;
            ring_w->initialized = 1;
        }
        if (!ring_x->initialized) {
            if ((st = do_quantize(x, M * K, fmt, nullptr, nullptr, ring_x->state, ring_x->len,
                                  ring_x->idx, margin, nullptr, stream)))
                return st;
            ring_x->initialized = 1;
        }
        // Each quantize reads the ring's published step (its snapshot goes
        // to scales_out) and takes its amax into the ring's group lines; the
        // fold of both rings is held back and runs as the GEMM launch's
        // last workgroup (the GEMM reads the snapshots, not the rings), so
        // no chain of dependent atomics ends the quantize.
        // With x8_bwd / w8_bwd the same pass also writes the backward's
        // codes: the same scaled values in fmt_bwd.
        // x and w go in one launch when both or neither write backward codes.
        fp8lin::QuantLaunch qx =
            make_quant(x, M * K, fmt, ring_x->state + ring_x->len, x8, ring_x->state,
                       ring_x->len, ring_x->idx, margin, sx, x8_bwd, x8_bwd ? (int)fmt_bwd : -1);
        fp8lin::QuantLaunch qw =
            make_quant(w, N * K, fmt, ring_w->state + ring_w->len, w8, ring_w->state,
                       ring_w->len, ring_w->idx, margin, sw, w8_bwd, w8_bwd ? (int)fmt_bwd : -1);
        qx.defer_fold = qw.defer_fold = true;
        fp8lin::fold_job_add(fold, qx);
        fp8lin::fold_job_add(fold, qw);
        if (fp8lin::quantize_two_supported(qx, qw)) {
            hipError_t e = fp8lin::launch_quantize_two(qx, qw, stream);
            if (e != hipSuccess) return hip_fail(e, "quantize launch");
        } else {
            hipError_t e = fp8lin::launch_quantize(qx, stream);
            if (e == hipSuccess) e = fp8lin::launch_quantize(qw, stream);
            if (e != hipSuccess) return hip_fail(e, "quantize launch");
        }
    }
    if ((st = do_gemm(x8, w8, fmt, 0, 1, M, N, K, K, K, sx, sw, bias, out, stream, &fold)))
        return st;
    if (!dynamic) {
        ring_x->idx = (ring_x->idx + 1) % ring_x->len;
        ring_w->idx = (ring_w->idx + 1) % ring_w->len;
    }
    return FP8_OK;
}

size_t fp8_linear_bwd_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    return bwd_layout(M, N, K).total;
}

size_t fp8_linear_bwd_workspace_codes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    return bwd_layout(M, N, K).base;
}

fp8_status_t fp8_linear_bwd(const uint16_t* g, const uint16_t* x, const uint16_t* w, int64_t M,
                            int64_t N, int64_t K, fp8_fmt_t fmt, int32_t dynamic,
                            int32_t margin, const float* scales_fwd, fp8_ring_t* ring_g,
                            void* workspace, size_t workspace_bytes, float* scales_out,
                            uint16_t* dx, uint16_t* dw, uint16_t* db, const uint8_t* x8_bwd,
                            const uint8_t* w8_bwd, hipStream_t stream) {
    g_err[0] = 0;
    if (!fmt_ok(fmt)) return fail(FP8_EINVAL, "fp8_linear_bwd: unsupported fp8 format %d", fmt);
    if (!g || !workspace) return fail(FP8_EINVAL, "fp8_linear_bwd: NULL g or workspace");
    if (dx && !w && !w8_bwd) return fail(FP8_EINVAL, "fp8_linear_bwd: dx needs w or w8_bwd");
    if (dw && !x && !x8_bwd) return fail(FP8_EINVAL, "fp8_linear_bwd: dw needs x or x8_bwd");
    if (dynamic && (x8_bwd || w8_bwd))
        return fail(FP8_EINVAL,
                    "fp8_linear_bwd: pre-quantized x / w need delayed scaling (the dynamic "
                    "backward measures its own steps)");
    if (M < 1 || N < 1 || K < 1) return fail(FP8_EINVAL, "fp8_linear_bwd: M, N, K must be >= 1");
    if (margin < 0 || margin > 64)
        return fail(FP8_EINVAL, "fp8_linear_bwd: margin %d outside [0, 64]", margin);
    if (!dynamic) {
        if (!scales_fwd)
            return fail(FP8_EINVAL, "fp8_linear_bwd: delayed scaling needs scales_fwd");
        fp8_status_t st = check_ring(ring_g, "fp8_linear_bwd ring_g");
        if (st) return st;
    }
    const BwdLayout L = bwd_layout(M, N, K);
    // the x / w code regions are needed only for codes made here
    const size_t need = (dw && !x8_bwd) || (dx && !w8_bwd) ? L.total : L.base;
    if (workspace_bytes < need)
        return fail(FP8_EINVAL, "fp8_linear_bwd: workspace %zu < %zu bytes", workspace_bytes,
                    need);
    if ((uintptr_t)workspace & 255)
        return fail(FP8_EINVAL, "fp8_linear_bwd: workspace not 256-byte aligned");
    fp8_status_t st = check_device();
    if (st) return st;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* g8 = ws + L.g8;
    uint8_t* x8 = ws + L.x8;
    uint8_t* w8 = ws + L.w8;
    // Scales used: in scales_out when given, else in the control block.
    float* sc = scales_out ? scales_out : scratch_ring(workspace, 3);
    // With dX and dW both wanted, the bias gradient's last pass rides on
    // their paired launch.
    fp8lin::ColsumFinalJob cf;
    fp8lin::ColsumFinalJob* defer = dx && dw ? &cf : nullptr;
    float* sg = sc;
    const float* sx;
    const float* sw;
    bool xw_cast = false;  // x8 / w8 already made (small dynamic path)
    fp8lin::FoldJob fold;  // delayed: g's ring fold, held back for the GEMM's launch
    if (dynamic) {
        float* rg = scratch_ring(workspace, 0);
        float* rx = scratch_ring(workspace, 1);
        float* rw = scratch_ring(workspace, 2);
        // each tensor is read again right after its measure: cached loads
        if ((st = do_quantize(g, M * N, fmt, nullptr, nullptr, rg, kScratchRingLen, 0, margin,
                              nullptr, stream, nullptr, -1, fp8lin::kInBf16, nullptr, true)))
            return st;
        if (db) {
            if ((st = do_quantize_colsum(g, M, N, fmt, rg + kScratchRingLen, g8, nullptr, 0, 0,
                                         margin, sg, db, ws + L.colsum, stream, defer)))
                return st;
        } else if ((st = do_quantize(g, M * N, fmt, rg + kScratchRingLen, g8, nullptr, 0, 0,
                                     margin, sg, stream, nullptr, -1, fp8lin::kInBf16, nullptr, true))) {
            return st;
        }
        const bool small = (!dw || M * K <= fp8lin::kSmallDynamicNumel) &&
                           (!dx || N * K <= fp8lin::kSmallDynamicNumel);
        if (small && (dx || dw)) {
            // small x and w: measure, step and cast in one launch
            float* sxo = scales_out ? scales_out + 1 : rx + kScratchRingLen;
            float* swo = scales_out ? scales_out + 2 : rw + kScratchRingLen;
            fp8lin::SmallDynamicJob jobs[2];
            int nj = 0;
            if (dx) {
                jobs[nj].x = w, jobs[nj].numel = N * K, jobs[nj].out = w8, jobs[nj].scale_out = swo;
                ++nj;
            }
            if (dw) {
                jobs[nj].x = x, jobs[nj].numel = M * K, jobs[nj].out = x8, jobs[nj].scale_out = sxo;
                ++nj;
            }
            hipError_t e = fp8lin::launch_quantize_small_dynamic(jobs, nj, fmt, pow2f(margin),
                                                                 stream);
            if (e != hipSuccess) return hip_fail(e, "quantize launch");
            xw_cast = true;
            sx = sxo;
            sw = swo;
        } else {
            if (dw) {
                if ((st = do_quantize(x, M * K, fmt, nullptr, nullptr, rx, kScratchRingLen, 0,
                                      margin, nullptr, stream, nullptr, -1, fp8lin::kInBf16, nullptr, true)))
                    return st;
            }
            if (dx) {
                if ((st = do_quantize(w, N * K, fmt, nullptr, nullptr, rw, kScratchRingLen, 0,
                                      margin, nullptr, stream, nullptr, -1, fp8lin::kInBf16, nullptr, true)))
                    return st;
            }
            sx = rx + kScratchRingLen;
            sw = rw + kScratchRingLen;
        }
    } else {
        if (!ring_g->initialized) {
            if ((st = do_quantize(g, M * N, fmt, nullptr, nullptr, ring_g->state, ring_g->len,
                                  ring_g->idx, margin, nullptr, stream)))
                return st;
            ring_g->initialized = 1;
        }
        // g's amax goes into its ring's group lines; the fold runs as the
        // GEMM launch's last workgroup (or a launch of its own)
        if (db) {
            if ((st = do_quantize_colsum(g, M, N, fmt, ring_g->state + ring_g->len, g8,
                                         ring_g->state, ring_g->len, ring_g->idx, margin, sg, db,
                                         ws + L.colsum, stream, defer, &fold)))
                return st;
        } else {
            fp8lin::QuantLaunch q = make_quant(g, M * N, fmt, ring_g->state + ring_g->len, g8,
                                               ring_g->state, ring_g->len, ring_g->idx, margin,
                                               sg);
            q.defer_fold = true;
            fp8lin::fold_job_add(fold, q);
            hipError_t e = fp8lin::launch_quantize(q, stream);
            if (e != hipSuccess) return hip_fail(e, "quantize launch");
        }
        sx = scales_fwd;
        sw = scales_fwd + 1;
    }
    // dynamic: w and x were just measured (cached); delayed: last read in the
    // forward (cold, non-temporal loads)
    const bool cached = dynamic != 0;
    const int in = fp8lin::kInBf16;
    if (dx && !xw_cast && !w8_bwd &&
        (st = do_quantize(w, N * K, fmt, sw, w8, nullptr, 0, 0, margin,
                          scales_out ? scales_out + 2 : nullptr, stream, nullptr, -1, in,
                          nullptr, cached)))
        return st;
    if (dw && !xw_cast && !x8_bwd &&
        (st = do_quantize(x, M * K, fmt, sx, x8, nullptr, 0, 0, margin,
                          scales_out ? scales_out + 1 : nullptr, stream, nullptr, -1, in,
                          nullptr, cached)))
        return st;
    // dX[M][K] = g8[M][N] . w8[N][K]  (NN)
    // dW[N][K] = g8^T . x8: A = g8 stored [M][N] (k-major rows of m), B = x8 [M][K]  (TN)
    // Both from one launch when both are wanted (independent products).
    const uint8_t* w8u = w8_bwd ? w8_bwd : w8;  // caller's pre-quantized codes, if any
    const uint8_t* x8u = x8_bwd ? x8_bwd : x8;
    const fp8lin::GemmLaunch gdx = gemm_of(g8, w8u, fmt, 0, 0, M, K, N, N, K, sg, sw, nullptr, dx);
    const fp8lin::GemmLaunch gdw = gemm_of(g8, x8u, fmt, 1, 0, N, K, M, N, K, sg, sx, nullptr, dw);
    if (dx && dw) {
        if ((st = do_gemm_pair(gdx, gdw, stream, &cf, &fold))) return st;
    } else if (dx) {
        if ((st = do_gemm_launch(gdx, stream, &fold))) return st;
    } else if (dw) {
        if ((st = do_gemm_launch(gdw, stream, &fold))) return st;
    }
    if (fold.n > 0) {  // no GEMM carried it (only the bias gradient wanted)
        hipError_t e = fp8lin::launch_fold_job(fold, stream);
        if (e != hipSuccess) return hip_fail(e, "fold launch");
    }
    if (!dynamic) ring_g->idx = (ring_g->idx + 1) % ring_g->len;
    return FP8_OK;
}

}  // extern "C"
