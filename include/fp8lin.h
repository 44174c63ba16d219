/*
 * fp8lin.h -- C ABI of the FP8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer has two stages (AstrAI web pages by ViperEkura; "compare view
 * 3e57cc8...main" is the split diff of the fp8 extension, "author commit
 * search" the benchmark commit log):
 *   1. quantize: amax of the raw bf16 values, a per-tensor scale derived
 *      from it (current amax, or the max over a history ring of previous
 *      amaxes), and a saturating round-to-nearest-even cast to OCP E4M3 or
 *      E5M2;
 *   2. scaled GEMM: fp8 x fp8 with fp32 accumulation in the forward NT,
 *      the dX NN and the dW TN layouts (plus batched / broadcast operands),
 *      dequantized by the product of the two steps, with a fused bf16 bias
 *      and bf16 output; and the bias gradient (column sum of the output
 *      gradient).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless its comment says
 *     "host".  bf16 tensors are passed as uint16_t bit patterns, fp8 tensors
 *     as uint8_t codes; matrices are row-major.
 *   - A "scale" is the quantization STEP s (dequantization multiplier):
 *     fp8 code q represents q * s.  A quantize multiplies each element by
 *     the fp32 reciprocal 1.0f / s.
 *   - The caller owns all memory and the stream.  No entry point allocates,
 *     frees, or synchronizes; every call only enqueues kernels on `stream`
 *     (NULL = the default stream) and returns.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     bad argument returns FP8_EINVAL (or FP8_EUNSUPPORTED for a device
 *     that is not gfx950) and enqueues nothing; a failed launch returns
 *     FP8_EHIP.  fp8_last_error() then describes the failure.  Errors that
 *     only the device could see (a bad device pointer) surface as HIP
 *     errors on the stream.
 *   - Calls that share a ring or a workspace must be ordered (same stream,
 *     or synchronized); the library never locks.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* fp8 formats (compare view: csrc/kernels/fp8/common.h, FP8Format).
 * E4M3: OCP e4m3fn, no infinities, largest finite 448, NaN S.1111.111.
 * E5M2: OCP e5m2, largest finite 57344, infinities and NaNs. */
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_fmt_t;

typedef enum {
    FP8_OK = 0,
    FP8_EINVAL = 1,      /* bad argument; nothing was enqueued */
    FP8_EUNSUPPORTED = 2, /* current device is not gfx950 */
    FP8_EHIP = 3          /* a HIP call or launch failed */
} fp8_status_t;

/* Delayed-scaling state of one operand (compare view: astrai/extension/
 * fp8.py, _ScaleRing; csrc/kernels/fp8/quantize.cuh, publish_amax).
 *
 * `state` is a device buffer of fp8_ring_state_floats(len) fp32 words:
 *     [ hist[0..len) | scale | legacy | amax | done | pad | groups ]
 * hist  : amax history window;
 * scale : the published step for the next use;
 * legacy: unused (kept so the buffer layout matches the pages' ring);
 * amax, done: kernel scratch (running amax as fp32 bits, block counter as
 *        uint32 bits) that every fold leaves at zero again;
 * pad, groups: more kernel scratch, also left at zero by every fold: from
 *        the first 128-byte boundary after `done`, 16 lines of 32 words
 *        (the first level of the quantize kernels' amax reduction; the
 *        linear calls' quantizes leave their maxima there for the fold
 *        that their GEMM launch runs).
 * Only the first len + 4 words have a meaning for callers.
 * The caller zero-fills `state` once when the ring is created.
 * `len`, `idx`, `initialized` live on the host: `idx` is the slot the next
 * fold writes; `initialized` = 0 makes the linear calls seed the ring from
 * the current tensor before using it.  fp8_quantize and
 * fp8_scale_ring_finalize read the struct and never change it;
 * fp8_linear_fwd / fp8_linear_bwd seed (set initialized = 1) and advance
 * idx = (idx + 1) % len after enqueueing their work. */
typedef struct fp8_ring {
    float* state;        /* device, fp8_ring_state_floats(len) floats */
    int32_t len;         /* history length, 1 <= len <= 4096 */
    int32_t idx;         /* 0 <= idx < len */
    int32_t initialized; /* host flag for the linear calls */
    int32_t reserved;
} fp8_ring_t;

/* Number of fp32 words of a ring state buffer with history length len
 * (0 for len < 1): len + 4 rounded up to a multiple of 32, plus 512. */
int64_t fp8_ring_state_floats(int32_t len);

/* Largest finite value of a format (448 or 57344); 0 for a bad format. */
float fp8_format_max(fp8_fmt_t fmt);

/* ---------------------------------------------------------------------
 * fp8_quantize -- bf16 -> fp8 with fused amax and optional ring fold.
 * (compare view: quantize.cuh fp8_quantize_kernel and publish_amax;
 *  astrai/extension/ops/fp8.py quantize)
 *
 *   out[i] = encode_fmt( fp32( x[i] * (1.0f / *scale) ) )
 *
 * encode_fmt rounds to nearest, ties to even, and saturates: any value
 * beyond the format's largest finite value (infinity included) becomes
 * +-max.  NaN inputs produce a NaN code.
 *
 * x         : bf16 [numel]; any 2-byte alignment (16-byte alignment of x and
 *             out takes the vector path).
 * numel     : >= 0.
 * scale     : fp32 step s > 0, read once per workgroup before any fold
 *             publishes; may alias ring->state + ring->len.  Required when
 *             out != NULL, ignored otherwise.
 * out       : fp8 [numel], or NULL for a measure-only pass (amax + fold).
 * amax_out  : nullable fp32 [1]; receives amax = max_i |x[i]| over the raw
 *             values (NaN skipped; +0 for numel == 0), the quantize's
 *             second result in the pages.  The library initializes it (the
 *             caller need not clear it): with a ring the folding workgroup
 *             writes it; without one a one-thread launch arms it to +0 first
 *             and each workgroup folds its max in with one atomic max.
 * ring      : host pointer, nullable.  When set, the launch's last
 *             workgroup folds amax = max_i |x[i]| over the raw bf16 values
 *             (NaN skipped; 0 for numel == 0) into hist[ring->idx] and
 *             publishes scale = max(max(hist) / FMAX / 2^margin, 1e-12f)
 *             (two IEEE fp32 divisions) into the ring's scale slot.
 *             A length-1 ring therefore yields dynamic (current-amax)
 *             scaling: measure-only into it, then quantize with
 *             scale = ring->state + 1.
 * margin    : 0 <= margin <= 64, used by the fold only.
 * scale_used: nullable fp32 [1]; receives *scale as this launch read it
 *             (the snapshot a later GEMM must dequantize with).
 * One of out, amax_out and ring must be non-NULL, except that an empty
 * call (numel == 0) with neither ring nor amax_out does nothing and
 * returns FP8_OK.
 * ------------------------------------------------------------------- */
fp8_status_t fp8_quantize(const uint16_t* x, int64_t numel, fp8_fmt_t fmt,
                          const float* scale, uint8_t* out, float* amax_out,
                          const fp8_ring_t* ring, int32_t margin, float* scale_used,
                          hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_quantize_ex -- fp8_quantize for bf16, fp16 or fp32 inputs.
 * (compare view: csrc/kernels/fp8/quantize.cuh quant_in_traits, the input
 *  element types bf16 / fp16 / fp32 each widened to fp32 before the max and
 *  the multiply; astrai/extension/ops/fp8.py quantize; commit log 3e57cc8,
 *  quantize templated on the input type)
 *
 * x: numel elements of type in_type (device): FP8_IN_BF16 / FP8_IN_F16 as
 *    uint16 bit patterns, FP8_IN_F32 as float.  Every other argument, the
 *    result and the errors are those of fp8_quantize: amax = max |fp32(x)|
 *    (NaN skipped), q = enc(fp32(fp32(x) * fp32(1/s))).  fp16 and bf16 are
 *    exact in fp32, so the same values give the same codes in every type.
 * ------------------------------------------------------------------- */
typedef enum { FP8_IN_BF16 = 0, FP8_IN_F16 = 1, FP8_IN_F32 = 2 } fp8_in_t;

fp8_status_t fp8_quantize_ex(const void* x, fp8_in_t in_type, int64_t numel, fp8_fmt_t fmt,
                             const float* scale, uint8_t* out, float* amax_out,
                             const fp8_ring_t* ring, int32_t margin, float* scale_used,
                             hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_quantize_t -- transposed / dual-orientation quantize.
 * (compare view: csrc/kernels/fp8/quantize.cuh fp8_quantize_tiled_kernel,
 *  layouts Transposed and Dual; astrai/extension/fp8.py
 *  _LinearFp8.backward, which feeds its two NT GEMMs with g8 / g8^T from
 *  one dual pass and with x8^T, w8^T)
 *
 * x: bf16 [rows][cols] (device).  out_t: uint8 [cols][rows] receives the
 * codes of x transposed: out_t[c][r] = enc(fp32(x[r][c]) * fp32(1/s)).
 * out: nullable uint8 [rows][cols]; when given, the row-major codes too
 * (one read of x gives both orientations).  scale (required), ring, margin
 * and scale_used as fp8_quantize; the fold records max |x| like any
 * quantize.  out and out_t must not overlap.  rows * cols == 0 without a
 * ring does nothing.
 * ------------------------------------------------------------------- */
fp8_status_t fp8_quantize_t(const uint16_t* x, int64_t rows, int64_t cols, fp8_fmt_t fmt,
                            const float* scale, uint8_t* out, uint8_t* out_t,
                            const fp8_ring_t* ring, int32_t margin, float* scale_used,
                            hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_quantize2 -- one pass over x, two encodings of the same scaled values.
 * (compare view: astrai/extension/fp8.py _LinearFp8.backward, where under
 *  the HYBRID recipe x and w are quantized again in E5M2 with the forward's
 *  steps, and commit log 3e57cc8: an operand that arrives pre-quantized
 *  skips its quantize)
 *
 *   out[i]  = encode_fmt ( fp32( x[i] * (1.0f / *scale) ) )
 *   out2[i] = encode_fmt2( fp32( x[i] * (1.0f / *scale) ) )
 *
 * Both outputs are bit-identical to two fp8_quantize calls with the same
 * scale (the second without a ring): the forward can emit the backward's
 * E5M2 copies of x and w while it reads them for its E4M3 ones.
 * x, numel, scale, ring, margin, scale_used: as fp8_quantize; the ring (if
 * any) folds with fmt's largest value.  out, out2: fp8 [numel], both
 * required (no measure-only form).  Empty calls behave as fp8_quantize's.
 * ------------------------------------------------------------------- */
fp8_status_t fp8_quantize2(const uint16_t* x, int64_t numel, fp8_fmt_t fmt,
                           const float* scale, uint8_t* out, fp8_fmt_t fmt2, uint8_t* out2,
                           const fp8_ring_t* ring, int32_t margin, float* scale_used,
                           hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_scale_ring_finalize -- fold an externally measured amax.
 * (compare view: publish_amax's last-block step, as a standalone launch)
 *
 *   hist[ring->idx] = *amax;
 *   scale = max(max(hist) / FMAX / 2^margin, 1e-12f)
 *
 * ring : host pointer, required.  amax: fp32 [1] (device), >= 0.
 * Typical use: an amax reduced elsewhere (e.g. a MAX all-reduce across
 * data-parallel ranks of per-rank measure-only passes).
 * ------------------------------------------------------------------- */
fp8_status_t fp8_scale_ring_finalize(const fp8_ring_t* ring, fp8_fmt_t fmt,
                                     const float* amax, int32_t margin,
                                     hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_mm -- scaled fp8 GEMM with fp32 accumulation and bf16 output.
 * (compare view: astrai/extension/ops/fp8.py mm_fp8; csrc/kernels/fp8/
 *  common.h FP8Params and layout tags; gemm/epilogue.cuh)
 *
 *   out[b][i][j] = bf16_rne( sum_k A_b[i][k] * B_b[k][j] * fp32(sa * sb)
 *                            + bias[j] )
 *
 * A_b is m x k, stored at a + b * stride_a as
 *     trans_a == 0: [m][k] rows of stride lda (>= k)
 *     trans_a == 1: [k][m] rows of stride lda (>= m)
 * B_b is k x n, stored at b + b * stride_b as
 *     trans_b == 0: [k][n] rows of stride ldb (>= n)
 *     trans_b == 1: [n][k] rows of stride ldb (>= k)  (nn.Linear weight)
 * The linear layer uses NT (0,1) forward, NN (0,0) for dX and TN (1,0)
 * for dW; TT (1,1) is accepted too.
 * stride_a / stride_b: element strides between batches; 0 broadcasts the
 *     operand over the batch.  Ignored when batch == 1.
 * m, n, k >= 1 (k == 0 is rejected); batch >= 1; m*n*batch < 2^40.
 * scale_a, scale_b: fp32 [1] steps of A and B (device).
 * bias: bf16 [n] or NULL.  out: bf16 [batch][m][n], contiguous.
 * Both operands use the same fp8 format.  Accumulation is fp32 in an
 * unspecified order; the epilogue computes acc * s + bias in fp32 and
 * rounds once to bf16.
 * ------------------------------------------------------------------- */
fp8_status_t fp8_mm(const uint8_t* a, const uint8_t* b, fp8_fmt_t fmt, int32_t trans_a,
                    int32_t trans_b, int64_t m, int64_t n, int64_t k, int64_t lda,
                    int64_t ldb, int64_t batch, int64_t stride_a, int64_t stride_b,
                    const float* scale_a, const float* scale_b, const uint16_t* bias,
                    uint16_t* out, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_mm_ex -- fp8_mm with an fp8 bias and / or an fp8 output.
 * (compare view: astrai/extension/ops/fp8.py, the removed fp8_gemm op:
 *  out_dtype selects an fp8 E4M3 output, which needs out_scale, the
 *  output's quantization step; commit log 3e57cc8: FP8Params' bias becomes
 *  untyped with a bias_scale beside it -- none for a bf16 bias, else fp8
 *  storage dequantized after the operand scaling and before the output is
 *  quantized)
 *
 *   v[b][i][j] = fp32( sum_k A_b[i][k] * B_b[k][j] * fp32(sa * sb) + bv[j] )
 *   bv[j]      = bias_scale ? fp32( dec(bias8[j]) * bias_scale[0] )
 *                           : bf16 bias[j]               (0 without a bias)
 *   out        = bf16_rne(v)                              FP8_OUT_BF16
 *                enc( fp32( v * fp32(1 / out_scale[0]) ) ) FP8_OUT_E4M3 / _E5M2
 * enc rounds to nearest even and saturates at the format's largest value
 * (the quantize's cast); an fp8 bias is in the operands' format `fmt`.
 *
 * a .. scale_b: as fp8_mm.
 * bias: NULL, bf16 [n] (bias_scale NULL) or fp8 codes [n] (bias_scale:
 *     fp32 [1] step of the codes, device).
 * out_type: FP8_OUT_BF16 -> out is bf16 [batch][m][n] and out_scale must be
 *     NULL; FP8_OUT_E4M3 / FP8_OUT_E5M2 -> out is fp8 codes [batch][m][n]
 *     (one byte each) and out_scale (fp32 [1], device) is required.
 * With bias_scale NULL and FP8_OUT_BF16 this is fp8_mm exactly (same
 * kernels, same bits).  Accumulation order: as fp8_mm's.
 * ------------------------------------------------------------------- */
typedef enum { FP8_OUT_BF16 = 0, FP8_OUT_E4M3 = 1, FP8_OUT_E5M2 = 2 } fp8_out_t;

fp8_status_t fp8_mm_ex(const uint8_t* a, const uint8_t* b, fp8_fmt_t fmt, int32_t trans_a,
                       int32_t trans_b, int64_t m, int64_t n, int64_t k, int64_t lda,
                       int64_t ldb, int64_t batch, int64_t stride_a, int64_t stride_b,
                       const float* scale_a, const float* scale_b, const void* bias,
                       const float* bias_scale, fp8_out_t out_type, const float* out_scale,
                       void* out, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_mm_pair -- two independent fp8_mm products from one call: the
 * linear backward's dX = g . W (NN) and dW = g^T . X (TN), which use the
 * same g and nothing of each other (compare view: astrai/extension/fp8.py
 * _LinearFp8.backward).
 *
 * p0, p1: host pointers to the two problems' fp8_mm arguments (the struct
 *     below; fields as in fp8_mm).  When p0 is NN (trans_a 0, trans_b 0)
 *     and p1 is TN (trans_a 1, trans_b 0) in the same format and together
 *     they fill the GPU (at least 256 tiles of 256 x 256 each, or 256 tiles
 *     of 128 x 128 between them), one kernel runs both, problem 0's tiles
 *     first; otherwise the two products are enqueued one after the other.
 *     Either way each output is bit-identical to fp8_mm with the same
 *     arguments.
 * The problems must be independent: neither output may overlap the other
 * problem's operands (checked: the two outputs must not overlap).
 * Validation is fp8_mm's for each problem; on FP8_EINVAL nothing is
 * enqueued.
 * ------------------------------------------------------------------- */
typedef struct fp8_mm_args {
    const uint8_t* a;
    const uint8_t* b;
    fp8_fmt_t fmt;
    int32_t trans_a;
    int32_t trans_b;
    int32_t reserved;
    int64_t m, n, k, lda, ldb, batch, stride_a, stride_b;
    const float* scale_a;
    const float* scale_b;
    const uint16_t* bias; /* NULL: no bias */
    uint16_t* out;
} fp8_mm_args_t;

fp8_status_t fp8_mm_pair(const fp8_mm_args_t* p0, const fp8_mm_args_t* p1, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_colsum -- bias gradient db[j] = bf16( sum_i g[i][j] ), g bf16 [m][n].
 * (compare view: astrai/extension/fp8.py _LinearFp8.backward, grad_b)
 * fp32 accumulation in a fixed order (deterministic).  workspace: device
 * scratch of fp8_colsum_workspace(m, n) bytes (no initialization needed).
 * ------------------------------------------------------------------- */
size_t fp8_colsum_workspace(int64_t m, int64_t n);
fp8_status_t fp8_colsum(const uint16_t* g, int64_t m, int64_t n, uint16_t* db,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_quantize_colsum -- quantize of the output gradient g [m][n] fused with
 * the bias gradient: one read of g gives the codes, the amax / ring fold of
 * fp8_quantize and db[j] = bf16( sum_i g[i][j] ).
 * (compare view: astrai/extension/fp8.py _LinearFp8.backward quantizes g and
 *  takes grad_bias as the column sum of g; compare view quantize.cuh for
 *  the quantize)
 *
 * out, db, the ring and scale_used are exactly what fp8_quantize (numel =
 * m*n) and fp8_colsum give for the same arguments, bit for bit.
 * workspace: device scratch of fp8_colsum_workspace(m, n) bytes.
 * Every pointer is required except ring and scale_used.
 * ------------------------------------------------------------------- */
fp8_status_t fp8_quantize_colsum(const uint16_t* g, int64_t m, int64_t n, fp8_fmt_t fmt,
                                 const float* scale, uint8_t* out, const fp8_ring_t* ring,
                                 int32_t margin, float* scale_used, uint16_t* db,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_quantize_colsum_noalloc -- fp8_quantize_colsum for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, serving loops, harnesses that forbid allocation): the same
 * arguments without the workspace, the same results bit for bit.
 *
 * The column-sum partials go to a static scratch array inside the library
 * (one per GPU, kept until the process ends): no hipMalloc, hipFree or
 * other allocation happens in the call.  Its size bounds the shapes:
 * fp8_colsum_workspace(m, n) must be at most
 * fp8_quantize_colsum_noalloc_max_bytes() (1 MiB: every m for n up to
 * 262144 columns), else FP8_EINVAL and nothing is enqueued.  Every call on
 * one GPU shares that GPU's scratch: calls that may overlap on one GPU
 * (unordered streams) race and must not be made; calls ordered on one
 * stream are safe (each writes the partials before reading them).
 * ------------------------------------------------------------------- */
size_t fp8_quantize_colsum_noalloc_max_bytes(void);
fp8_status_t fp8_quantize_colsum_noalloc(const uint16_t* g, int64_t m, int64_t n,
                                         fp8_fmt_t fmt, const float* scale, uint8_t* out,
                                         const fp8_ring_t* ring, int32_t margin,
                                         float* scale_used, uint16_t* db, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_linear_fwd -- out[M][N] = x[M][K] w[N][K]^T * (sx*sw) + bias
 * (compare view: astrai/extension/fp8.py fp8_linear_forward)
 *
 * dynamic != 0: sx, sw are derived from the current amax of x and w
 *     (measure-only pass into length-1 scratch rings, then quantize; when
 *     x and w have at most 2^17 elements each, one launch measures and
 *     casts both, with the same codes and steps).
 *     ring_x / ring_w are ignored (may be NULL).
 * dynamic == 0 (delayed): ring_x and ring_w (host pointers, required) are
 *     seeded from the current tensors when not initialized; the scale in
 *     each ring is snapshotted by the quantize that reads it, the GEMM
 *     dequantizes with the snapshots, the current amax is folded and the
 *     next scale published (by one extra workgroup of the GEMM's launch,
 *     or a small launch after it: the quantize only gathers the amax), and
 *     both rings advance.  When the call's work has run, each ring holds
 *     what a quantize with its own fold would have left.
 * workspace: device scratch of fp8_linear_fwd_workspace(M, N, K) bytes,
 *     256-byte aligned; its first fp8_linear_fwd_x8_offset(M, N, K) bytes
 *     (6656, whatever the shape) are control slots (scratch rings for the
 *     dynamic amax) that must be zero before the first use and whose
 *     reduction words every call leaves at zero (allocate zeroed, then
 *     reuse).
 *     It receives x8 [M][K] and w8 [N][K] (fmt codes) at
 *     fp8_linear_fwd_x8_offset / _w8_offset.
 * scales_out: fp32 [2] (device) receives the steps used, [sx, sw]; the
 *     delayed backward reuses them.
 * bias: bf16 [N] or NULL.  out: bf16 [M][N].  M, N, K >= 1.
 * x8_bwd, w8_bwd: nullable outputs, fp8 [M][K] and [N][K] in fmt_bwd:
 *     x and w quantized with the forward's steps sx, sw in the backward
 *     format, written by the same pass that makes the forward's codes --
 *     exactly the operands fp8_linear_bwd makes from bf16 x and w under
 *     delayed scaling (commit log 3e57cc8: a pre-quantized operand skips
 *     its quantize kernel).  Delayed scaling only (FP8_EINVAL with
 *     dynamic != 0: the dynamic backward measures its own steps).
 *     fmt_bwd is read only when one of them is given.
 * ------------------------------------------------------------------- */
size_t fp8_linear_fwd_workspace(int64_t M, int64_t N, int64_t K);
size_t fp8_linear_fwd_x8_offset(int64_t M, int64_t N, int64_t K);
size_t fp8_linear_fwd_w8_offset(int64_t M, int64_t N, int64_t K);
fp8_status_t fp8_linear_fwd(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                            int64_t M, int64_t N, int64_t K, fp8_fmt_t fmt,
                            int32_t dynamic, int32_t margin, fp8_ring_t* ring_x,
                            fp8_ring_t* ring_w, void* workspace, size_t workspace_bytes,
                            float* scales_out, uint16_t* out, fp8_fmt_t fmt_bwd,
                            uint8_t* x8_bwd, uint8_t* w8_bwd, hipStream_t stream);

/* ---------------------------------------------------------------------
 * fp8_linear_bwd -- gradients of the linear layer in the backward format.
 * (compare view: astrai/extension/fp8.py _LinearFp8.backward; the removed
 *  linear_backward_fp8 binding in csrc/kernels/fp8/ops.cu for the NN / TN
 *  layouts)
 *
 *   dx[M][K] = g8 . w8b        * fp32(sg*sw)   (NN)
 *   dw[N][K] = g8^T . x8b      * fp32(sg*sx)   (TN)
 *   db[N]    = bf16( sum_m g[m][:] )
 * g bf16 [M][N], x bf16 [M][K], w bf16 [N][K]; g8, x8b, w8b are g, x, w
 * quantized in `fmt` (the backward format, E5M2 under HYBRID).
 *
 * dynamic == 0 (delayed): sg is ring_g's scale (seeded from g when not
 *     initialized), snapshotted by the g quantize; amax(g) is folded and
 *     the next scale published within the call (by an extra workgroup of
 *     the GEMM launch, or a small launch of its own); ring_g advances.  sx, sw are the forward's
 *     steps, scales_fwd = [sx, sw] (device fp32 [2], required).
 * dynamic != 0: sg, sx, sw are measured now from g, x, w in `fmt`;
 *     scales_fwd and ring_g are ignored.
 * dx, dw, db: each NULL to skip that gradient (x8b is only made for dw,
 *     w8b only for dx).  With both dx and dw, the two products run as
 *     fp8_mm_pair (one launch when the shapes allow); that launch then
 *     also runs db's last pass (the sum of the column-sum partials) in
 *     extra workgroups, else that pass is a launch of its own.
 * workspace: fp8_linear_bwd_workspace(M, N, K) bytes, 256-byte aligned,
 *     with the forward's 6656-byte control block and zero-once contract;
 *     it receives g8 [M][N] at fp8_linear_fwd_x8_offset(M, N, K).  When
 *     every product made takes the caller's codes (dx only with w8_bwd, dw
 *     only with x8_bwd), fp8_linear_bwd_workspace_codes(M, N, K) bytes
 *     suffice: the regions for x's and w's codes come last.
 * scales_out: nullable fp32 [3] receives [sg, sx, sw]; sx is written only
 *     when dw is made from x here, sw only when dx is made from w here.
 * x8_bwd, w8_bwd: nullable, the backward-format codes of x and w with the
 *     forward's steps (fp8_linear_fwd's outputs of the same names); when
 *     given, that quantize is skipped and x (or w) may be NULL.  Delayed
 *     scaling only (FP8_EINVAL with dynamic != 0).
 * ------------------------------------------------------------------- */
size_t fp8_linear_bwd_workspace(int64_t M, int64_t N, int64_t K);
size_t fp8_linear_bwd_workspace_codes(int64_t M, int64_t N, int64_t K);
fp8_status_t fp8_linear_bwd(const uint16_t* g, const uint16_t* x, const uint16_t* w,
                            int64_t M, int64_t N, int64_t K, fp8_fmt_t fmt,
                            int32_t dynamic, int32_t margin, const float* scales_fwd,
                            fp8_ring_t* ring_g, void* workspace, size_t workspace_bytes,
                            float* scales_out, uint16_t* dx, uint16_t* dw, uint16_t* db,
                            const uint8_t* x8_bwd, const uint8_t* w8_bwd, hipStream_t stream);

/* Message of the last non-OK status returned on the calling thread
 * (thread-local; "" if none). */
const char* fp8_last_error(void);

/* Library version string. */
const char* fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
