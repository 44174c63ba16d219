/*
 * fp8_oracle.c -- plain, slow, CPU reference of the FP8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product
 * path (the HIP library and its Python binding) never calls it, and the two
 * share no source, header, table or helper.
 *
 * Every routine is the written-out definition of what it computes: no
 * blocking, no fusion, no reordering beyond what the definition states.
 * Floating point that the method performs in fp32 is done here in fp32 with
 * IEEE round-to-nearest-even (x86-64 SSE, no contraction: build with
 * -ffp-contract=off and without fast-math); sums are carried in fp64.
 *
 * Sources (the web pages of the AstrAI repository by ViperEkura):
 *   [CMP]  compare view 3e57cc8...main (split diff), file hunks named below
 *   [LOG1] commit log at 3e57cc8 (astrai/extension)
 *   [LOG4] author commit search (benchmark commit messages)
 * plus the OCP 8-bit floating point specification (E4M3 / E5M2) for the
 * bit encodings, which the pages name but do not spell out.
 *
 * Parity pins: every exported function is pinned by a CPU test (see the
 * test module headers); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define FMT_E4M3 0
#define FMT_E5M2 1

/* Format constants of the OCP definition.  The maxima 448 and 57344 are the
 * ones [CMP] astrai/extension/fp8.py prints in its FP8_MAX table. */
static int fmt_mbits(int fmt) { return fmt == FMT_E5M2 ? 2 : 3; }
static int fmt_bias(int fmt) { return fmt == FMT_E5M2 ? 15 : 7; }
double orc_fmt_max(int fmt) { return fmt == FMT_E5M2 ? 57344.0 : 448.0; }
static uint8_t fmt_max_code(int fmt) { return fmt == FMT_E5M2 ? 0x7B : 0x7E; }

/* ------------------------------------------------------------------------
 * fp8 decode: byte -> exact value (OCP definition).
 * E4M3: bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN.
 * E5M2: bias 15, 2 mantissa bits, exponent field 31 is inf (mantissa 0) or
 * NaN (mantissa != 0).
 * ---------------------------------------------------------------------- */
float orc_decode(uint8_t byte, int fmt)
{
    const int mbits = fmt_mbits(fmt);
    const int bias = fmt_bias(fmt);
    const int sign = byte >> 7;
    const int expf = (byte & 0x7F) >> mbits;
    const int mant = byte & ((1 << mbits) - 1);
    double v;
    if (fmt == FMT_E4M3 && (byte & 0x7F) == 0x7F) return NAN;
    if (fmt == FMT_E5M2 && expf == 31) {
        if (mant) return NAN;
        return sign ? -INFINITY : INFINITY;
    }
    if (expf == 0)
        v = ldexp((double)mant, 1 - bias - mbits); /* subnormal */
    else
        v = ldexp((double)((1 << mbits) + mant), expf - bias - mbits);
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------------
 * fp8 encode: fp32 -> byte, round to nearest with ties to even, saturating
 * to the largest finite value ("satfinite").  [CMP] quantize.cuh, cvt_fp8 /
 * cvt_fp8x2: the kernel converts with round-nearest-even and satfinite.
 *
 * Method: find the spacing q of representable values around |v| (the
 * subnormal spacing below the smallest normal), round |v|/q to the nearest
 * integer with ties to even (nearbyint in the default rounding mode), and
 * rebuild the bit fields from the rounded value.  Any |v| >= max (including
 * infinity) saturates.  NaN maps to the NaN code S.1111111 with the sign
 * kept (the pages never feed NaN; this choice is documented, not pinned).
 * ---------------------------------------------------------------------- */
uint8_t orc_encode(float v, int fmt)
{
    const int mbits = fmt_mbits(fmt);
    const int bias = fmt_bias(fmt);
    const int e_min = 1 - bias; /* exponent of the smallest normal */
    const double fmax = orc_fmt_max(fmt);
    uint32_t bits;
    memcpy(&bits, &v, sizeof bits);
    const uint8_t sign = (bits >> 31) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;
    const double a = fabs((double)v);
    if (a >= fmax) return sign | fmt_max_code(fmt);
    if (a == 0.0) return sign;
    int e = ilogb(a);
    if (e < e_min) e = e_min;
    const double q = ldexp(1.0, e - mbits);
    const double n = nearbyint(a / q); /* a / q is exact: q is a power of 2 */
    double r = n * q;
    if (r > fmax) r = fmax; /* unreachable for a < fmax; kept as a guard */
    if (r == 0.0) return sign;
    const int er = ilogb(r);
    if (er < e_min) {
        const int mant = (int)(r / ldexp(1.0, e_min - mbits));
        return sign | (uint8_t)mant;
    }
    const int mant = (int)(r / ldexp(1.0, er - mbits)) - (1 << mbits);
    return sign | (uint8_t)(((er + bias) << mbits) | mant);
}

/* Encode an fp32 array (used by the exhaustive pin). */
void orc_encode_array(const float* v, int64_t n, int fmt, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(v[i], fmt);
}

/* Encode every fp32 bit pattern in [first, first + n) (exhaustive pin). */
void orc_encode_bits_range(uint32_t first, int64_t n, int fmt, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t b = first + (uint32_t)i;
        float f;
        memcpy(&f, &b, sizeof f);
        out[i] = orc_encode(f, fmt);
    }
}

/* ------------------------------------------------------------------------
 * bf16 helpers.  A bf16 value is the upper half of an fp32 bit pattern, so
 * widening is exact.  Narrowing from fp64 rounds ONCE to nearest-even
 * (bias 127, 7 stored mantissa bits, subnormal spacing 2^-133, overflow to
 * infinity), with no intermediate fp32 rounding.
 * ---------------------------------------------------------------------- */
float orc_bf16_to_f32(uint16_t h)
{
    const uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

uint16_t orc_bf16_from_f64(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    if (isnan(v)) return sign | 0x7FC0;
    const double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e = ilogb(a);
    if (e < -126) e = -126;
    const double q = ldexp(1.0, e - 7);
    const double n = nearbyint(a / q);
    const double r = n * q;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    const int er = ilogb(r);
    if (er < -126) return sign | (uint16_t)(r / ldexp(1.0, -133));
    const int mant = (int)(r / ldexp(1.0, er - 7)) - 128;
    return sign | (uint16_t)(((er + 127) << 7) | mant);
}

void orc_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f64(v[i]);
}

/* ------------------------------------------------------------------------
 * amax: max |x_i| over the raw (pre-quantization) bf16 values, as fp32.
 * [CMP] quantize.cuh, fp8_quantize_kernel: the running max takes fabsf of
 * the unscaled input; [LOG1] records the bug where the quantized max was
 * used instead.  NaN inputs are skipped (fmaxf semantics); an all-zero or
 * empty tensor gives 0.
 * ---------------------------------------------------------------------- */
float orc_amax(const uint16_t* x, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        const float a = fabsf(orc_bf16_to_f32(x[i]));
        if (a > m) m = a; /* a NaN compares false and is skipped */
    }
    return m;
}

/* ------------------------------------------------------------------------
 * Other input types.  [CMP] csrc/kernels/fp8/quantize.cuh, quant_in_traits
 * (bf16, fp16 and fp32 inputs, each widened to fp32 before the max and the
 * multiply) and ops/fp8.py quantize ("bf16/fp16/fp32"); [LOG1] "templated
 * on input type".  IEEE binary16 (the spec, not the pages): sign, 5-bit
 * exponent with bias 15, 10-bit fraction; exponent 0 is subnormal with
 * spacing 2^-24; exponent 31 is infinity (fraction 0) or NaN.  Every
 * binary16 value is exact in fp32.
 * in_type: 0 bf16 bits, 1 fp16 bits, 2 fp32.
 * ---------------------------------------------------------------------- */
float orc_f16_to_f32(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 0x1F, frac = h & 0x3FF;
    float v;
    if (e == 0) v = ldexpf((float)frac, -24);
    else if (e == 31) v = frac ? NAN : INFINITY;
    else v = ldexpf((float)(1024 + frac), e - 25);
    return sign ? -v : v;
}

static float in_value(const void* x, int64_t i, int in_type)
{
    if (in_type == 0) return orc_bf16_to_f32(((const uint16_t*)x)[i]);
    if (in_type == 1) return orc_f16_to_f32(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

float orc_amax_in(const void* x, int64_t n, int in_type)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        const float a = fabsf(in_value(x, i, in_type));
        if (a > m) m = a; /* NaN skipped */
    }
    return m;
}

/* ------------------------------------------------------------------------
 * Scale from an amax peak.  [CMP] astrai/extension/fp8.py,
 * FP8Recipe.scale_from_history, and quantize.cuh publish_amax: the scale is
 * the quantization step (peak / FP8_MAX) / 2^margin, clamped below at
 * 1e-12, computed as two IEEE fp32 divisions.
 * ---------------------------------------------------------------------- */
float orc_scale_from_peak(float peak, int fmt, int margin)
{
    const float fmax = (float)orc_fmt_max(fmt);
    const float pow2 = ldexpf(1.0f, margin);
    const float t = peak / fmax;
    const float s = t / pow2;
    return s > 1e-12f ? s : 1e-12f;
}

/* The multiplier a quantize applies: the fp32 reciprocal of the step.
 * [CMP] fp8.py passes scale.reciprocal() to quantize, and the kernel
 * multiplies each element by it. */
float orc_multiplier(float s) { return 1.0f / s; }

/* ------------------------------------------------------------------------
 * Quantize: q_i = encode(fp32(x_i * m)), m = fp32(1 / s).
 * [CMP] quantize.cuh, fp8_quantize_kernel (multiply, then convert).
 * ---------------------------------------------------------------------- */
void orc_quantize(const uint16_t* x, int64_t n, int fmt, float s, uint8_t* out)
{
    const float m = orc_multiplier(s);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float prod = orc_bf16_to_f32(x[i]) * m;
        out[i] = orc_encode(prod, fmt);
    }
}

/* The same quantize for any input type (widened to fp32 first). */
void orc_quantize_in(const void* x, int64_t n, int in_type, int fmt, float s, uint8_t* out)
{
    const float m = orc_multiplier(s);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(in_value(x, i, in_type) * m, fmt);
}

/* ------------------------------------------------------------------------
 * Scaled GEMM.  [CMP] ops/fp8.py mm_fp8 and csrc/kernels/fp8/common.h
 * (operand layout tags, batch strides where 0 broadcasts) and epilogue.cuh
 * (accumulate, apply the combined scale, add the bias, round once to bf16).
 *
 *   out[b,i,j] = bf16( (sum_k A[b,i,k] * B[b,k,j]) * fp32(sa*sb) + bias[j] )
 *
 * A is M x K: stored [M][K] with row stride lda (trans_a = 0) or [K][M]
 * (trans_a = 1).  B is K x N: stored [K][N] (trans_b = 0) or [N][K]
 * (trans_b = 1, the nn.Linear weight).  The sum, the scale product and the
 * bias add are carried in fp64; the result rounds once to bf16.
 * out is contiguous [batch][M][N].
 * ---------------------------------------------------------------------- */
static float g_dec[2][256];
static int g_dec_ready = 0;

static void dec_tables(void)
{
    if (g_dec_ready) return;
    for (int f = 0; f < 2; ++f)
        for (int c = 0; c < 256; ++c) g_dec[f][c] = orc_decode((uint8_t)c, f);
    g_dec_ready = 1;
}

static double gemm_one(const uint8_t* A, const uint8_t* B, int fmt, int trans_a,
                       int trans_b, int64_t K, int64_t lda, int64_t ldb,
                       int64_t b, int64_t i, int64_t j, int64_t stride_a,
                       int64_t stride_b)
{
    const uint8_t* Ab = A + b * stride_a;
    const uint8_t* Bb = B + b * stride_b;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const uint8_t ca = trans_a ? Ab[k * lda + i] : Ab[i * lda + k];
        const uint8_t cb = trans_b ? Bb[j * ldb + k] : Bb[k * ldb + j];
        acc += (double)g_dec[fmt][ca] * (double)g_dec[fmt][cb];
    }
    return acc;
}

static uint16_t epilogue_one(double acc, float s, const uint16_t* bias, int64_t j)
{
    double y = acc * (double)s;
    if (bias) y += (double)orc_bf16_to_f32(bias[j]);
    return orc_bf16_from_f64(y);
}

/* Magnitude statistics of one output's products p_k = A[b,i,k] * B[b,k,j]
 * (exact in fp64): *absdot = sum_k |p_k|, *groupmax = sum over the aligned
 * groups k in [8g, 8g + 8) of max_k |p_k|.  Tolerance tooling: they scale
 * the rounding a correct fp32-accumulating kernel may carry. */
static void dot_stats(const uint8_t* A, const uint8_t* B, int fmt, int trans_a, int trans_b,
                      int64_t K, int64_t lda, int64_t ldb, int64_t b, int64_t i, int64_t j,
                      int64_t stride_a, int64_t stride_b, double* absdot, double* groupmax)
{
    const uint8_t* Ab = A + b * stride_a;
    const uint8_t* Bb = B + b * stride_b;
    double sum = 0.0, gsum = 0.0, gmax = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const uint8_t ca = trans_a ? Ab[k * lda + i] : Ab[i * lda + k];
        const uint8_t cb = trans_b ? Bb[j * ldb + k] : Bb[k * ldb + j];
        const double p = fabs((double)g_dec[fmt][ca] * (double)g_dec[fmt][cb]);
        sum += p;
        if (p > gmax) gmax = p;
        if (k % 8 == 7 || k == K - 1) {
            gsum += gmax;
            gmax = 0.0;
        }
    }
    *absdot = sum;
    *groupmax = gsum;
}

void orc_gemm(const uint8_t* A, const uint8_t* B, int fmt, int trans_a, int trans_b,
              int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
              int64_t batch, int64_t stride_a, int64_t stride_b, float sa, float sb,
              const uint16_t* bias, uint16_t* out)
{
    dec_tables();
    const float s = sa * sb; /* fp32 product of the two steps */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                const double acc = gemm_one(A, B, fmt, trans_a, trans_b, K, lda, ldb,
                                            b, i, j, stride_a, stride_b);
                out[(b * M + i) * N + j] = epilogue_one(acc, s, bias, j);
            }
}

/* The same definition evaluated only at listed output coordinates, for
 * parity at sizes where the full product is too slow on the CPU.  Also
 * returns, per sample, sum_k |A*B| * |s| in absdot and the aligned 8-k group
 * maxima's sum times |s| in groupmax (both nullable; see dot_stats). */
void orc_gemm_sampled(const uint8_t* A, const uint8_t* B, int fmt, int trans_a,
                      int trans_b, int64_t K, int64_t lda, int64_t ldb,
                      int64_t stride_a, int64_t stride_b, float sa, float sb,
                      const uint16_t* bias, int64_t n_samples, const int64_t* sb_idx,
                      const int64_t* si_idx, const int64_t* sj_idx, uint16_t* out,
                      double* absdot, double* groupmax)
{
    dec_tables();
    const float s = sa * sb;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_samples; ++t) {
        const double acc = gemm_one(A, B, fmt, trans_a, trans_b, K, lda, ldb, sb_idx[t],
                                    si_idx[t], sj_idx[t], stride_a, stride_b);
        out[t] = epilogue_one(acc, s, bias, sj_idx[t]);
        if (absdot || groupmax) {
            double ad, gm;
            dot_stats(A, B, fmt, trans_a, trans_b, K, lda, ldb, sb_idx[t], si_idx[t], sj_idx[t],
                      stride_a, stride_b, &ad, &gm);
            if (absdot) absdot[t] = ad * fabs((double)s);
            if (groupmax) groupmax[t] = gm * fabs((double)s);
        }
    }
}

/* Sum of |A*B| * |s| for every output (same indexing as orc_gemm): the
 * scale of the fp32 rounding error of any summation order (Higham's bound
 * for a dot product is gamma_n times this sum). */
void orc_gemm_absdot(const uint8_t* A, const uint8_t* B, int fmt, int trans_a, int trans_b,
                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t batch, int64_t stride_a, int64_t stride_b, float sa, float sb,
                     double* out)
{
    dec_tables();
    const float s = sa * sb;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                double ad, gm;
                dot_stats(A, B, fmt, trans_a, trans_b, K, lda, ldb, b, i, j, stride_a,
                          stride_b, &ad, &gm);
                out[(b * M + i) * N + j] = ad * fabs((double)s);
            }
}

/* Sum over the aligned groups of 8 consecutive k (k in [8g, 8g + 8)) of the
 * group's largest |A*B|, times |s|, for every output (same indexing as
 * orc_gemm).  This is the scale of the cut that the fp8 matrix instructions
 * of gfx950 make when they add a group's products aligned to its largest one
 * (at most 7 products per group lose less than 2^-13 of that product each);
 * the GEMM tolerance's error bound is built from it and orc_gemm_absdot. */
void orc_gemm_groupmax(const uint8_t* A, const uint8_t* B, int fmt, int trans_a, int trans_b,
                       int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                       int64_t batch, int64_t stride_a, int64_t stride_b, float sa, float sb,
                       double* out)
{
    dec_tables();
    const float s = sa * sb;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                double ad, gm;
                dot_stats(A, B, fmt, trans_a, trans_b, K, lda, ldb, b, i, j, stride_a,
                          stride_b, &ad, &gm);
                out[(b * M + i) * N + j] = gm * fabs((double)s);
            }
}

/* orc_gemm_absdot and orc_gemm_groupmax in one pass over the products. */
void orc_gemm_stats(const uint8_t* A, const uint8_t* B, int fmt, int trans_a, int trans_b,
                    int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                    int64_t batch, int64_t stride_a, int64_t stride_b, float sa, float sb,
                    double* absdot, double* groupmax)
{
    dec_tables();
    const float s = sa * sb;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                double ad, gm;
                dot_stats(A, B, fmt, trans_a, trans_b, K, lda, ldb, b, i, j, stride_a,
                          stride_b, &ad, &gm);
                absdot[(b * M + i) * N + j] = ad * fabs((double)s);
                groupmax[(b * M + i) * N + j] = gm * fabs((double)s);
            }
}

/* ------------------------------------------------------------------------
 * Bias gradient: db[j] = bf16( sum_m g[m, j] ), the column sum of the bf16
 * output gradient, carried in fp64 and rounded once.  [CMP] fp8.py,
 * _LinearFp8.backward (grad_b is the sum of g over rows, cast to bf16).
 * ---------------------------------------------------------------------- */
void orc_colsum(const uint16_t* g, int64_t M, int64_t N, uint16_t* db)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0;
        for (int64_t m = 0; m < M; ++m) acc += (double)orc_bf16_to_f32(g[m * N + j]);
        db[j] = orc_bf16_from_f64(acc);
    }
}

/* ------------------------------------------------------------------------
 * GEMM with an fp8 bias and / or an fp8 output.  [CMP] ops/fp8.py, the
 * removed fp8_gemm custom op (out_dtype 1: an fp8 E4M3 output that needs
 * out_scale, the quantization step of the output); [LOG1] the FP8Params
 * bias becomes untyped with a bias_scale beside it (no scale: a bf16 bias;
 * a scale: fp8 codes, dequantized after the operand scaling and before any
 * output quantization).
 *
 *   bv[j] = bias_fp8 ? fp32( dec_fmt(bias[j]) * bias_scale ) : bf16 bias[j]
 *   y     = (sum_k A[b,i,k] * B[b,k,j]) * fp32(sa*sb) + bv[j]     (fp64)
 *   out   = bf16(y)                                  out_type 0
 *           enc_fo( fp32( fp32(y) * fp32(1/out_scale) ) )   out_type 1, 2
 * with fo = E4M3 for out_type 1 and E5M2 for out_type 2; the codes are the
 * cast's: nearest even, saturating at the format's largest value.  The fp8
 * bias uses the operands' format.  Evaluated at listed coordinates (all of
 * them for a full product); out holds uint16 bf16 bits or uint8 codes; yval
 * (nullable) receives y, absdot and groupmax (nullable) the statistics of
 * dot_stats times |s|.
 * ---------------------------------------------------------------------- */
uint8_t orc_out_code(double y, int out_fmt, float out_scale)
{
    const float r = orc_multiplier(out_scale); /* fp32(1 / out_scale) */
    const float prod = (float)y * r;           /* two fp32 roundings */
    return orc_encode(prod, out_fmt);
}

void orc_out_code_array(const double* y, int64_t n, int out_fmt, float out_scale,
                        uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_out_code(y[i], out_fmt, out_scale);
}

void orc_gemm_ex(const uint8_t* A, const uint8_t* B, int fmt, int trans_a, int trans_b,
                 int64_t K, int64_t lda, int64_t ldb, int64_t stride_a, int64_t stride_b,
                 float sa, float sb, const void* bias, int bias_fp8, float bias_scale,
                 int out_type, float out_scale, int64_t n_samples, const int64_t* sb_idx,
                 const int64_t* si_idx, const int64_t* sj_idx, void* out, double* yval,
                 double* absdot, double* groupmax)
{
    dec_tables();
    const float s = sa * sb;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_samples; ++t) {
        const int64_t b = sb_idx[t], i = si_idx[t], j = sj_idx[t];
        const double acc = gemm_one(A, B, fmt, trans_a, trans_b, K, lda, ldb, b, i, j,
                                    stride_a, stride_b);
        double y = acc * (double)s;
        if (bias) {
            float bv;
            if (bias_fp8)
                bv = g_dec[fmt][((const uint8_t*)bias)[j]] * bias_scale; /* fp32 product */
            else
                bv = orc_bf16_to_f32(((const uint16_t*)bias)[j]);
            y += (double)bv;
        }
        if (out_type == 0)
            ((uint16_t*)out)[t] = orc_bf16_from_f64(y);
        else
            ((uint8_t*)out)[t] = orc_out_code(y, out_type == 1 ? FMT_E4M3 : FMT_E5M2, out_scale);
        if (yval) yval[t] = y;
        if (absdot || groupmax) {
            double ad, gm;
            dot_stats(A, B, fmt, trans_a, trans_b, K, lda, ldb, b, i, j, stride_a, stride_b,
                      &ad, &gm);
            if (absdot) absdot[t] = ad * fabs((double)s);
            if (groupmax) groupmax[t] = gm * fabs((double)s);
        }
    }
}
