/*
 * CPU oracle for the fused Conv/MatMul -> BatchNorm -> activation operator.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library, and it never calls it.
 *
 * Every value is widened exactly to IEEE binary64 and every step is computed
 * in binary64 with plain loops, in the order the pages define the operator:
 * convolution, then a separate BatchNorm pass, then the residual add, then the
 * activation (the BN is *not* folded here; the fold exists only as the
 * self-check orc_fold_bn).  OpenMP splits independent outputs across threads;
 * no sum is split or reordered.
 *
 * Built with -ffp-contract=off so that no multiply is fused into an add.
 *
 * Sources (web pages; the section named is where the definition appears):
 *  [OPPL]  "OpenPPL算子融合深度解析：从图优化到推理性能提升" (OpenPPL operator
 *          fusion deep dive), codechina.net.
 *  [INFR]  discosf.com inference-fusion practice article (page titled
 *          "企业官网建设流程全解析").
 *  [RFC]   "RFC：自动融合: 扩展统一 Pattern Matcher 覆盖量化融合与 GMM/MM+激活",
 *          gitcode.com MindIE-SD issue 298.
 *  [FRT]   "FlashRT 跨层融合深度解析", sheratonhq.com.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Convolution: the definition of a zero-padded, strided 2-D convolution,     */
/* the operator [INFR] §3.3 computes (zero padding, optional bias):           */
/*   y[b][oh][ow][co] = sum_{r<kh} sum_{s<kw} sum_{ci<cin}                     */
/*       xpad[b][oh*sh + r][ow*sw + s][ci] * wt[co][r][s][ci]  (+ bias[co])    */
/* where xpad is x with ph zero rows above and below and pw zero columns on   */
/* each side.  NHWC x and y, OHWI weights.  xpad is never built: padded_row() */
/* gives its cin values at one position, the shared zero row outside x.       */
/* ------------------------------------------------------------------------ */
static const double *padded_row(const double *x, const double *zeros, int64_t h, int64_t w,
                                int64_t cin, int64_t ph, int64_t pw, int64_t b, int64_t i, int64_t j)
{
    const int64_t xi = i - ph, xj = j - pw;
    const int inside = xi >= 0 && xi < h && xj >= 0 && xj < w;
    return inside ? x + ((b * h + xi) * w + xj) * cin : zeros;
}

static double conv_point(int64_t h, int64_t w, int64_t cin, int64_t kh, int64_t kw,
                         int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                         const double *x, const double *zeros, const double *wt, const double *bias,
                         int64_t b, int64_t oh, int64_t ow, int64_t co)
{
    double sum = 0.0;
    for (int64_t r = 0; r < kh; ++r)
        for (int64_t s = 0; s < kw; ++s) {
            const double *xp = padded_row(x, zeros, h, w, cin, ph, pw, b, oh * sh + r, ow * sw + s);
            const double *wp = wt + ((co * kh + r) * kw + s) * cin;
            for (int64_t ci = 0; ci < cin; ++ci)
                sum += xp[ci] * wp[ci];
        }
    return bias ? sum + bias[co] : sum;
}

/* cin zeros: the value of xpad outside x */
static double *zero_row(int64_t cin)
{
    double *z = calloc((size_t)(cin > 0 ? cin : 1), sizeof(double));
    if (!z)
        abort();
    return z;
}

/* y[n][ho][wo][cout] = conv(x[n][h][w][cin], wt[cout][kh][kw][cin]) (+ bias). */
void orc_conv2d_nhwc(int64_t n, int64_t h, int64_t w, int64_t cin, int64_t cout,
                     int64_t kh, int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                     const double *x, const double *wt, const double *bias, double *y)
{
    const int64_t ho = (h + 2 * ph - kh) / sh + 1;
    const int64_t wo = (w + 2 * pw - kw) / sw + 1;
    double *zeros = zero_row(cin);
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n * ho; ++row) {
        const int64_t b = row / ho, oh = row % ho;
        for (int64_t ow = 0; ow < wo; ++ow)
            for (int64_t co = 0; co < cout; ++co)
                y[((b * ho + oh) * wo + ow) * cout + co] =
                    conv_point(h, w, cin, kh, kw, sh, sw, ph, pw, x, zeros, wt, bias, b, oh, ow, co);
    }
    free(zeros);
}

/* The same convolution evaluated only at the output pixels pts[i] = (n, ho, wo);
 * y is [npts][cout]. */
void orc_conv2d_nhwc_at(int64_t h, int64_t w, int64_t cin, int64_t cout,
                        int64_t kh, int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                        const double *x, const double *wt, const double *bias,
                        int64_t npts, const int64_t *pts, double *y)
{
    double *zeros = zero_row(cin);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i)
        for (int64_t co = 0; co < cout; ++co)
            y[i * cout + co] = conv_point(h, w, cin, kh, kw, sh, sw, ph, pw, x, zeros, wt, bias,
                                          pts[3 * i], pts[3 * i + 1], pts[3 * i + 2], co);
    free(zeros);
}

/* ------------------------------------------------------------------------ */
/* Matrix product y[m][n] = sum_k a[m][k] * b[n][k]  (a 1x1 convolution over  */
/* m tokens; b in the [out][in] layout of a linear layer).                    */
/* ------------------------------------------------------------------------ */
void orc_matmul_nt(int64_t m, int64_t n, int64_t k, const double *a, const double *b, double *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            const double *ap = a + i * k, *bp = b + j * k;
            for (int64_t p = 0; p < k; ++p)
                acc += ap[p] * bp[p];
            y[i * n + j] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* BatchNorm in inference mode, a separate per-channel pass:                  */
/*   z = gamma * (y - mean) / sqrt(var + eps) + beta                          */
/* [OPPL] §3.1 (the inference-time BN transform); [INFR] §2.1 (same form).    */
/* Rows are the N*H*W pixels (or tokens); c is the innermost (channel) index.  */
/* ------------------------------------------------------------------------ */
void orc_batchnorm(int64_t rows, int64_t c, const double *y, const double *gamma,
                   const double *beta, const double *mean, const double *var, double eps,
                   double *z)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t ch = 0; ch < c; ++ch) {
            const int64_t i = r * c + ch;
            z[i] = gamma[ch] * (y[i] - mean[ch]) / sqrt(var[ch] + eps) + beta[ch];
        }
}

/* z[r][ch] = y[r][ch] + bias[ch]  (the BiasAdd of a MatMul -> BiasAdd -> act chain). */
void orc_bias_add(int64_t rows, int64_t c, const double *y, const double *bias, double *z)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t ch = 0; ch < c; ++ch)
            z[r * c + ch] = y[r * c + ch] + bias[ch];
}

/* Residual add, [OPPL] §3.3 (Add absorbed as an epilogue): out = a + b. */
void orc_add(int64_t count, const double *a, const double *b, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = a[i] + b[i];
}

/* ReLU, [OPPL] §2.1 / §4.3: values not above zero become (+)0. */
void orc_relu(int64_t count, const double *in, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = in[i] > 0.0 ? in[i] : 0.0;
}

/* GELU, tanh form, [OPPL] §4.3 (epilogue activation type 2):
 *   gelu(u) = 0.5 u (1 + tanh( sqrt(2/pi) (u + 0.044715 u^3) ))
 * The page prints sqrt(2/pi) truncated to ten digits; it is evaluated here. */
void orc_gelu_tanh(int64_t count, const double *in, double *out)
{
    const double k0 = sqrt(2.0 / M_PI);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const double u = in[i];
        out[i] = 0.5 * u * (1.0 + tanh(k0 * (u + 0.044715 * u * u * u)));
    }
}

/* GELU, exact (erf) form, [RFC] §2.1 (the GELU type of the quantised MatMul +
 * GELU operator may be tanh or erf) and §2.4 (erf GELU as its own operator).
 * The pages do not print it; it is the Gaussian CDF form
 *   gelu(u) = u Phi(u) = 0.5 u (1 + erf(u / sqrt(2))) = 0.5 u erfc(-u / sqrt(2)),
 * evaluated through erfc, which keeps full relative precision in the negative
 * tail where 1 + erf cancels. */
void orc_gelu_erf(int64_t count, const double *in, double *out)
{
    const double r2 = 1.0 / sqrt(2.0);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const double u = in[i];
        out[i] = 0.5 * u * erfc(-u * r2);
    }
}

/* SiLU (swish), the gate of SwiGLU in [RFC] §2.2 - §2.4: silu(u) = u / (1 + e^-u). */
void orc_silu(int64_t count, const double *in, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const double u = in[i];
        out[i] = u / (1.0 + exp(-u));
    }
}

/* ------------------------------------------------------------------------ */
/* BN folding, used only as a self-check of the unfolded path.               */
/* [OPPL] §3.1: scale = gamma / sqrt(var + eps); W_new = W * scale per output */
/* channel; b_new = (b_conv - mean) * scale + beta; b_conv = 0 when the conv  */
/* has no bias.  [INFR] §2.1 derives the same closed form.                    */
/* w is [cout][kdim]; w_out and b_out are binary64.                          */
/* ------------------------------------------------------------------------ */
void orc_fold_bn(int64_t cout, int64_t kdim, const double *w, const double *conv_bias,
                 const double *gamma, const double *beta, const double *mean, const double *var,
                 double eps, double *w_out, double *b_out)
{
    for (int64_t c = 0; c < cout; ++c) {
        const double scale = gamma[c] / sqrt(var[c] + eps);
        const double bc = conv_bias ? conv_bias[c] : 0.0;
        for (int64_t j = 0; j < kdim; ++j)
            w_out[c * kdim + j] = w[c * kdim + j] * scale;
        b_out[c] = (bc - mean[c]) * scale + beta[c];
    }
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn") codec.                                             */
/* Format: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is */
/* subnormal (m * 2^-9); no infinities; S.1111.111 is NaN, so the largest     */
/* finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).                          */
/* Q(v): the nearest finite e4m3 value, ties to the code whose mantissa LSB   */
/* is 0 (the even code), magnitudes >= 448 saturate to 448 (the clamp a       */
/* quantised ReLU epilogue needs, [OPPL] §6.4).  The sign bit is kept, so     */
/* negative values that round to zero give 0x80.                              */
/* Implementation: a decode table of the 127 non-negative finite codes and a  */
/* search for the neighbours of |v|.                                          */
/* ------------------------------------------------------------------------ */
static double e4m3_mag(int code7)
{
    const int e = (code7 >> 3) & 0xF, m = code7 & 7;
    if (e == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

double orc_e4m3_to_double(int code)
{
    const int c = code & 0xFF;
    if ((c & 0x7F) == 0x7F)
        return NAN;
    const double mag = e4m3_mag(c & 0x7F);
    return (c & 0x80) ? -mag : mag;
}

static int e4m3_from_double(double v)
{
    static double table[127];
    static int ready = 0;
    if (!ready) {                       /* benign race: every thread writes the same values */
        for (int c = 0; c < 127; ++c)
            table[c] = e4m3_mag(c);
        ready = 1;
    }
    const int sign = signbit(v) ? 0x80 : 0;
    const double a = fabs(v);
    if (a >= table[126])
        return sign | 126;
    /* largest lo with table[lo] <= a (table is increasing; table[0] = 0) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (table[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    const double dlo = a - table[lo], dhi = table[hi] - a;
    int code;
    if (dlo < dhi)
        code = lo;
    else if (dhi < dlo)
        code = hi;
    else
        code = (lo & 1) ? hi : lo;      /* tie: the even code */
    return sign | code;
}

int orc_e4m3_from_double(double v) { return e4m3_from_double(v); }

void orc_e4m3_decode(int64_t count, const uint8_t *codes, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = orc_e4m3_to_double(codes[i]);
}

void orc_e4m3_encode(int64_t count, const double *v, uint8_t *codes)
{
    e4m3_from_double(0.0);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        codes[i] = (uint8_t)e4m3_from_double(v[i]);
}

/* ------------------------------------------------------------------------ */
/* bfloat16 storage rounding: the nearest bf16 value of a binary64 value,     */
/* ties to the even significand, in one step (never through binary32, whose  */
/* first rounding could move a value onto a bf16 tie: the double rounding of */
/* [OPPL] §6.2).  bf16 keeps binary32's exponent range and 8 significant     */
/* bits: a value in [2^e, 2^(e+1)) rounds to a multiple of 2^(e-7); below    */
/* 2^-126 the spacing stays 2^-133 (subnormals); a result of 2^128 or more   */
/* is infinite.  Returned widened back to binary64.                          */
/* ------------------------------------------------------------------------ */
static double bf16_round(double v)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    frexp(v, &e);                       /* |v| in [2^(e-1), 2^e) */
    int q = e - 8;                      /* spacing exponent: 8 significant bits */
    if (q < -133)
        q = -133;
    const double r = ldexp(nearbyint(ldexp(v, -q)), q);   /* exact scaling; RNE */
    if (fabs(r) >= ldexp(1.0, 128))
        return copysign(INFINITY, v);
    return r;
}

void orc_round_bf16(int64_t count, const double *in, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = bf16_round(in[i]);
}

/* Static output quantisation of fp32 values exactly as an fp32 epilogue takes
 * it: p = fp32(u * inv_scale) (one IEEE binary32 multiply, round to nearest
 * even), then code = Q(p).  [FRT] §3 (static-scale FP8 written by the
 * producing kernel's epilogue); [RFC] §3.4 (quantised MatMul + activation). */
void orc_quant_f32(int64_t count, const float *u, float inv_scale, uint8_t *codes)
{
    e4m3_from_double(0.0);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const float p = u[i] * inv_scale;
        codes[i] = (uint8_t)e4m3_from_double((double)p);
    }
}
