/*
 * fp8_oracle.c -- plain CPU oracle for the per-output-channel scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  It shares no
 * source, header, table or helper with the HIP library in
 * fp8_gemm_channel_amd/, and neither side includes or links the other.
 *
 * What it computes, written out as its definition (no blocking, no fusion, no
 * reordering beyond what the definition states):
 *
 *     y[m,n] = bf16_rne( ( sum_{k<K} dec(x[m,k]) * dec(w[n,k]) ) * scale[n] )
 *
 *   x     [M,K] FP8 E4M3 codes, row-major ("activation")
 *   w     [N,K] FP8 E4M3 codes, row-major ("weight", one row per output channel)
 *   scale [N]   fp32, one dequantisation factor per output channel
 *   y     [M,N] bf16 bit patterns, row-major
 *
 * Sources on the pages (kernelbench.com model pages; cells named by the kernel
 * they audit):
 *   - fp8 x fp8 products summed with fp32 accumulation, written as bf16:
 *     "DeepSeek V4 Flash (0731)" page, CUTLASS 3.x SM90 fp8 GEMM cell.
 *   - the per-output-channel scale is applied to the accumulated sum, once,
 *     before the bf16 store: "Kimi K3 (256k)" page, SM120 warp-specialised FP8
 *     GEMM cell; same page, SM100 persistent-TMA Triton cell (dequant scale in
 *     the fp32 epilogue); "Claude Fable 5" page, Triton split-K cell.
 *   - correctness is judged against a float reference matmul of the same
 *     operands: "Kimi K3 (256k)" page, SM90 WGMMA cell.
 *   - zero bytes appended along K add exactly nothing to each dot product:
 *     "Kimi K3 (256k)" page, SM100 persistent-TMA Triton cell; "Claude Fable 5"
 *     page, CUTLASS 4.0 SM100 cell.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *   - "E4M3" is the OCP FP8 E4M3 format without infinities (torch.float8_e4m3fn):
 *     bias 7, largest finite 448, codes 0x7F and 0xFF are NaN.
 *   - The oracle accumulates in fp64 instead of fp32.  Every E4M3 value is an
 *     integer multiple of 2^-9 with magnitude at most 448 = 229376 * 2^-9, so
 *     every product is an integer multiple of 2^-18 below 2^18 in magnitude and
 *     every partial sum stays an exact fp64 integer multiple of 2^-18 while
 *     K <= 171196 (K * 229376^2 < 2^53).  In that range the fp64 sum is the
 *     exact sum, independent of summation order.  Only the scale product and
 *     the bf16 conversion round.
 *   - The product acc * scale is formed in fp64 (one rounding) and rounded
 *     directly from fp64 to bf16, to nearest, ties to even.  NaN stays NaN
 *     (0x7FC0); magnitudes at or beyond the bf16 overflow threshold become inf.
 *   - K = 0 gives the empty sum, +0.
 *
 * The general entry points (oracle_fp8_gemm_epilogue and _at) also compute
 *
 *     y[m,n] = bf16_rne( act( acc[m,n] * scale[n] + bias[n] ) )
 *
 * for either FP8 format on either operand.  Sources on the pages: the CUTLASS
 * epilogue that applies the per-output-channel scale is the per-column
 * linear-combination + per-column bias + elementwise-activation kind
 * ("DeepSeek V4 Flash (0731)" page, CUTLASS 3.x SM90 fp8 GEMM cell); the
 * f8f6f4 tensor-core kind takes either FP8 format ("Claude Fable 5" page,
 * tcgen05 fp8 GEMM cell).  Readings (listed in the design doc):
 *   - "E5M2" is the OCP FP8 E5M2 format (torch.float8_e5m2): bias 15, largest
 *     finite 57344, exponent 31 holds +-inf (mantissa 0) and NaN.
 *   - The sum is exact for every K: each finite code is an integer multiple of
 *     2^-16 (the smallest E5M2 subnormal; E4M3 values are multiples of 2^-9),
 *     each product an integer multiple of 2^-32 below 2^64 in magnitude, and
 *     the products are added as 128-bit integers, then rounded once to fp64
 *     (to nearest, ties to even).  A NaN operand, or an infinite operand times
 *     zero, makes the sum NaN; infinite products of both signs make it NaN;
 *     otherwise an infinite product makes it that infinity (IEEE rules for a
 *     sum of exact products).
 *   - z = acc * scale[n] + bias[n] is formed in fp64 (bias 0 when absent).
 *   - Activations, in fp64: none; ReLU  max(z, 0);  SiLU  z / (1 + e^-z);
 *     GELU in its tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
 *     (Hendrycks and Gimpel).  At z = +-inf each takes its limit (+inf for
 *     z = +inf; 0 for ReLU at -inf, -0 for SiLU and GELU); NaN stays NaN.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Decode one FP8 E4M3 (OCP, no infinities) code to double.
 * s = sign bit, e = 4-bit biased exponent, m = 3-bit mantissa.
 *   e = 15, m = 7 : NaN
 *   e = 0         : subnormal, m * 2^-9
 *   otherwise     : (8 + m) * 2^(e - 10)  (= (1 + m/8) * 2^(e - 7))           */
double oracle_e4m3_to_double(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp((double)(8 + m), e - 10);
    return s ? -mag : mag;
}

/* Round a double to the nearest bf16 (8 exponent bits, bias 127, 7 stored
 * mantissa bits), ties to even, and return its bit pattern.
 * The value is split as |v| = f * 2^e with f in [0.5, 1).  The bf16 spacing at
 * that magnitude is 2^(e-1-7) for normal results and 2^-133 in the subnormal
 * range (e - 1 < -126).  q = |v| / spacing is exact (power-of-two scaling);
 * rint() under the default rounding mode rounds q to nearest, ties to even,
 * which is exactly the bf16 decision.  The bit pattern is then assembled from
 * the integer significand: a carry out of the significand (q rounding up to
 * 256) lands in the exponent field by plain addition.                         */
uint16_t oracle_double_to_bf16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    int e, unb;
    double q;
    uint32_t bits;

    if (isnan(v))
        return 0x7FC0u;
    if (isinf(v))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;

    (void)frexp(a, &e);        /* a = f * 2^e, 0.5 <= f < 1 */
    unb = e - 1;               /* unbiased exponent: 2^unb <= a < 2^(unb+1) */
    if (unb < -126) {
        /* bf16 subnormal range: spacing 2^-133, significand q in [0, 128] */
        q = rint(ldexp(a, 133));
        bits = (uint32_t)q;    /* q == 128 is exactly the smallest normal 0x0080 */
    } else {
        if (unb > 127)
            return (uint16_t)(sign | 0x7F80u);
        /* normal range: significand q in [128, 256] */
        q = rint(ldexp(a, 7 - unb));
        bits = ((uint32_t)(unb + 127) << 7) + ((uint32_t)q - 128u);
    }
    if (bits >= 0x7F80u)       /* rounded up past the largest finite value */
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | bits);
}

static int oracle_threads(int requested)
{
#ifdef _OPENMP
    return requested > 0 ? requested : omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

int oracle_max_threads(void)
{
    return oracle_threads(0);
}

static int bad_dims(int64_t M, int64_t N, int64_t K)
{
    return M < 0 || N < 0 || K < 0;
}

/* acc[m*N + n] = sum_k dec(x[m,k]) * dec(w[n,k]) in fp64 (exact, see header). */
int oracle_fp8_gemm_acc(const uint8_t *x, const uint8_t *w, int64_t M, int64_t N,
                        int64_t K, double *acc, int threads)
{
    double lut[256];
    int64_t m;
    int i;
    if (bad_dims(M, N, K))
        return 1;
    for (i = 0; i < 256; ++i)
        lut[i] = oracle_e4m3_to_double((uint8_t)i);
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads(threads))
    for (m = 0; m < M; ++m) {
        const uint8_t *xr = x + (size_t)m * (size_t)K;
        int64_t n, k;
        for (n = 0; n < N; ++n) {
            const uint8_t *wr = w + (size_t)n * (size_t)K;
            double s = 0.0;
            for (k = 0; k < K; ++k)
                s += lut[xr[k]] * lut[wr[k]];
            acc[(size_t)m * (size_t)N + (size_t)n] = s;
        }
    }
    return 0;
}

/* y[m*N + n] = bf16_rne(acc[m,n] * scale[n]): the full definition. */
int oracle_fp8_gemm_scaled(const uint8_t *x, const uint8_t *w, const float *scale,
                           uint16_t *y, int64_t M, int64_t N, int64_t K, int threads)
{
    double lut[256];
    int64_t m;
    int i;
    if (bad_dims(M, N, K))
        return 1;
    for (i = 0; i < 256; ++i)
        lut[i] = oracle_e4m3_to_double((uint8_t)i);
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads(threads))
    for (m = 0; m < M; ++m) {
        const uint8_t *xr = x + (size_t)m * (size_t)K;
        int64_t n, k;
        for (n = 0; n < N; ++n) {
            const uint8_t *wr = w + (size_t)n * (size_t)K;
            double s = 0.0;
            for (k = 0; k < K; ++k)
                s += lut[xr[k]] * lut[wr[k]];
            y[(size_t)m * (size_t)N + (size_t)n] =
                oracle_double_to_bf16_rne(s * (double)scale[n]);
        }
    }
    return 0;
}

/* The same definition evaluated only at `count` positions (m_idx[i], n_idx[i]);
 * out[i] receives the bf16 bits of y[m_idx[i], n_idx[i]].  Used to check large
 * outputs element by element on a sample.                                      */
int oracle_fp8_gemm_scaled_at(const uint8_t *x, const uint8_t *w, const float *scale,
                              int64_t M, int64_t N, int64_t K,
                              const int64_t *m_idx, const int64_t *n_idx, int64_t count,
                              uint16_t *out, int threads)
{
    double lut[256];
    int64_t i;
    int c;
    if (bad_dims(M, N, K) || count < 0)
        return 1;
    for (i = 0; i < count; ++i)
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N)
            return 1;
    for (c = 0; c < 256; ++c)
        lut[c] = oracle_e4m3_to_double((uint8_t)c);
#pragma omp parallel for schedule(static) num_threads(oracle_threads(threads))
    for (i = 0; i < count; ++i) {
        const uint8_t *xr = x + (size_t)m_idx[i] * (size_t)K;
        const uint8_t *wr = w + (size_t)n_idx[i] * (size_t)K;
        double s = 0.0;
        int64_t k;
        for (k = 0; k < K; ++k)
            s += lut[xr[k]] * lut[wr[k]];
        out[i] = oracle_double_to_bf16_rne(s * (double)scale[n_idx[i]]);
    }
    return 0;
}

/* Elementwise helpers exported for the oracle's own pins. */
void oracle_e4m3_decode_array(const uint8_t *codes, int64_t count, double *out)
{
    int64_t i;
    for (i = 0; i < count; ++i)
        out[i] = oracle_e4m3_to_double(codes[i]);
}

void oracle_bf16_rne_array(const double *v, int64_t count, uint16_t *out)
{
    int64_t i;
    for (i = 0; i < count; ++i)
        out[i] = oracle_double_to_bf16_rne(v[i]);
}

/* ------------------------------------------------ general formats, epilogue */

#define ORACLE_FMT_E4M3 0
#define ORACLE_FMT_E5M2 1
#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_SILU 2
#define ORACLE_ACT_GELU_TANH 3

/* Decode one FP8 E5M2 (OCP) code to double.
 * s = sign bit, e = 5-bit biased exponent, m = 2-bit mantissa.
 *   e = 31, m = 0 : +-inf;  e = 31, m != 0 : NaN
 *   e = 0         : subnormal, m * 2^-16
 *   otherwise     : (4 + m) * 2^(e - 17)  (= (1 + m/4) * 2^(e - 15))          */
double oracle_e5m2_to_double(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 2) & 0x1F;
    int m = code & 0x3;
    double mag;
    if (e == 31)
        return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0)
        mag = ldexp((double)m, -16);
    else
        mag = ldexp((double)(4 + m), e - 17);
    return s ? -mag : mag;
}

/* A code as an exact integer multiple of 2^-16.  Returns 0 for a finite code
 * (*units set, sign included), 1 for +inf, 2 for -inf, 3 for NaN.            */
static int oracle_code_units(uint8_t code, int fmt, int64_t *units)
{
    int s = code >> 7;
    int64_t u;
    if (fmt == ORACLE_FMT_E4M3) {
        int e = (code >> 3) & 0xF, m = code & 0x7;
        if (e == 15 && m == 7)
            return 3;
        u = e == 0 ? (int64_t)m << 7 : (int64_t)(8 + m) << (e + 6);
    } else {
        int e = (code >> 2) & 0x1F, m = code & 0x3;
        if (e == 31)
            return m ? 3 : (s ? 2 : 1);
        u = e == 0 ? (int64_t)m : (int64_t)(4 + m) << (e - 1);
    }
    *units = s ? -u : u;
    return 0;
}

/* Round a 128-bit integer to the nearest double, ties to even (exact below
 * 2^53; above, the bits shifted out decide against exactly one half).        */
static double oracle_i128_to_double(__int128 v)
{
    unsigned __int128 a = v < 0 ? -(unsigned __int128)v : (unsigned __int128)v;
    int len = 0, drop;
    unsigned __int128 t = a, q, rem, half;
    double d;
    while (t) {
        ++len;
        t >>= 1;
    }
    if (len <= 53) {
        d = (double)(uint64_t)a;
    } else {
        drop = len - 53;
        q = a >> drop;
        rem = a - (q << drop);
        half = (unsigned __int128)1 << (drop - 1);
        if (rem > half || (rem == half && (q & 1)))
            q += 1;                       /* may carry to 2^53: still exact */
        d = ldexp((double)(uint64_t)q, drop);
    }
    return v < 0 ? -d : d;
}

/* The activation of the epilogue, in fp64 (see the header). */
double oracle_activation(double z, int act)
{
    if (isnan(z))
        return z;
    switch (act) {
    case ORACLE_ACT_RELU:
        return z > 0.0 ? z : 0.0;
    case ORACLE_ACT_SILU:
        if (isinf(z))
            return z > 0.0 ? z : -0.0;
        return z / (1.0 + exp(-z));
    case ORACLE_ACT_GELU_TANH:
        if (isinf(z))
            return z > 0.0 ? z : -0.0;
        return 0.5 * z * (1.0 + tanh(sqrt(2.0 / 3.14159265358979323846) * (z + 0.044715 * z * z * z)));
    default:
        return z;
    }
}

/* Exact dot product of x row and w row (see the header), rounded to fp64. */
static double oracle_dot_exact(const uint8_t *xr, const uint8_t *wr, int64_t K, int xf, int wf)
{
    __int128 s = 0;
    int nan = 0, pinf = 0, ninf = 0;
    int64_t k;
    for (k = 0; k < K; ++k) {
        int64_t ux = 0, uw = 0;
        int cx = oracle_code_units(xr[k], xf, &ux);
        int cw = oracle_code_units(wr[k], wf, &uw);
        if (cx == 3 || cw == 3) {
            nan = 1;
        } else if (cx || cw) {
            /* an infinite factor: inf * 0 is NaN, otherwise a signed inf */
            int neg = ((xr[k] >> 7) ^ (wr[k] >> 7)) & 1;
            if ((cx == 0 && ux == 0) || (cw == 0 && uw == 0))
                nan = 1;
            else if (neg)
                ninf = 1;
            else
                pinf = 1;
        } else {
            s += (__int128)ux * (__int128)uw;
        }
    }
    if (nan || (pinf && ninf))
        return NAN;
    if (pinf)
        return INFINITY;
    if (ninf)
        return -INFINITY;
    return ldexp(oracle_i128_to_double(s), -32);
}

static double oracle_epilogue_value(double acc, float scale, const float *bias, int64_t n, int act)
{
    double z = acc * (double)scale + (bias ? (double)bias[n] : 0.0);
    return oracle_activation(z, act);
}

static int bad_formats(int xf, int wf, int act)
{
    return (xf != ORACLE_FMT_E4M3 && xf != ORACLE_FMT_E5M2) ||
           (wf != ORACLE_FMT_E4M3 && wf != ORACLE_FMT_E5M2) || act < 0 || act > 3;
}

/* y = bf16_rne(act(acc * scale + bias)) for any operand formats (header). */
int oracle_fp8_gemm_epilogue(const uint8_t *x, const uint8_t *w, int xf, int wf, const float *scale,
                             const float *bias, int act, uint16_t *y, int64_t M, int64_t N,
                             int64_t K, int threads)
{
    int64_t m;
    if (bad_dims(M, N, K) || bad_formats(xf, wf, act))
        return 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads(threads))
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n) {
            double acc = oracle_dot_exact(x + (size_t)m * (size_t)K, w + (size_t)n * (size_t)K, K, xf, wf);
            y[(size_t)m * (size_t)N + (size_t)n] =
                oracle_double_to_bf16_rne(oracle_epilogue_value(acc, scale[n], bias, n, act));
        }
    }
    return 0;
}

/* The same at `count` positions (m_idx[i], n_idx[i]). */
int oracle_fp8_gemm_epilogue_at(const uint8_t *x, const uint8_t *w, int xf, int wf, const float *scale,
                                const float *bias, int act, int64_t M, int64_t N, int64_t K,
                                const int64_t *m_idx, const int64_t *n_idx, int64_t count,
                                uint16_t *out, int threads)
{
    int64_t i;
    if (bad_dims(M, N, K) || count < 0 || bad_formats(xf, wf, act))
        return 1;
    for (i = 0; i < count; ++i)
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N)
            return 1;
#pragma omp parallel for schedule(static) num_threads(oracle_threads(threads))
    for (i = 0; i < count; ++i) {
        double acc = oracle_dot_exact(x + (size_t)m_idx[i] * (size_t)K, w + (size_t)n_idx[i] * (size_t)K, K,
                                      xf, wf);
        out[i] = oracle_double_to_bf16_rne(oracle_epilogue_value(acc, scale[n_idx[i]], bias, n_idx[i], act));
    }
    return 0;
}

void oracle_e5m2_decode_array(const uint8_t *codes, int64_t count, double *out)
{
    int64_t i;
    for (i = 0; i < count; ++i)
        out[i] = oracle_e5m2_to_double(codes[i]);
}

void oracle_activation_array(const double *z, int64_t count, int act, double *out)
{
    int64_t i;
    for (i = 0; i < count; ++i)
        out[i] = oracle_activation(z[i], act);
}
