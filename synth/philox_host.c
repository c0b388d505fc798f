/*
 * Host (CPU) side of the seeded input generator.
 *
 * Counter-based generator: Philox4x32 with 10 rounds, written from its
 * published definition (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11): each round maps the
 * 128-bit counter (c0,c1,c2,c3) through two 32x32->64 multiplies by the
 * constants 0xD2511F53 and 0xCD9E8D57, with the round key (k0,k1) XORed into
 * the high halves; the key advances by the Weyl constants 0x9E3779B9 and
 * 0xBB67AE85 between rounds.
 *
 * Element e of stream (seed, key1) uses counter (e mod 2^32, e / 2^32, 0, 0)
 * and key (seed, key1).  The top 52 bits of its first two output words give a
 * uniform p = (k + 1/2) 2^-52 in (0, 1); the value is the standard normal
 * quantile at p (Acklam's rational approximation, relative error below
 * 1.15e-9), rounded to fp32 and multiplied by the standard deviation in fp32.
 * The quantile, its logarithm and square root use fp64 basic operations only,
 * in a fixed order, so the device implementation gives the same bits.  Modes:
 * 0 = fp32 value, 1 = |fp32 value|, 2 = bf16 bits of the value (round to
 * nearest even).
 *
 * This file holds input generation only; the device implementation lives in
 * philox_dev.hip and must produce identical bits.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static inline void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma GCC unroll 10
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    philox10(c, key[0], key[1]);
    memcpy(out, c, sizeof c);
}

static inline uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint64_t f64_bits(double x) { uint64_t u; memcpy(&u, &x, 8); return u; }
static inline double bits_f64(uint64_t u) { double x; memcpy(&x, &u, 8); return x; }

/* Natural logarithm of a normal x > 0 from basic operations only: x = 2^e * m
 * with m in [sqrt(1/2), sqrt(2)), log m = 2 atanh(s) = 2 (s + s^3/3 + s^5/5 + ...)
 * with s = (m - 1)/(m + 1), |s| < 0.172, summed to s^23 (relative error below
 * 1e-15).  Written out so that the host and the device give the same bits. */
static inline double synth_log(double x) {
    const uint64_t u = f64_bits(x);
    // the biased exponent as a double, exactly: 2^52 + b has b in its low bits
    const double e0 = (bits_f64(0x4330000000000000ull | ((u >> 52) & 0x7FF)) - 0x1p52) - 1023.0;
    const double m0 = bits_f64((u & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
    const int up = m0 > 1.4142135623730951;
    const double m = up ? m0 * 0.5 : m0, e = up ? e0 + 1.0 : e0;
    const double s = (m - 1.0) / (m + 1.0), s2 = s * s;
    double t = 1.0 / 23.0;
    t = t * s2 + 1.0 / 21.0; t = t * s2 + 1.0 / 19.0; t = t * s2 + 1.0 / 17.0;
    t = t * s2 + 1.0 / 15.0; t = t * s2 + 1.0 / 13.0; t = t * s2 + 1.0 / 11.0;
    t = t * s2 + 1.0 / 9.0; t = t * s2 + 1.0 / 7.0; t = t * s2 + 1.0 / 5.0;
    t = t * s2 + 1.0 / 3.0; t = t * s2 + 1.0;
    return e * 0.6931471805599453 + 2.0 * s * t;
}

/* Square root of a > 0 without division: five Newton steps on 1/sqrt(a) from
 * the halved-exponent estimate (the constant of Lomont's and Robertson's fast
 * inverse square root for doubles), then a * y and one Newton step on the root
 * (a few ulps; the same bits on the host and the device). */
static inline double synth_sqrt(double a) {
    double y = bits_f64(0x5FE6EB50C7B537A9ull - (f64_bits(a) >> 1));
#pragma GCC unroll 5
    for (int i = 0; i < 5; ++i) y = y * (1.5 - (0.5 * a) * (y * y));
    const double x = a * y;
    return x + 0.5 * y * (a - x * x);
}

/* Standard normal quantile at p in (0, 1): P. J. Acklam's rational
 * approximation (relative error below 1.15e-9), a rational function of p - 1/2
 * in the centre and of sqrt(-2 log p) in the tails (p < 0.02425 or
 * 1 - p < 0.02425). */
static inline double synth_normal_quantile(double p) {
    const double a1 = -3.969683028665376e+01, a2 = 2.209460984245205e+02,
                 a3 = -2.759285104469687e+02, a4 = 1.383577518672690e+02,
                 a5 = -3.066479806614716e+01, a6 = 2.506628277459239e+00;
    const double b1 = -5.447609879822406e+01, b2 = 1.615858368580409e+02,
                 b3 = -1.556989798598866e+02, b4 = 6.680131188771972e+01,
                 b5 = -1.328068155288572e+01;
    const double c1 = -7.784894002430293e-03, c2 = -3.223964580411365e-01,
                 c3 = -2.400758277161838e+00, c4 = -2.549732539343734e+00,
                 c5 = 4.374664141464968e+00, c6 = 2.938163982698783e+00;
    const double d1 = 7.784695709041462e-03, d2 = 3.224671290700398e-01,
                 d3 = 2.445134137142996e+00, d4 = 3.754408661907416e+00;
    // both branches are evaluated and one is selected (no branch, so the host
    // loop vectorizes); the tail's argument is kept in (0, 1/2] either way
    const double plow = 0.02425;
    const double pt = p < 0.5 ? p : 1.0 - p;
    const double q = synth_sqrt(-2.0 * synth_log(pt));
    const double xt = (((((c1 * q + c2) * q + c3) * q + c4) * q + c5) * q + c6) /
                      ((((d1 * q + d2) * q + d3) * q + d4) * q + 1.0);
    const double qc = p - 0.5, r = qc * qc;
    const double xc = (((((a1 * r + a2) * r + a3) * r + a4) * r + a5) * r + a6) * qc /
                      (((((b1 * r + b2) * r + b3) * r + b4) * r + b5) * r + 1.0);
    const int tail = (p < plow) | (p > 1.0 - plow);
    return tail ? (p < 0.5 ? xt : -xt) : xc;
}

/* Value of element e: a uniform p = (k + 1/2) 2^-52 from the top 52 bits of
 * the first two output words (never 0 or 1), mapped through the normal
 * quantile, rounded once to fp32 and scaled by the standard deviation. */
static inline float value_at(uint32_t seed, uint32_t key1, uint64_t e, float scale) {
    uint32_t c[4] = {(uint32_t)e, (uint32_t)(e >> 32), 0u, 0u};
    philox10(c, seed, key1);
    const uint64_t k = (((uint64_t)c[1] << 32) | c[0]) >> 12;
    const double p = ((bits_f64(0x4330000000000000ull | k) - 0x1p52) + 0.5) * 0x1p-52;  // exact
    return (float)synth_normal_quantile(p) * scale;
}

static inline uint16_t to_bf16_rne(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* Fill kernels over a range, one per output mode, each compiled for three
 * instruction sets (AVX-512, AVX2, baseline x86-64) and chosen at run time:
 * the loop over elements vectorizes, and the integer and fp32 operations give
 * the same bits at every width.  idx == NULL means element start + i. */
#define MODE_LOOPS(GEN)                                                                \
    if (mode == 0) {                                                                   \
        float* o = (float*)out;                                                        \
        for (int64_t i = 0; i < n; ++i) o[i] = GEN(i);                                 \
    } else if (mode == 1) {                                                            \
        float* o = (float*)out;                                                        \
        for (int64_t i = 0; i < n; ++i) o[i] = bits_f32(f32_bits(GEN(i)) & 0x7FFFFFFFu); \
    } else {                                                                           \
        uint16_t* o = (uint16_t*)out;                                                  \
        for (int64_t i = 0; i < n; ++i) o[i] = to_bf16_rne(GEN(i));                    \
    }
#define GEN_SEQ(i) value_at(seed, key1, start + (uint64_t)(i), scale)
#define GEN_IDX(i) value_at(seed, key1, (uint64_t)idx[i], scale)
#define RANGE_BODY                    \
    if (idx) { MODE_LOOPS(GEN_IDX) }  \
    else { MODE_LOOPS(GEN_SEQ) }
#define RANGE_ARGS uint32_t seed, uint32_t key1, uint64_t start, const int64_t* idx, int64_t n, \
                   float scale, int mode, void* out

__attribute__((target("avx512f,avx512dq,avx512vl,avx512bw")))
static void fill_range_avx512(RANGE_ARGS) { RANGE_BODY }
__attribute__((target("avx2")))
static void fill_range_avx2(RANGE_ARGS) { RANGE_BODY }
static void fill_range_base(RANGE_ARGS) { RANGE_BODY }

typedef void (*fill_range_fn)(RANGE_ARGS);

static fill_range_fn fill_range(void) {
    __builtin_cpu_init();
    if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512dq") &&
        __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512bw"))
        return fill_range_avx512;
    if (__builtin_cpu_supports("avx2")) return fill_range_avx2;
    return fill_range_base;
}

/* The range [0, n) in chunks, one thread per chunk. */
static void fill_chunks(uint32_t seed, uint32_t key1, uint64_t start, const int64_t* idx,
                        int64_t n, float scale, int mode, void* out) {
    const fill_range_fn f = fill_range();
    const int64_t chunk = (int64_t)1 << 16, esize = mode == 2 ? 2 : 4;
    const int64_t nch = (n + chunk - 1) / chunk;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t a = c * chunk, m = n - a < chunk ? n - a : chunk;
        f(seed, key1, start + (uint64_t)a, idx ? idx + a : NULL, m, scale, mode,
          (char*)out + a * esize);
    }
}

/* out[i] = value(start + i) for i in [0, n). */
int synth_fill_host(uint32_t seed, uint32_t key1, uint64_t start, int64_t n,
                    float scale, int mode, void* out) {
    if (n < 0 || mode < 0 || mode > 2 || (n > 0 && !out)) return -1;
    fill_chunks(seed, key1, start, NULL, n, scale, mode, out);
    return 0;
}

/* out[i] = value(idx[i]) for i in [0, n). */
int synth_fill_host_idx(uint32_t seed, uint32_t key1, const int64_t* idx, int64_t n,
                        float scale, int mode, void* out) {
    if (n < 0 || mode < 0 || mode > 2 || (n > 0 && (!out || !idx))) return -1;
    fill_chunks(seed, key1, 0, idx, n, scale, mode, out);
    return 0;
}

/* out[i] = the standard normal quantile at p[i] in (0, 1), in fp64 (for the
 * tests of the transform). */
void synth_normal_quantile_host(const double* p, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = synth_normal_quantile(p[i]);
}
