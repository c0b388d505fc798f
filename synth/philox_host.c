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
 * and key (seed, key1).  Its four output words give eight 16-bit halves h_j;
 * z = 2*sum(h_j) - 8*65535 is an even integer in [-524280, 524280], exact in
 * fp32, and the value is fp32(z) * scale with one correctly rounded multiply
 * (an Irwin-Hall approximation of a normal with the standard deviation folded
 * into scale).  Modes: 0 = fp32 value, 1 = |fp32 value|, 2 = bf16 bits of the
 * value (round to nearest even).
 *
 * This file holds input generation only; the device implementation lives in
 * philox_dev.hip and must produce identical bits.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static inline void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
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

static inline float value_at(uint32_t seed, uint32_t key1, uint64_t e, float scale) {
    uint32_t c[4] = {(uint32_t)e, (uint32_t)(e >> 32), 0u, 0u};
    philox10(c, seed, key1);
    int32_t s = 0;
    for (int i = 0; i < 4; ++i) s += (int32_t)(c[i] & 0xFFFFu) + (int32_t)(c[i] >> 16);
    int32_t z = 2 * s - 8 * 65535;
    return (float)z * scale;
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
