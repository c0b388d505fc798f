// Device (gfx950) side of the seeded input generator, plus plain streaming
// probes (copy, read, write, multi-buffer read) that measure HBM ceilings; the
// copy is also the byte-counter calibration kernel.
//
// Same generator as the host side: Philox4x32 with 10 rounds, from its
// published definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC'11).  Element e of stream (seed, key1) uses counter
// (e mod 2^32, e / 2^32, 0, 0) and key (seed, key1); the top 52 bits of its
// first two output words give p = (k + 1/2) 2^-52, and the value is fp32 of
// the standard normal quantile at p (P. J. Acklam's rational approximation)
// times the standard deviation.  Modes: 0 fp32, 1 |fp32|, 2 bf16 bits (round
// to nearest even).
//
// Input generation only: nothing here is part of the shard-step library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

__device__ __forceinline__ uint64_t f64_bits(double x) { return (uint64_t)__double_as_longlong(x); }
__device__ __forceinline__ double bits_f64(uint64_t u) { return __longlong_as_double((long long)u); }

// The same fp64 operations, in the same order, as the host implementation
// (philox_host.c), so the bits agree: log from the 2 atanh series, square root
// by Newton steps on the reciprocal root, Acklam's normal quantile with both
// branches evaluated and one selected.
__device__ __forceinline__ double synth_log(double x) {
    const uint64_t u = f64_bits(x);
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

__device__ __forceinline__ double synth_sqrt(double a) {
    double y = bits_f64(0x5FE6EB50C7B537A9ull - (f64_bits(a) >> 1));
#pragma unroll
    for (int i = 0; i < 5; ++i) y = y * (1.5 - (0.5 * a) * (y * y));
    const double x = a * y;
    return x + 0.5 * y * (a - x * x);
}

__device__ __forceinline__ double synth_normal_quantile(double p) {
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

__device__ __forceinline__ float synth_value(uint32_t seed, uint32_t key1, uint64_t e,
                                             float scale) {
    uint32_t x0 = (uint32_t)e, x1 = (uint32_t)(e >> 32), x2 = 0u, x3 = 0u;
    uint32_t k0 = seed, k1 = key1;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint32_t lo0 = 0xD2511F53u * x0, hi0 = __umulhi(0xD2511F53u, x0);
        const uint32_t lo1 = 0xCD9E8D57u * x2, hi1 = __umulhi(0xCD9E8D57u, x2);
        const uint32_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
        x0 = y0; x1 = lo1; x2 = y2; x3 = lo0;
    }
    const uint64_t k = (((uint64_t)x1 << 32) | x0) >> 12;
    const double p = ((bits_f64(0x4330000000000000ull | k) - 0x1p52) + 0.5) * 0x1p-52;
    return (float)synth_normal_quantile(p) * scale;
}

// out[i] <- x in the mode's type: fp32, |fp32|, or bf16 bits (round to nearest even).
__device__ __forceinline__ void synth_store(void* out, int64_t i, float x, int mode) {
    if (mode == 0) {
        ((float*)out)[i] = x;
    } else if (mode == 1) {
        ((float*)out)[i] = __uint_as_float(__float_as_uint(x) & 0x7FFFFFFFu);
    } else {
        const uint32_t u = __float_as_uint(x);
        uint16_t b;
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) b = (uint16_t)((u >> 16) | 0x0040u);
        else b = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        ((uint16_t*)out)[i] = b;
    }
}

__global__ void synth_fill_kernel(uint32_t seed, uint32_t key1, uint64_t start, int64_t n,
                                  float scale, int mode, void* out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        synth_store(out, i, synth_value(seed, key1, start + (uint64_t)i, scale), mode);
}

// Pieces: out[place(dst_k + j)] = value(param_k + j) for j < len_k.  tab holds
// np + 1 rows {cum_k, dst_k, param_k} with cum_k = len_0 + ... + len_{k-1}; the
// last row is {total, 0, 0}.  Virtual index v in [0, total) belongs to the
// largest k with cum_k <= v (empty pieces are skipped that way).  place is the
// identity when ilv_P == 0; otherwise it puts shard index d where rank ilv_q's
// value sits in a rank-interleaved receive buffer of ilv_P ranks:
// ((d / 512) * ilv_P + ilv_q) * 512 + d mod 512.
__device__ __forceinline__ int64_t synth_place(int64_t d, int ilv_P, int ilv_q) {
    if (ilv_P == 0) return d;
    return ((d >> 9) * ilv_P + ilv_q) * 512 + (d & 511);
}

__global__ void synth_fill_pieces_kernel(uint32_t seed, uint32_t key1,
                                         const int64_t* __restrict__ tab, int np, float scale,
                                         int mode, void* out, int ilv_P, int ilv_q) {
    const int64_t total = tab[3 * np];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total; v += stride) {
        int lo = 0, hi = np - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tab[3 * mid] <= v) lo = mid; else hi = mid - 1;
        }
        const int64_t j = v - tab[3 * lo];
        synth_store(out, synth_place(tab[3 * lo + 1] + j, ilv_P, ilv_q),
                    synth_value(seed, key1, (uint64_t)(tab[3 * lo + 2] + j), scale), mode);
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming probes: one 16-byte vector per lane, one short block per tile and a
// grid that covers the data (blocks stride over the rest when the grid is
// capped) -- the launch shape that moves the most bytes per second on MI355X.
// The copy is also the byte-counter calibration kernel.
constexpr int64_t kProbeMaxGrid = (int64_t)1 << 23;

// Copy: 64-lane blocks and nontemporal loads and stores, the fastest copy shape
// measured (6.7 TB/s; 256-lane blocks: 6.5 with the hints, 6.3 without).
__global__ __launch_bounds__(64) void synth_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 64;
    for (int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// XOR of the 64 lanes' words, written by lane 0 to out[wave]: one word per
// wave keeps every load live without a barrier.
__device__ __forceinline__ void wave_xor_out(unsigned acc, unsigned* __restrict__ out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (unsigned)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

// Read-only stream of n16 vectors; out[4 * block + wave] = XOR of the words
// its wave loaded.  Reads alone go fastest as a grid-stride loop with 8
// nontemporal loads in flight per lane and 8 blocks per CU (7.0 TB/s against
// 6.6-6.7 for one short block per tile).
__global__ __launch_bounds__(256) void synth_read_kernel(const u32x4* __restrict__ src,
                                                         unsigned* __restrict__ out, int64_t n16) {
    constexpr int U = 8;
    const int64_t stride = (int64_t)gridDim.x * 256;
    unsigned acc = 0;
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < n16; b += stride * U) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = b + k * stride;
            if (i < n16) {
                const u32x4 w = __builtin_nontemporal_load(src + i);
                acc ^= w.x ^ w.y ^ w.z ^ w.w;
            }
        }
    }
    wave_xor_out(acc, out);
}

// Write-only stream of n16 vectors: dst[i] = {i, 1, 2, 3}.
__global__ __launch_bounds__(256) void synth_write_kernel(u32x4* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        dst[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
}

// Read-only stream over ns buffers at the same offsets (the access pattern of
// a reduction over ns contributions): n16 vectors of 16 bytes from each; out
// as for the single-buffer read.
struct StreamPtrs { const u32x4* p[256]; };
__global__ __launch_bounds__(256) void synth_read_streams_kernel(StreamPtrs ps, int ns, int64_t n16,
                                                                 unsigned* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    unsigned acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        int k = 0;
        for (; k + 8 <= ns; k += 8) {
            u32x4 w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = ps.p[k + j][i];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc ^= w[j].x ^ w[j].y ^ w[j].z ^ w[j].w;
        }
        for (; k < ns; ++k) {
            const u32x4 w = ps.p[k][i];
            acc ^= w.x ^ w.y ^ w.z ^ w.w;
        }
    }
    wave_xor_out(acc, out);
}

// Blocks of a probe over n16 vectors: one per 256 vectors, capped.
int64_t probe_grid(int64_t n16) {
    const int64_t g = (n16 + 255) / 256;
    return g < 1 ? 1 : (g < kProbeMaxGrid ? g : kProbeMaxGrid);
}

// Blocks of the single-buffer read probe: 8 per CU.
int64_t read_grid() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    return (int64_t)cus * 8;
}

int grid_for(int64_t n, int block) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
    int64_t want = (n + block - 1) / block;
    int64_t cap = (int64_t)cus * 16;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return (int)want;
}

}  // namespace

extern "C" {

// out[i] = value(start + i), i in [0, n), enqueued on `stream`.  Returns 0 or a
// HIP error code.
int synth_fill_dev(uint32_t seed, uint32_t key1, uint64_t start, int64_t n, float scale,
                   int mode, void* out, hipStream_t stream) {
    if (n < 0 || mode < 0 || mode > 2) return -1;
    if (n == 0) return 0;
    if (!out) return -1;
    const int block = 256;
    hipLaunchKernelGGL(synth_fill_kernel, dim3(grid_for(n, block)), dim3(block), 0, stream,
                       seed, key1, start, n, scale, mode, out);
    return (int)hipGetLastError();
}

// The pieces form of synth_fill_dev (see synth_fill_pieces_kernel): tab is a
// device array of np + 1 rows; the caller guarantees every placed index fits
// in out.  ilv_P = 0 places at dst_k + j; ilv_P > 0 places rank ilv_q's values
// in a rank-interleaved buffer of ilv_P ranks.  One launch for any number of
// pieces.
int synth_fill_dev_pieces(uint32_t seed, uint32_t key1, const int64_t* tab, int np, int64_t total,
                          float scale, int mode, void* out, int ilv_P, int ilv_q,
                          hipStream_t stream) {
    if (np < 0 || total < 0 || mode < 0 || mode > 2 || ilv_P < 0 || ilv_q < 0 ||
        (ilv_P > 0 && ilv_q >= ilv_P))
        return -1;
    if (np == 0 || total == 0) return 0;
    if (!tab || !out) return -1;
    const int block = 256;
    hipLaunchKernelGGL(synth_fill_pieces_kernel, dim3(grid_for(total, block)), dim3(block), 0,
                       stream, seed, key1, tab, np, scale, mode, out, ilv_P, ilv_q);
    return (int)hipGetLastError();
}

// Copies nbytes (a multiple of 16; both pointers 16-byte aligned).  grid <= 0
// covers the data (one block per 64 vectors, at most 2^25 blocks).
int synth_copy_dev(const void* src, void* dst, int64_t nbytes, int grid, hipStream_t stream) {
    if (nbytes < 0 || (nbytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    if (nbytes == 0) return 0;
    const int64_t n16 = nbytes / 16;
    int64_t g = grid > 0 ? grid : (n16 + 63) / 64;
    if (g > 4 * kProbeMaxGrid) g = 4 * kProbeMaxGrid;
    hipLaunchKernelGGL(synth_copy_kernel, dim3((unsigned)g), dim3(64), 0, stream,
                       (const u32x4*)src, (u32x4*)dst, n16);
    return (int)hipGetLastError();
}

// Words of `out` that either read probe over nbytes (per buffer) may write
// with grid <= 0: 4 per block (one per wave).
int64_t synth_probe_out_words(int64_t nbytes) {
    const int64_t a = probe_grid(nbytes / 16), b = read_grid();
    return 4 * (a > b ? a : b);
}

// Read-only probe over nbytes of src (a multiple of 16, 16-byte aligned).
// `out` must hold 4 * grid words (grid <= 0: 8 blocks per CU).
int synth_read_dev(const void* src, void* out, int64_t nbytes, int grid, hipStream_t stream) {
    if (nbytes <= 0 || (nbytes & 15) || ((uintptr_t)src & 15) || !out) return -1;
    const int64_t g = grid > 0 ? grid : read_grid();
    hipLaunchKernelGGL(synth_read_kernel, dim3((unsigned)g), dim3(256), 0, stream, (const u32x4*)src,
                       (unsigned*)out, nbytes / 16);
    return (int)hipGetLastError();
}

// Multi-buffer read probe: reads nbytes (a multiple of 16) from each of the ns
// buffers in srcs (host array of device pointers, 16-byte aligned, ns <= 256).
// `out` as for synth_read_dev.
int synth_read_streams_dev(const void* const* srcs, int ns, int64_t nbytes, void* out, int grid,
                           hipStream_t stream) {
    if (ns < 1 || ns > 256 || nbytes <= 0 || (nbytes & 15) || !out || !srcs) return -1;
    StreamPtrs ps{};
    for (int k = 0; k < ns; ++k) {
        if (!srcs[k] || ((uintptr_t)srcs[k] & 15)) return -1;
        ps.p[k] = (const u32x4*)srcs[k];
    }
    const int64_t g = grid > 0 ? grid : probe_grid(nbytes / 16);
    hipLaunchKernelGGL(synth_read_streams_kernel, dim3((unsigned)g), dim3(256), 0, stream, ps, ns,
                       nbytes / 16, (unsigned*)out);
    return (int)hipGetLastError();
}

// Write-only probe over nbytes of dst (a multiple of 16, 16-byte aligned).
int synth_write_dev(void* dst, int64_t nbytes, int grid, hipStream_t stream) {
    if (nbytes <= 0 || (nbytes & 15) || ((uintptr_t)dst & 15)) return -1;
    const int64_t g = grid > 0 ? grid : probe_grid(nbytes / 16);
    hipLaunchKernelGGL(synth_write_kernel, dim3((unsigned)g), dim3(256), 0, stream, (u32x4*)dst, nbytes / 16);
    return (int)hipGetLastError();
}

}  // extern "C"
