// Device (gfx950) side of the seeded input generator, plus plain streaming
// probes (copy, read, write, multi-buffer read) that measure HBM ceilings; the
// copy is also the byte-counter calibration kernel.
//
// Same generator as the host side: Philox4x32 with 10 rounds, from its
// published definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC'11).  Element e of stream (seed, key1) uses counter
// (e mod 2^32, e / 2^32, 0, 0) and key (seed, key1); the eight 16-bit halves of
// the four output words give z = 2*sum - 8*65535 (exact in fp32) and the value
// fp32(z) * scale.  Modes: 0 fp32, 1 |fp32|, 2 bf16 bits (round to nearest even).
//
// Input generation only: nothing here is part of the shard-step library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

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
    const int32_t s = (int32_t)((x0 & 0xFFFFu) + (x0 >> 16) + (x1 & 0xFFFFu) + (x1 >> 16) +
                                (x2 & 0xFFFFu) + (x2 >> 16) + (x3 & 0xFFFFu) + (x3 >> 16));
    const int32_t z = 2 * s - 8 * 65535;
    return (float)z * scale;
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
