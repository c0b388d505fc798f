// Device (gfx950) side of the seeded input generator, plus a plain copy kernel
// used as the measured HBM ceiling and as the byte-counter calibration.
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

__global__ void synth_fill_kernel(uint32_t seed, uint32_t key1, uint64_t start, int64_t n,
                                  float scale, int mode, void* out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = synth_value(seed, key1, start + (uint64_t)i, scale);
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
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Plain copy of n16 16-byte vectors.  Each block copies runs of 8 * 256
// vectors (8 loads in flight per lane, then 8 stores), with nontemporal hints:
// the fastest of the simple copy variants measured on MI355X.
__global__ __launch_bounds__(256) void synth_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n16) {
    constexpr int U = 8;
    const int64_t per_block = 256 * U;
    const int64_t nblk = (n16 + per_block - 1) / per_block;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t base = blk * per_block + threadIdx.x;
        u32x4 w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * 256;
            if (i < n16) w[k] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * 256;
            if (i < n16) __builtin_nontemporal_store(w[k], dst + i);
        }
    }
}

// Read-only stream of n16 vectors (8 nontemporal loads in flight per lane); one
// word per thread is written so the loads are not removed.
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
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Write-only stream of n16 vectors (4 stores per lane per iteration).
__global__ __launch_bounds__(256) void synth_write_kernel(u32x4* __restrict__ dst, int64_t n16) {
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < n16; b += stride * U) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = b + k * stride;
            if (i < n16) dst[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
        }
    }
}

// Read-only stream over ns buffers at the same offsets (the access pattern of
// a reduction over ns contributions): n16 vectors of 16 bytes from each.
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
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
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

// Copies nbytes (a multiple of 16; both pointers 16-byte aligned).
int synth_copy_dev(const void* src, void* dst, int64_t nbytes, int grid, hipStream_t stream) {
    if (nbytes < 0 || (nbytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    if (nbytes == 0) return 0;
    const int block = 256;
    const int64_t n16 = nbytes / 16;
    const int g = grid > 0 ? grid : grid_for(n16, block);
    hipLaunchKernelGGL(synth_copy_kernel, dim3(g), dim3(block), 0, stream,
                       (const u32x4*)src, (u32x4*)dst, n16);
    return (int)hipGetLastError();
}

// Read-only probe over nbytes of src (a multiple of 16, 16-byte aligned).
// `out` must hold grid * 256 words; grid <= 0 picks 8 blocks per CU.
int synth_read_dev(const void* src, void* out, int64_t nbytes, int grid, hipStream_t stream) {
    if (nbytes <= 0 || (nbytes & 15) || ((uintptr_t)src & 15) || !out) return -1;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int g = grid > 0 ? grid : cus * 8;
    hipLaunchKernelGGL(synth_read_kernel, dim3(g), dim3(256), 0, stream, (const u32x4*)src,
                       (unsigned*)out, nbytes / 16);
    return (int)hipGetLastError();
}

// Multi-buffer read probe: reads nbytes (a multiple of 16) from each of the ns
// buffers in srcs (host array of device pointers, 16-byte aligned, ns <= 256).
// `out` must hold grid * 256 words; grid <= 0 picks 16 blocks per CU.
int synth_read_streams_dev(const void* const* srcs, int ns, int64_t nbytes, void* out, int grid,
                           hipStream_t stream) {
    if (ns < 1 || ns > 256 || nbytes <= 0 || (nbytes & 15) || !out || !srcs) return -1;
    StreamPtrs ps{};
    for (int k = 0; k < ns; ++k) {
        if (!srcs[k] || ((uintptr_t)srcs[k] & 15)) return -1;
        ps.p[k] = (const u32x4*)srcs[k];
    }
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int g = grid > 0 ? grid : cus * 16;
    hipLaunchKernelGGL(synth_read_streams_kernel, dim3(g), dim3(256), 0, stream, ps, ns, nbytes / 16,
                       (unsigned*)out);
    return (int)hipGetLastError();
}

// Write-only probe over nbytes of dst; grid <= 0 picks 2 blocks per CU.
int synth_write_dev(void* dst, int64_t nbytes, int grid, hipStream_t stream) {
    if (nbytes <= 0 || (nbytes & 15) || ((uintptr_t)dst & 15)) return -1;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const int g = grid > 0 ? grid : cus * 2;
    hipLaunchKernelGGL(synth_write_kernel, dim3(g), dim3(256), 0, stream, (u32x4*)dst, nbytes / 16);
    return (int)hipGetLastError();
}

}  // extern "C"
