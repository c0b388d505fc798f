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

// Plain 16-byte-per-lane copy: n16 vectors of 16 bytes.
__global__ void synth_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                  int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
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
                       (const uint4*)src, (uint4*)dst, n16);
    return (int)hipGetLastError();
}

}  // extern "C"
