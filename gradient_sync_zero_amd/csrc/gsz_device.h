// Device-side building blocks shared by the kernels of the shard step: vector
// types, launch constants, bf16 conversions, 16-byte loads and stores, the
// fixed-order block sum, the bucket-segment cursor and the XCD-aware block order.
//
// Every kernel of the library is HBM-bound streaming work (no contraction, so no
// MFMA): 16-byte loads and stores per lane, 64-wide wavefronts, and one short
// block per tile with the grid covering the data.  Blocks are dispatched in
// index order, so the lines in flight stay close together in the address space;
// on MI355X that moves 10-20% more bytes per second than long-running
// grid-stride blocks.  fp64 reductions run in a fixed order (wave shuffles, LDS,
// one partial per block, then fixed ranges of partials) so results are
// bit-reproducible.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gsz_internal.h"

#pragma clang fp contract(off)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kBlock = 256;
// The pack kernels' block: one wave per 1 KiB tile copied 2.7% faster than
// 256-lane blocks on 2 KiB tiles (7B share, MI355X).
constexpr int kPackBlock = 64;
// The fp32 accumulation buckets' block: 128 lanes, one group of 4 elements per
// lane per 512-element tile (3% faster than 64 lanes with two groups each).
constexpr int kF32Block = 128;
// AdamW: one wave per block and one tile of 256 elements (4 per lane) per
// block, with nontemporal hints on every access: 6% (7B share) to 10% (70B
// share) faster than 512-lane blocks of 512 elements per wave without them.
constexpr int kAdamBlock = 64;
constexpr int64_t kAdamTile = 4 * kAdamBlock;
// Dynamic LDS that AdamW's launches reserve and never touch: 13 KiB per block
// leaves room for 12 resident blocks per CU in gfx950's 160 KiB, against 32
// without it.  Fewer waves in flight over AdamW's eight streams ran 3-8% faster
// (7B share) and 5% faster (70B share); at 10 or fewer blocks per CU it slows
// down again.
constexpr size_t kAdamLdsBytes = 13 * 1024;
// The same occupancy cap for the lane-contiguous reduce (256-lane blocks):
// 32 KiB per block leaves 5 resident blocks per CU.  It pays where each
// element's contributions add up to 16 bytes or more (bf16 at P >= 8, fp32 at
// P >= 4): 3% faster at P=8 bf16 (7B share), 1.7% for fp32 contributions at
// P=8.  Below that the loads of one wave are too few to keep HBM busy with so
// few waves: P=2 and 3 ran 15-25% slower with the cap, so they launch without.
constexpr size_t kRedLcLdsBytes = 32 * 1024;
constexpr int kRedLcLdsMinBytes = 16;
// Work-items of one dispatch stay at or below 2^31 (the dispatch packet's grid
// size is a 32-bit count).  Grids are capped accordingly; bigger inputs make
// blocks stride over the remaining tiles.
constexpr int64_t kMaxWorkItems = (int64_t)1 << 31;
constexpr int64_t kMaxFlatGrid = kMaxWorkItems / kBlock;          // 2^23 blocks of 256
// MI355X dispatches block b of a grid to XCD b mod 8.  xcd_remap gives XCD x one
// contiguous range of logical blocks instead (a bijection on [0, G)): the
// reduce, which reads P buffers at the same offsets, runs 1.7-1.9% faster that
// way on the 7B and 70B shares; pack and AdamW run slower and keep the plain order.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t G) {
    const int64_t q = G / kXcds, rem = G % kXcds, x = b % kXcds;
    return x * q + (x < rem ? x : rem) + b / kXcds;
}
// Elements per block of the reductions (8 per lane).
constexpr int64_t kRedTile = 8 * kBlock;
static_assert(kRedTile == gsz::kRedElems && kMaxFlatGrid == gsz::kMaxRedGrid,
              "the workspace size assumes these grids");

template <typename T>
struct RankPtrsT { const T* p[GSZ_MAX_RANKS]; };
using RankPtrs = RankPtrsT<uint16_t>;
using RankPtrsF = RankPtrsT<float>;
struct PackPtrs { const uint16_t* p[gsz::kPackBatch]; };

// fp32 constants of the AdamW update, each rounded once from double on the host.
struct AdamScalars { float b1, omb1, b2, omb2, bc1, bc2, lr, eps, decay; };

// ----------------------------------------------------------- device utils --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Nontemporal forms, for bytes a kernel touches once: with the hint on both
// its loads and its stores a streaming kernel moves 2-10% more bytes per second
// on MI355X (the hint on one side alone changes little).
__device__ __forceinline__ u32x4 ld16_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x4 ldf4_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st16_nt(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stf4_nt(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st8_nt(uint16_t* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ f32x4 ldf4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void stf4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Raw buffer accesses through a resource descriptor built from a wave-uniform
// base: every lane then carries one 32-bit byte offset that all the buffers
// at the same position share, instead of a 64-bit address per buffer, and each
// access names its cache policy.  On MI355X, against 64-bit nontemporal global
// accesses (two builds alternating on the same buffers): the lane-contiguous
// reduce at P = 8 0.3-0.7% faster with nontemporal buffer loads and g stored
// with sc1; AdamW 0.4-2.0% faster on the 1.3B model and the 7B share and 5%
// on the 70B share, the pack 2.6%, the bf16 and fp32 accumulations 3.6% and
// 5.9% and the all-gather writer 3.4% (7B share) with nontemporal loads and
// nontemporal sc1 stores.  (In probes g stored with plain or nontemporal-only
// bits gained nothing; the burst reduce at P = 64 ran 1.4% slower with buffer
// loads, one descriptor per contribution and row, and the tile reduce at
// P = 64 0.2% slower, so both keep 64-bit addresses.)
// Offsets are below 2^31.  A descriptor's range runs from its base to its
// buffer's end (for a rank's pieces of an interleaved receive buffer, to at
// most (P - 1) * 512 elements past it), capped at 2^32 - 1 bytes; accesses past
// the range would read 0 and store nothing, and the kernels make none.  Word 3
// holds the format bits of a plain 32-bit raw buffer.
typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr int kBufWord3 = 0x00020000;
// Cache-policy operand of the buffer builtins: bit 1 nt, bit 4 sc1.
constexpr int kCpNt = 2, kCpSc1 = 16, kCpNtSc1 = kCpNt | kCpSc1;
__device__ __forceinline__ BufRes buf_res(const void* base, int64_t bytes) {
    const uint32_t n = bytes >= (int64_t)0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)(bytes > 0 ? bytes : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufWord3);
}
// Four consecutive contribution values widened to fp32: bf16 as one 8-byte
// load, fp32 as one 16-byte load (nontemporal).
__device__ __forceinline__ f32x4 bld4f(BufRes r, int off, const uint16_t*) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpNt);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
}
__device__ __forceinline__ f32x4 bld4f(BufRes r, int off, const float*) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpNt));
}
__device__ __forceinline__ f32x4 bldf4_nt(BufRes r, int off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpNt));
}
template <int CP>
__device__ __forceinline__ void bstf4(BufRes r, int off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void bst8(BufRes r, int off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CP);
}
// A 64-bit value that is the same in every lane, as a wave-uniform value.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void widen8(u32x4 w, float a[8]) {
    a[0] = bf16_lo(w.x); a[1] = bf16_hi(w.x); a[2] = bf16_lo(w.y); a[3] = bf16_hi(w.y);
    a[4] = bf16_lo(w.z); a[5] = bf16_hi(w.z); a[6] = bf16_lo(w.w); a[7] = bf16_hi(w.w);
}

// a[j] = a[j] + widen(w)[j]: one IEEE fp32 add per element, partial sum on the left.
__device__ __forceinline__ void add8(u32x4 w, float a[8]) {
    a[0] = a[0] + bf16_lo(w.x); a[1] = a[1] + bf16_hi(w.x);
    a[2] = a[2] + bf16_lo(w.y); a[3] = a[3] + bf16_hi(w.y);
    a[4] = a[4] + bf16_lo(w.z); a[5] = a[5] + bf16_hi(w.z);
    a[6] = a[6] + bf16_lo(w.w); a[7] = a[7] + bf16_hi(w.w);
}

// Four consecutive contribution values widened to fp32 (nontemporal): bf16 as
// one 8-byte load, fp32 as one 16-byte load.
__device__ __forceinline__ f32x4 ld4f_nt(const uint16_t* p) {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
}
__device__ __forceinline__ f32x4 ld4f_nt(const float* p) { return ldf4_nt(p); }

// a <- a + b, one IEEE fp32 add per element, partial sum on the left.
__device__ __forceinline__ f32x4 add4(f32x4 a, f32x4 b) {
    return f32x4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
}
// Each element rounded to bf16 (nearest even), kept as fp32.
__device__ __forceinline__ f32x4 round4_bf16(f32x4 a) {
    return f32x4{__uint_as_float(bf16_rne(a.x) << 16), __uint_as_float(bf16_rne(a.y) << 16),
                 __uint_as_float(bf16_rne(a.z) << 16), __uint_as_float(bf16_rne(a.w) << 16)};
}

// a[j] <- bf16(a[j]) (round to nearest even), kept as fp32.
__device__ __forceinline__ void round8_bf16(float a[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __uint_as_float(bf16_rne(a[j]) << 16);
}

// Sum over the block in a fixed order; the result is valid in thread 0.
__device__ double block_sum(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = x + __shfl_xor(x, o, 64);
    __shared__ double part[kBlock / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < kBlock / 64; ++k) s = s + part[k];
    }
    return s;
}

// Plan lookup tables (position -> interval) on the device: one 8-byte cell per
// 2^shift positions holding {lo, hi} (int32 each), the intervals that contain the
// cell's first and last position.  Kernels take the cells as a __restrict__
// pointer argument: only then may the compiler read them through the scalar
// cache (as a plain pointer they became vector loads and cost 7% of the pack's
// rate).
// The interval k in [lo_min, hi_max] that holds position x: the largest k with
// starts[k * stride] <= x, starts non-decreasing.  One 8-byte load of the cell;
// a binary search only over the intervals that start inside it (none for most
// cells).  The bounds narrow the search to a subset known to hold the answer.
// Host-callable so that a CPU test runs this very code against brute force.
__host__ __device__ __forceinline__ int lut_find(const uint64_t* __restrict__ cells, int shift,
                                                 const int64_t* __restrict__ starts, int stride,
                                                 int64_t x, int lo_min, int hi_max) {
    const uint64_t c = cells[x >> shift];
    int lo = (int)(uint32_t)c, hi = (int)(uint32_t)(c >> 32);
    lo = lo > lo_min ? lo : lo_min;
    hi = hi < hi_max ? hi : hi_max;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (starts[(int64_t)mid * stride] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Walks the bucket segments of a shard in increasing order.  seg rows are
// {shard_off, base, chunk}, one per bucket, then {S, 0, 0}.  For shard index i
// in bucket b, the all-gather / flat position is i + delta with
// delta = base_b + owner*C_b - shard_off_b.
struct SegCursor {
    const int64_t* seg;
    int64_t owner, end, delta;
    int b;
    __device__ void seek(int64_t i, const uint64_t* __restrict__ lut, int shift) {   // i < S
        b = lut_find(lut, shift, seg, 3, i, 0, 0x7fffffff);   // the bucket that holds i
        load();
    }
    __device__ void load() {
        end = seg[3 * (b + 1)];
        delta = seg[3 * b + 1] + owner * seg[3 * b + 2] - seg[3 * b];
    }
    __device__ __forceinline__ int64_t map(int64_t i) {
        while (i >= end) { ++b; load(); }
        return i + delta;
    }
};

}  // namespace
