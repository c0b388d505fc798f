// gfx950 kernels of the shard step and the device half of the C ABI.
//
// Every kernel here is HBM-bound streaming work (no contraction, so no MFMA):
// 16-byte loads and stores per lane, 64-wide wavefronts, and one short block per
// tile with the grid covering the data.  Blocks are dispatched in index order,
// so the lines in flight stay close together in the address space; on MI355X
// that moves 10-20% more bytes per second than long-running grid-stride blocks.
// fp64 reductions run in a fixed order (wave shuffles, LDS, one partial per
// block, then fixed ranges of partials) so results are bit-reproducible.
//
// Pages cited (title, section): see gsz.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "gsz_internal.h"

#pragma clang fp contract(off)

using gsz::set_error;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kBlock = 256;
// The pack kernels' block: one wave per 1 KiB tile copied 2.7% faster than
// 256-lane blocks on 2 KiB tiles (7B share, MI355X).
constexpr int kPackBlock = 64;
// AdamW's block size (8 waves of 512 elements): measured faster than 256.
constexpr int kAdamBlock = 512;
// Largest grid: grid * block work-items must stay below 2^32 per dispatch.
// Bigger inputs make blocks stride over the remaining tiles.
constexpr int64_t kMaxFlatGrid = (int64_t)1 << 23;
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

struct RankPtrs { const uint16_t* p[GSZ_MAX_RANKS]; };
struct RankPtrsF { const float* p[GSZ_MAX_RANKS]; };
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
__device__ __forceinline__ f32x4 ldf4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void stf4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

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

// Walks the bucket segments of a shard in increasing order.  seg rows are
// {shard_off, base, chunk}; row nseg is {S, 0, 0}.  For shard index i in bucket
// b, the all-gather / flat position is i + delta with
// delta = base_b + owner*C_b - shard_off_b.
struct SegCursor {
    const int64_t* seg;
    int64_t owner, end, delta;
    int b;
    __device__ void seek(int64_t i, int nseg) {
        int lo = 0, hi = nseg - 1;          // largest b with shard_off[b] <= i
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seg[3 * mid] <= i) lo = mid; else hi = mid - 1;
        }
        b = lo;
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

// ------------------------------------------------------------------ pack --

// Pack modes: copy tensors into the flat buffer, copy flat ranges back into the
// tensors, or add tensors into the flat buffer (bf16 += bf16 in fp32, rounded
// to nearest even).
enum PackMode { kPack = 0, kUnpack = 1, kAccumulate = 2 };

__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
    return bf16_rne(bf16_lo(a) + bf16_lo(b)) | (bf16_rne(bf16_hi(a) + bf16_hi(b)) << 16);
}
__device__ __forceinline__ u32x4 add_bf16x8(u32x4 a, u32x4 b) {
    return u32x4{add_bf16x2(a.x, b.x), add_bf16x2(a.y, b.y), add_bf16x2(a.z, b.z),
                 add_bf16x2(a.w, b.w)};
}
__device__ __forceinline__ uint16_t add_bf16(uint16_t a, uint16_t b) {
    return (uint16_t)bf16_rne(__uint_as_float((uint32_t)a << 16) + __uint_as_float((uint32_t)b << 16));
}

// Moves the tensors of one batch (bucket-order positions [k0, k0+nk)) to or
// from the flat buffer as MODE says.  tab rows: {flat offset, numel, first
// tile}.  One block per tile of kPackTile = 8 * kPackBlock elements (one
// 16-byte vector per lane), the grid covering the batch's tiles [t_begin, t_end): short
// blocks dispatched in address order keep the lines in flight close together,
// which MI355X's HBM rewards over long-running grid-stride blocks.  Grids are
// capped below the dispatch limit; blocks then stride over the remaining tiles.
template <int MODE>
__global__ __launch_bounds__(kPackBlock) void k_pack(PackPtrs pp, const int64_t* __restrict__ tab,
                                                 int k0, int nk, int64_t t_begin, int64_t t_end,
                                                 uint16_t* __restrict__ flat) {
    const int tid = threadIdx.x;
    for (int64_t tile = t_begin + blockIdx.x; tile < t_end; tile += gridDim.x) {
        int lo = k0, hi = k0 + nk - 1;          // largest k with first_tile[k] <= tile
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tab[3 * mid + 2] <= tile) lo = mid; else hi = mid - 1;
        }
        const int k = lo;
        const int64_t n = tab[3 * k + 1];
        const int64_t j0 = (tile - tab[3 * k + 2]) * gsz::kPackTile;
        const int64_t j1 = j0 + gsz::kPackTile < n ? j0 + gsz::kPackTile : n;
        const uint16_t* __restrict__ src = MODE == kUnpack ? flat + tab[3 * k] : pp.p[k - k0];
        uint16_t* __restrict__ dst = MODE == kUnpack ? const_cast<uint16_t*>(pp.p[k - k0]) : flat + tab[3 * k];
        const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
        if (vec && j1 - j0 == gsz::kPackTile) {
            static_assert(gsz::kPackTile == 8 * kPackBlock, "one vector per lane");
            // Nontemporal hints on both sides: the bytes are used once (2-3% faster).
            const int64_t j = j0 + 8 * tid;
            u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + j));
            if (MODE == kAccumulate) w = add_bf16x8(ld16(dst + j), w);
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst + j));
        } else if (vec) {
            const int64_t jv = j0 + ((j1 - j0) & ~(int64_t)7);
            for (int64_t j = j0 + 8 * tid; j < jv; j += 8 * kPackBlock)
                st16(dst + j, MODE == kAccumulate ? add_bf16x8(ld16(dst + j), ld16(src + j)) : ld16(src + j));
            for (int64_t j = jv + tid; j < j1; j += kPackBlock)
                dst[j] = MODE == kAccumulate ? add_bf16(dst[j], src[j]) : src[j];
        } else {
            for (int64_t j = j0 + tid; j < j1; j += kPackBlock)
                dst[j] = MODE == kAccumulate ? add_bf16(dst[j], src[j]) : src[j];
        }
    }
}

// Zeroes the padding at the end of each padded bucket; one block per bucket.
__global__ __launch_bounds__(kBlock) void k_zero_pads(const int64_t* __restrict__ pads,
                                                      uint16_t* __restrict__ flat) {
    const int64_t s = pads[2 * blockIdx.x], n = pads[2 * blockIdx.x + 1];
    for (int64_t j = threadIdx.x; j < n; j += kBlock) flat[s + j] = 0;
}

// fp32 accumulation buckets (gradient accumulation with an fp32 reduction
// dtype): ACC = false widens the tensors of one batch into flat32 (the first
// micro-batch), ACC = true adds them: flat32[off_t + j] = flat32[off_t + j] +
// f32(grad_t[j]), one IEEE fp32 addition.  Tiles and grid as k_pack.  In a full
// tile lane l takes elements 4l..4l+3 and 256+4l..256+4l+3 (two 8-byte bf16
// loads), so each 16-byte fp32 load and store of the wave covers whole lines;
// with nontemporal hints on every access this runs 5-6% faster than one 16-byte
// bf16 load per lane widened into two half-line fp32 stores.
__device__ __forceinline__ void stf8(float* p, const float a[8]) {
    stf4(p, f32x4{a[0], a[1], a[2], a[3]});
    stf4(p + 4, f32x4{a[4], a[5], a[6], a[7]});
}
template <bool ACC>
__global__ __launch_bounds__(kPackBlock) void k_pack_f32(PackPtrs pp, const int64_t* __restrict__ tab,
                                                     int k0, int nk, int64_t t_begin, int64_t t_end,
                                                     float* __restrict__ flat) {
    const int tid = threadIdx.x;
    for (int64_t tile = t_begin + blockIdx.x; tile < t_end; tile += gridDim.x) {
        int lo = k0, hi = k0 + nk - 1;          // largest k with first_tile[k] <= tile
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tab[3 * mid + 2] <= tile) lo = mid; else hi = mid - 1;
        }
        const int k = lo;
        const int64_t n = tab[3 * k + 1];
        const int64_t j0 = (tile - tab[3 * k + 2]) * gsz::kPackTile;
        const int64_t j1 = j0 + gsz::kPackTile < n ? j0 + gsz::kPackTile : n;
        const uint16_t* __restrict__ src = pp.p[k - k0];
        float* __restrict__ dst = flat + tab[3 * k];
        const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
        if (vec && j1 - j0 == gsz::kPackTile) {
            static_assert(gsz::kPackTile == 8 * kPackBlock, "two groups of 4 elements per lane");
            const int64_t ja = j0 + 4 * tid, jb = ja + 4 * kPackBlock;
            const u32x2 wa = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src + ja));
            const u32x2 wb = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src + jb));
            f32x4 xa = f32x4{bf16_lo(wa.x), bf16_hi(wa.x), bf16_lo(wa.y), bf16_hi(wa.y)};
            f32x4 xb = f32x4{bf16_lo(wb.x), bf16_hi(wb.x), bf16_lo(wb.y), bf16_hi(wb.y)};
            if (ACC) {
                const f32x4 da = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dst + ja));
                const f32x4 db = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dst + jb));
                xa = f32x4{da.x + xa.x, da.y + xa.y, da.z + xa.z, da.w + xa.w};
                xb = f32x4{db.x + xb.x, db.y + xb.y, db.z + xb.z, db.w + xb.w};
            }
            __builtin_nontemporal_store(xa, reinterpret_cast<f32x4*>(dst + ja));
            __builtin_nontemporal_store(xb, reinterpret_cast<f32x4*>(dst + jb));
        } else if (vec) {
            const int64_t jv = j0 + ((j1 - j0) & ~(int64_t)7);
            for (int64_t j = j0 + 8 * tid; j < jv; j += 8 * kPackBlock) {
                float a[8];
                widen8(ld16(src + j), a);
                if (ACC) {
                    const f32x4 d0 = ldf4(dst + j), d1 = ldf4(dst + j + 4);
                    a[0] = d0.x + a[0]; a[1] = d0.y + a[1]; a[2] = d0.z + a[2]; a[3] = d0.w + a[3];
                    a[4] = d1.x + a[4]; a[5] = d1.y + a[5]; a[6] = d1.z + a[6]; a[7] = d1.w + a[7];
                }
                stf8(dst + j, a);
            }
            for (int64_t j = jv + tid; j < j1; j += kPackBlock) {
                const float x = __uint_as_float((uint32_t)src[j] << 16);
                dst[j] = ACC ? dst[j] + x : x;
            }
        } else {
            for (int64_t j = j0 + tid; j < j1; j += kPackBlock) {
                const float x = __uint_as_float((uint32_t)src[j] << 16);
                dst[j] = ACC ? dst[j] + x : x;
            }
        }
    }
}

// Zeroes the padding of each padded bucket of an fp32 buffer; one block per bucket.
__global__ __launch_bounds__(kBlock) void k_zero_pads_f32(const int64_t* __restrict__ pads,
                                                          float* __restrict__ flat) {
    const int64_t s = pads[2 * blockIdx.x], n = pads[2 * blockIdx.x + 1];
    for (int64_t j = threadIdx.x; j < n; j += kBlock) flat[s + j] = 0.0f;
}

// ---------------------------------------------------------- reduce-mean --

// g[i] = (((c0 + c1) + c2) + ... + c_{P-1}) / P with rp.p[k] = contribution of
// rank (owner+1+k) mod P, so the owner's own value is added last.  Each lane
// handles 8 consecutive shard elements per iteration (one 16-byte load per
// rank).  PS > 0 fixes P at compile time; loads are issued in groups of up to
// 16 ranks before their adds so many 16-byte requests are in flight.  With
// OUTFLAT (bucket-flat input only) g is indexed by flat position instead of
// shard index: P launches, one per chunk owner, give the all-reduce result.
// W16: the partial sum is rounded to bf16 after every addition (a ring whose
// wire carries bf16 partial sums); the final division stays fp32.
template <int PS, bool NORM, bool FLAT, bool OUTFLAT = false, bool W16 = false>
__global__ __launch_bounds__(kBlock) void k_reduce_mean(RankPtrs rp, int P, float invP, int pow2,
                                                        const int64_t* __restrict__ seg, int nseg,
                                                        int64_t owner, int64_t nvec,
                                                        float* __restrict__ g,
                                                        double* __restrict__ ws) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    const int64_t bx = xcd_remap(blockIdx.x, gridDim.x);      // logical block: tile bx
    int64_t v = bx * kBlock + threadIdx.x;
    double sq = 0.0;
    SegCursor cur{seg, owner, 0, 0, 0};
    if (FLAT && v < nvec) cur.seek(bx * kRedTile, nseg);      // uniform: scalar loads
    const float fP = (float)P;
    for (; v < nvec; v += stride) {
        const int64_t i = v * 8;
        const int64_t off = FLAT ? cur.map(i) : i;
        float a[8];
        if constexpr (PS > 0) {
            constexpr int G = PS < 16 ? PS : 16;
#pragma unroll
            for (int k0 = 0; k0 < PS; k0 += G) {
                u32x4 w[G];
#pragma unroll
                for (int j = 0; j < G; ++j) w[j] = ld16(rp.p[k0 + j] + off);
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (k0 + j == 0) widen8(w[j], a);
                    else { add8(w[j], a); if (W16) round8_bf16(a); }
                }
            }
        } else {
            widen8(ld16(rp.p[0] + off), a);
            int k = 1;
            for (; k + 8 <= P; k += 8) {
                u32x4 w[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) w[j] = ld16(rp.p[k + j] + off);
#pragma unroll
                for (int j = 0; j < 8; ++j) { add8(w[j], a); if (W16) round8_bf16(a); }
            }
            for (; k < P; ++k) { add8(ld16(rp.p[k] + off), a); if (W16) round8_bf16(a); }
        }
        if (PS > 0 ? ((PS & (PS - 1)) == 0) : pow2) {
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = a[j] * invP;   // exact: invP is a power of two
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = a[j] / fP;
        }
        const int64_t o = OUTFLAT ? off : i;    // all-reduce output: the flat position
        stf4(g + o, f32x4{a[0], a[1], a[2], a[3]});
        stf4(g + o + 4, f32x4{a[4], a[5], a[6], a[7]});
        if (NORM) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double d = (double)a[j];
                sq = __fma_rn(d, d, sq);                        // d*d is exact in fp64
            }
        }
    }
    if (NORM) {
        const double s = block_sum(sq);
        if (threadIdx.x == 0) ws[bx] = s;
    }
}

// The reduce over fp32 contributions (fp32 accumulation buckets, fp32 on the
// ring's wire): the same ring order and division as k_reduce_mean, inputs
// taken as they are.  A wave owns 512 shard elements of its block's tile as two
// groups of 256; lane l handles elements 4l..4l+3 of each, so every 16-byte
// load and store of a wave covers whole lines.  Blocks, XCD order and norm
// partials as k_reduce_mean.
template <int PS, bool NORM, bool FLAT>
__global__ __launch_bounds__(kBlock) void k_reduce_mean_f32(RankPtrsF rp, int P, float invP, int pow2,
                                                            const int64_t* __restrict__ seg, int nseg,
                                                            int64_t owner, int64_t S,
                                                            float* __restrict__ g,
                                                            double* __restrict__ ws) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t bx = xcd_remap(blockIdx.x, gridDim.x);
    double sq = 0.0;
    SegCursor cur{seg, owner, 0, 0, 0};
    int64_t t = bx * kRedTile;
    if (FLAT && t < S) cur.seek(t, nseg);                     // uniform: scalar loads
    const float fP = (float)P;
    for (; t < S; t += (int64_t)gridDim.x * kRedTile) {
        const int64_t i0 = t + 512 * wave + 4 * lane, i1 = i0 + 256;
        const bool ok0 = i0 < S, ok1 = i1 < S;               // S and i are multiples of 4
        const int64_t off0 = ok0 ? (FLAT ? cur.map(i0) : i0) : 0;
        const int64_t off1 = ok1 ? (FLAT ? cur.map(i1) : i1) : 0;
        const f32x4 zero = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 a = zero, b = zero;
        if constexpr (PS > 0) {
            constexpr int G = PS < 16 ? PS : 16;
#pragma unroll
            for (int k0 = 0; k0 < PS; k0 += G) {
                f32x4 w0[G], w1[G];
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    w0[j] = ok0 ? ldf4(rp.p[k0 + j] + off0) : zero;
                    w1[j] = ok1 ? ldf4(rp.p[k0 + j] + off1) : zero;
                }
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (k0 + j == 0) { a = w0[j]; b = w1[j]; }
                    else {
                        a.x = a.x + w0[j].x; a.y = a.y + w0[j].y; a.z = a.z + w0[j].z; a.w = a.w + w0[j].w;
                        b.x = b.x + w1[j].x; b.y = b.y + w1[j].y; b.z = b.z + w1[j].z; b.w = b.w + w1[j].w;
                    }
                }
            }
        } else {
            a = ok0 ? ldf4(rp.p[0] + off0) : zero;
            b = ok1 ? ldf4(rp.p[0] + off1) : zero;
            for (int k = 1; k < P; ++k) {
                const f32x4 w0 = ok0 ? ldf4(rp.p[k] + off0) : zero;
                const f32x4 w1 = ok1 ? ldf4(rp.p[k] + off1) : zero;
                a.x = a.x + w0.x; a.y = a.y + w0.y; a.z = a.z + w0.z; a.w = a.w + w0.w;
                b.x = b.x + w1.x; b.y = b.y + w1.y; b.z = b.z + w1.z; b.w = b.w + w1.w;
            }
        }
        if (PS > 0 ? ((PS & (PS - 1)) == 0) : pow2) {
            a = f32x4{a.x * invP, a.y * invP, a.z * invP, a.w * invP};   // exact: a power of two
            b = f32x4{b.x * invP, b.y * invP, b.z * invP, b.w * invP};
        } else {
            a = f32x4{a.x / fP, a.y / fP, a.z / fP, a.w / fP};
            b = f32x4{b.x / fP, b.y / fP, b.z / fP, b.w / fP};
        }
        if (ok0) stf4(g + i0, a);
        if (ok1) stf4(g + i1, b);
        if (NORM) {
            const double d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) sq = __fma_rn(d[j], d[j], sq);   // zeros where !ok
        }
    }
    if (NORM) {
        const double s = block_sum(sq);
        if (threadIdx.x == 0) ws[bx] = s;
    }
}

// Standalone squared norm of n fp32 values (16-byte aligned): block b sums
// elements [b * kRedTile, (b + 1) * kRedTile) (two lane-contiguous 16-byte
// loads per lane) into ws[b].
__global__ __launch_bounds__(kBlock) void k_sqnorm(const float* __restrict__ g, int64_t n,
                                                   double* __restrict__ ws) {
    const int tid = threadIdx.x;
    double sq = 0.0;
    for (int64_t base = (int64_t)blockIdx.x * kRedTile; base < n; base += (int64_t)gridDim.x * kRedTile) {
        if (base + kRedTile <= n) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 x = ldf4(g + base + h * (4 * kBlock) + 4 * tid);
                const double d0 = x.x, d1 = x.y, d2 = x.z, d3 = x.w;
                sq = __fma_rn(d0, d0, sq); sq = __fma_rn(d1, d1, sq);
                sq = __fma_rn(d2, d2, sq); sq = __fma_rn(d3, d3, sq);
            }
        } else {
            for (int64_t i = base + tid; i < n; i += kBlock) {
                const double d = g[i];
                sq = __fma_rn(d, d, sq);
            }
        }
    }
    const double s = block_sum(sq);
    if (threadIdx.x == 0) ws[blockIdx.x] = s;
}

// ws2[b] = sum, in order, of the partials in the b-th of gridDim.x contiguous
// ranges of ws[0, n).
__global__ __launch_bounds__(kBlock) void k_finalize_ranges(const double* __restrict__ ws, int64_t n,
                                                            double* __restrict__ ws2) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t a = (int64_t)blockIdx.x * per, e = a + per < n ? a + per : n;
    double s = 0.0;
    for (int64_t k = a + threadIdx.x; k < e; k += kBlock) s = s + ws[k];
    s = block_sum(s);
    if (threadIdx.x == 0) ws2[blockIdx.x] = s;
}

// out = sum of the n block partials, in block order, one block.
__global__ __launch_bounds__(kBlock) void k_finalize(const double* __restrict__ ws, int64_t n,
                                                     double* __restrict__ out) {
    double s = 0.0;
    for (int64_t k = threadIdx.x; k < n; k += kBlock) s = s + ws[k];
    s = block_sum(s);
    if (threadIdx.x == 0) *out = s;
}

// total = partials[0] + ... + partials[n-1] (rank order); norm = fp32(sqrt(total));
// coef = min(1, max_norm / (norm + 1e-6)); NaN propagates.
__global__ void k_clip(const double* __restrict__ partials, int n, float max_norm,
                       float* __restrict__ coef, float* __restrict__ norm,
                       double* __restrict__ total) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    double t = 0.0;
    for (int q = 0; q < n; ++q) t = t + partials[q];
    const float nr = (float)sqrt(t);
    const float c = max_norm / (nr + 1e-6f);
    *coef = (c != c) ? c : (c < 1.0f ? c : 1.0f);
    if (norm) *norm = nr;
    if (total) *total = t;
}

// ----------------------------------------------------------------- AdamW --

__device__ __forceinline__ void adamw1(float& th, float& mm, float& vv, float gg, float coef,
                                       const AdamScalars& s) {
    const float gc = gg * coef;
    const float m1 = (s.b1 * mm) + (s.omb1 * gc);
    const float v1 = (s.b2 * vv) + (s.omb2 * (gc * gc));
    const float mh = m1 / s.bc1;
    const float vh = v1 / s.bc2;
    const float u = mh / (sqrtf(vh) + s.eps);
    th = (th * s.decay) - (s.lr * u);
    mm = m1;
    vv = v1;
}

// A wave owns 512 consecutive shard elements per iteration, as two groups of
// 256; lane l updates elements 4l..4l+3 of each group, so every 16-byte load
// and store instruction of the wave covers 1 KiB of whole 128-byte lines (a
// lane that loads 32 contiguous bytes as two 16-byte halves makes each
// instruction touch half of every line, and half-line misses to the same line
// are fetched twice).  The bf16 result goes out as 8 bytes per lane.
template <bool GATH, bool SHARD>
__global__ __launch_bounds__(kAdamBlock) void k_adamw(float* __restrict__ master, float* __restrict__ m,
                                                      float* __restrict__ v, const float* __restrict__ g,
                                                      const float* __restrict__ coefp, AdamScalars s,
                                                      const int64_t* __restrict__ seg, int nseg,
                                                      int64_t owner, int64_t S,
                                                      uint16_t* __restrict__ gathered,
                                                      uint16_t* __restrict__ shard_bf16) {
    constexpr int kWaves = kAdamBlock / 64;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    int64_t wv = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t ntile = (S + 511) / 512;
    const float coef = *coefp;
    SegCursor cur{seg, owner, 0, 0, 0};
    if (GATH && wv < ntile) cur.seek(wv * 512, nseg);        // wave-uniform: scalar loads
    for (; wv < ntile; wv += nwaves) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t i = wv * 512 + h * 256 + 4 * lane;
            if (i < S) {                       // S and i are multiples of 4
                const f32x4 g4 = ldf4(g + i);
                const f32x4 t4 = ldf4(master + i), m4 = ldf4(m + i), v4 = ldf4(v + i);
                float th[4] = {t4.x, t4.y, t4.z, t4.w};
                float mm[4] = {m4.x, m4.y, m4.z, m4.w};
                float vv[4] = {v4.x, v4.y, v4.z, v4.w};
                const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) adamw1(th[j], mm[j], vv[j], gg[j], coef, s);
                stf4(master + i, f32x4{th[0], th[1], th[2], th[3]});
                stf4(m + i, f32x4{mm[0], mm[1], mm[2], mm[3]});
                stf4(v + i, f32x4{vv[0], vv[1], vv[2], vv[3]});
                const u32x2 p = u32x2{bf16_rne(th[0]) | (bf16_rne(th[1]) << 16),
                                      bf16_rne(th[2]) | (bf16_rne(th[3]) << 16)};
                if (GATH) *reinterpret_cast<u32x2*>(gathered + cur.map(i)) = p;
                if (SHARD) *reinterpret_cast<u32x2*>(shard_bf16 + i) = p;
            }
        }
    }
}

// gathered[i + delta_b] = shard[i] for shard index i of bucket b.
__global__ __launch_bounds__(kBlock) void k_ag_write(const uint16_t* __restrict__ shard,
                                                     const int64_t* __restrict__ seg, int nseg,
                                                     int64_t owner, int64_t nvec,
                                                     uint16_t* __restrict__ gathered) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t v = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    SegCursor cur{seg, owner, 0, 0, 0};
    if (v < nvec) cur.seek((int64_t)blockIdx.x * kBlock * 8, nseg);   // the block's first element
    for (; v < nvec; v += stride) {
        const int64_t i = v * 8;
        st16(gathered + cur.map(i), ld16(shard + i));
    }
}

// ------------------------------------------------------------ host side --

std::atomic<int> g_dev_state[64];   // 0 unknown, 1 gfx950, -1 other

int hip_fail(const char* what, hipError_t e) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return GSZ_ERR_HIP;
}

// Current device, checked to be gfx950.
int current_device(int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= 64) { set_error("device index %d unsupported", dev); return GSZ_ERR_DEVICE; }
    int st = g_dev_state[dev].load();
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_dev_state[dev].store(st);
    }
    if (st != 1) { set_error("device %d is not gfx950 (MI355X); this library targets gfx950 only", dev); return GSZ_ERR_DEVICE; }
    *dev_out = dev;
    return GSZ_OK;
}

// Blocks of a one-tile-per-block launch over n_tiles tiles.
int flat_grid(int64_t n_tiles) {
    if (n_tiles < 1) return 1;
    return (int)(n_tiles < kMaxFlatGrid ? n_tiles : kMaxFlatGrid);
}

// Partials of the reductions: grid blocks wrote ws[0, grid); sum them in a
// fixed order into *out (two stages when there are many).
void launch_finalize(double* ws, int64_t grid, double* out, hipStream_t stream) {
    if (grid > gsz::kFinalBlocks) {
        hipLaunchKernelGGL(k_finalize_ranges, dim3(gsz::kFinalBlocks), dim3(kBlock), 0, stream,
                           static_cast<const double*>(ws), grid, ws + grid);
        hipLaunchKernelGGL(k_finalize, dim3(1), dim3(kBlock), 0, stream,
                           static_cast<const double*>(ws + grid), (int64_t)gsz::kFinalBlocks, out);
    } else {
        hipLaunchKernelGGL(k_finalize, dim3(1), dim3(kBlock), 0, stream,
                           static_cast<const double*>(ws), grid, out);
    }
}

int launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(what, e);
    return GSZ_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// The fp32 constants of the update, each formed in double and rounded once.
AdamScalars adam_scalars(const gsz_adamw_hp& hp) {
    AdamScalars s;
    s.b1 = (float)hp.beta1;
    s.omb1 = (float)(1.0 - hp.beta1);
    s.b2 = (float)hp.beta2;
    s.omb2 = (float)(1.0 - hp.beta2);
    s.bc1 = (float)(1.0 - std::pow(hp.beta1, (double)hp.step));
    s.bc2 = (float)(1.0 - std::pow(hp.beta2, (double)hp.step));
    s.lr = (float)hp.lr;
    s.eps = (float)hp.eps;
    s.decay = (float)(1.0 - hp.lr * hp.weight_decay);
    return s;
}

// Checks a plan for a device call: uploaded to the current device, vector granule.
int check_plan(const gsz_plan* p, const char* who) {
    if (!p) { set_error("%s: NULL plan", who); return GSZ_ERR_INVALID_ARG; }
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (!p->dev_mem || p->device != dev) {
        set_error("%s: plan has no device tables on device %d (call gsz_plan_upload)", who, dev);
        return GSZ_ERR_NOT_UPLOADED;
    }
    if (p->align % 8 != 0) {
        set_error("%s: device calls need align a multiple of 8 elements (plan has %d)", who, p->align);
        return GSZ_ERR_INVALID_ARG;
    }
    return GSZ_OK;
}

int check_owner(const gsz_plan* p, int32_t owner, const char* who) {
    if (owner < 0 || owner >= p->P) {
        set_error("%s: owner %d outside [0, %d)", who, owner, p->P);
        return GSZ_ERR_BAD_RANK;
    }
    return GSZ_OK;
}

template <int PS>
void launch_reduce(bool norm, bool flat, dim3 grid, hipStream_t st, const RankPtrs& rp, int P,
                   float invP, int pow2, const int64_t* seg, int nseg, int64_t owner, int64_t nvec,
                   float* g, double* ws, bool outflat = false, bool wire16 = false) {
    if (wire16) {
        if (norm && flat)
            hipLaunchKernelGGL((k_reduce_mean<PS, true, true, false, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
        else if (norm)
            hipLaunchKernelGGL((k_reduce_mean<PS, true, false, false, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
        else if (flat)
            hipLaunchKernelGGL((k_reduce_mean<PS, false, true, false, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
        else
            hipLaunchKernelGGL((k_reduce_mean<PS, false, false, false, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
        return;
    }
    if (outflat && norm)
        hipLaunchKernelGGL((k_reduce_mean<PS, true, true, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
    else if (outflat)
        hipLaunchKernelGGL((k_reduce_mean<PS, false, true, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
    else if (norm && flat)
        hipLaunchKernelGGL((k_reduce_mean<PS, true, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
    else if (norm)
        hipLaunchKernelGGL((k_reduce_mean<PS, true, false>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
    else if (flat)
        hipLaunchKernelGGL((k_reduce_mean<PS, false, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
    else
        hipLaunchKernelGGL((k_reduce_mean<PS, false, false>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, nvec, g, ws);
}

template <int PS>
void launch_reduce_f32(bool norm, bool flat, dim3 grid, hipStream_t st, const RankPtrsF& rp, int P,
                       float invP, int pow2, const int64_t* seg, int nseg, int64_t owner, int64_t S,
                       float* g, double* ws) {
    if (norm && flat)
        hipLaunchKernelGGL((k_reduce_mean_f32<PS, true, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, S, g, ws);
    else if (norm)
        hipLaunchKernelGGL((k_reduce_mean_f32<PS, true, false>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, S, g, ws);
    else if (flat)
        hipLaunchKernelGGL((k_reduce_mean_f32<PS, false, true>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, S, g, ws);
    else
        hipLaunchKernelGGL((k_reduce_mean_f32<PS, false, false>), grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, nseg, owner, S, g, ws);
}

}  // namespace

// ---------------------------------------------------------------- C ABI --

extern "C" int gsz_plan_destroy(gsz_plan* p) {
    if (!p) return GSZ_OK;
    if (p->dev_mem) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(p->device) == hipSuccess) {
            (void)hipFree(p->dev_mem);
            (void)hipSetDevice(cur);
        }
    }
    delete p;
    return GSZ_OK;
}

extern "C" int gsz_plan_upload(gsz_plan* p) {
    if (!p) { set_error("gsz_plan_upload: NULL plan"); return GSZ_ERR_INVALID_ARG; }
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(p->mu);
    if (p->dev_mem && p->device == dev) return GSZ_OK;
    if (p->dev_mem) {
        hipError_t e = hipSetDevice(p->device);
        if (e == hipSuccess) e = hipFree(p->dev_mem);
        (void)hipSetDevice(dev);
        if (e != hipSuccess) return hip_fail("gsz_plan_upload: freeing old tables", e);
        p->dev_mem = nullptr;
        p->device = -1;
    }
    const size_t n_seg = p->seg.size(), n_pack = p->pack.size(), n_pads = p->pads.size();
    const size_t bytes = (n_seg + n_pack + n_pads + 2) * sizeof(int64_t);
    void* mem = nullptr;
    hipError_t e = hipMalloc(&mem, bytes);
    if (e != hipSuccess) return hip_fail("gsz_plan_upload: hipMalloc", e);
    int64_t* d = static_cast<int64_t*>(mem);
    std::vector<int64_t> img;
    img.reserve(n_seg + n_pack + n_pads + 2);
    img.insert(img.end(), p->seg.begin(), p->seg.end());
    img.insert(img.end(), p->pack.begin(), p->pack.end());
    img.insert(img.end(), p->pads.begin(), p->pads.end());
    img.resize(img.size() + 2, 0);
    e = hipMemcpy(mem, img.data(), img.size() * sizeof(int64_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) { (void)hipFree(mem); return hip_fail("gsz_plan_upload: hipMemcpy", e); }
    p->dev_mem = mem;
    p->device = dev;
    p->d_seg = d;
    p->d_pack = d + n_seg;
    p->d_pads = d + n_seg + n_pack;
    return GSZ_OK;
}

namespace {

// Modes of run_pack beyond PackMode: the fp32 bucket buffer's first micro-batch
// (widen) and later ones (add).
constexpr int kPackF32 = 3, kAccumulateF32 = 4;

// Launches the pack kernel in `mode` over every tensor: ptrs is the host array of
// the T tensor pointers (sources for kPack/kAccumulate and the fp32 modes,
// destinations for kUnpack); flat is bf16 (uint16) or, in the fp32 modes, float.
int run_pack(const gsz_plan* p, const uint16_t* const* ptrs, void* flat, int mode,
             hipStream_t stream, const char* who) {
    int rc = check_plan(p, who);
    if (rc) return rc;
    const int T = (int)p->numel.size();
    if (p->flat_len == 0) return GSZ_OK;
    if (!flat || (T > 0 && !ptrs)) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(flat)) { set_error("%s: flat is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    for (int t = 0; t < T; ++t)
        if (p->numel[t] > 0 && !ptrs[t]) {
            set_error("%s: tensor pointer %d is NULL", who, t); return GSZ_ERR_INVALID_ARG;
        }
    for (int k0 = 0; k0 < T; k0 += gsz::kPackBatch) {
        const int nk = T - k0 < gsz::kPackBatch ? T - k0 : gsz::kPackBatch;
        PackPtrs pp{};
        for (int k = 0; k < nk; ++k) pp.p[k] = ptrs[T - 1 - (k0 + k)];
        const int64_t tb = p->pack[3 * k0 + 2], te = p->pack[3 * (k0 + nk) + 2];
        if (te == tb) continue;
        constexpr int64_t kMaxPackGrid = ((int64_t)1 << 31) / kPackBlock;   // work-items < 2^32
        const int grid = (int)(te - tb < kMaxPackGrid ? te - tb : kMaxPackGrid);
        uint16_t* f16 = static_cast<uint16_t*>(flat);
        float* f32 = static_cast<float*>(flat);
        if (mode == kPack)
            hipLaunchKernelGGL(k_pack<kPack>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, k0, nk, tb, te, f16);
        else if (mode == kUnpack)
            hipLaunchKernelGGL(k_pack<kUnpack>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, k0, nk, tb, te, f16);
        else if (mode == kAccumulate)
            hipLaunchKernelGGL(k_pack<kAccumulate>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, k0, nk, tb, te, f16);
        else if (mode == kPackF32)
            hipLaunchKernelGGL(k_pack_f32<false>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, k0, nk, tb, te, f32);
        else
            hipLaunchKernelGGL(k_pack_f32<true>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, k0, nk, tb, te, f32);
        if ((rc = launched(who))) return rc;
    }
    const int npad = (int)(p->pads.size() / 2);
    if (mode == kPack && npad > 0) {
        hipLaunchKernelGGL(k_zero_pads, dim3(npad), dim3(kBlock), 0, stream, p->d_pads,
                           static_cast<uint16_t*>(flat));
        if ((rc = launched(who))) return rc;
    }
    if (mode == kPackF32 && npad > 0) {
        hipLaunchKernelGGL(k_zero_pads_f32, dim3(npad), dim3(kBlock), 0, stream, p->d_pads,
                           static_cast<float*>(flat));
        if ((rc = launched(who))) return rc;
    }
    return GSZ_OK;
}

}  // namespace

extern "C" int gsz_bucket_pack(const gsz_plan* p, const uint16_t* const* grads, uint16_t* flat,
                               hipStream_t stream) {
    return run_pack(p, grads, flat, kPack, stream, "gsz_bucket_pack");
}

extern "C" int gsz_bucket_accumulate(const gsz_plan* p, const uint16_t* const* grads,
                                     uint16_t* flat, hipStream_t stream) {
    return run_pack(p, grads, flat, kAccumulate, stream, "gsz_bucket_accumulate");
}

extern "C" int gsz_bucket_pack_f32(const gsz_plan* p, const uint16_t* const* grads, float* flat32,
                                   hipStream_t stream) {
    return run_pack(p, grads, flat32, kPackF32, stream, "gsz_bucket_pack_f32");
}

extern "C" int gsz_bucket_accumulate_f32(const gsz_plan* p, const uint16_t* const* grads,
                                         float* flat32, hipStream_t stream) {
    return run_pack(p, grads, flat32, kAccumulateF32, stream, "gsz_bucket_accumulate_f32");
}

namespace {

// The shard reduce over bf16 contributions (wire16: rounding the partial sums
// to bf16) or, with f32in, over fp32 contributions; contrib holds P device
// pointers of the matching type.
int reduce_impl(const gsz_plan* p, int32_t owner, const void* const* contrib, int32_t layout,
                float* g, double* partial_out, void* ws, size_t ws_bytes, hipStream_t stream,
                bool wire16, bool f32in, const char* who) {
    int rc = check_plan(p, who);
    if (rc) return rc;
    if ((rc = check_owner(p, owner, who))) return rc;
    if (layout != GSZ_LAYOUT_BUCKET_FLAT && layout != GSZ_LAYOUT_SHARD_COMPACT) {
        set_error("%s: unknown layout %d", who, layout); return GSZ_ERR_INVALID_ARG;
    }
    const int P = p->P;
    const int64_t S = p->shard_len;
    if (partial_out) {
        size_t need = 0;
        gsz_workspace_bytes(S, &need);
        if (!ws || ws_bytes < need) { set_error("%s: workspace of %zu bytes required", who, need); return GSZ_ERR_SIZE; }
        if (misaligned(ws)) { set_error("%s: workspace is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    }
    if (S > 0) {
        if (!g || !contrib) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
        if (misaligned(g)) { set_error("%s: g is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
        for (int q = 0; q < P; ++q) {
            if (!contrib[q]) { set_error("%s: contribution %d is NULL", who, q); return GSZ_ERR_INVALID_ARG; }
            if (misaligned(contrib[q])) { set_error("%s: contribution %d is not 16-byte aligned", who, q); return GSZ_ERR_MISALIGNED; }
        }
    }
    const int64_t nvec = S / 8;
    const int grid = flat_grid((S + kRedTile - 1) / kRedTile);
    if (S > 0 && f32in) {
        RankPtrsF rp{};
        for (int k = 0; k < P; ++k) rp.p[k] = static_cast<const float*>(contrib[(owner + 1 + k) % P]);
        const int pow2 = (P & (P - 1)) == 0;
        const float invP = pow2 ? 1.0f / (float)P : 0.0f;
        const bool norm = partial_out != nullptr;
        const bool flat = layout == GSZ_LAYOUT_BUCKET_FLAT;
        const int nseg = (int)p->buckets.size();
        double* wsd = static_cast<double*>(ws);
        const dim3 gr(grid);
        switch (P) {
            case 2: launch_reduce_f32<2>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
            case 4: launch_reduce_f32<4>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
            case 8: launch_reduce_f32<8>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
            case 16: launch_reduce_f32<16>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
            case 32: launch_reduce_f32<32>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
            case 64: launch_reduce_f32<64>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
            default: launch_reduce_f32<0>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, S, g, wsd); break;
        }
        if ((rc = launched(who))) return rc;
    } else if (S > 0) {
        RankPtrs rp{};
        for (int k = 0; k < P; ++k) rp.p[k] = static_cast<const uint16_t*>(contrib[(owner + 1 + k) % P]);
        const int pow2 = (P & (P - 1)) == 0;
        const float invP = pow2 ? 1.0f / (float)P : 0.0f;
        const bool norm = partial_out != nullptr;
        const bool flat = layout == GSZ_LAYOUT_BUCKET_FLAT;
        const int nseg = (int)p->buckets.size();
        double* wsd = static_cast<double*>(ws);
        const dim3 gr(grid);
        switch (P) {
            case 2: launch_reduce<2>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
            case 4: launch_reduce<4>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
            case 8: launch_reduce<8>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
            case 16: launch_reduce<16>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
            case 32: launch_reduce<32>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
            case 64: launch_reduce<64>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
            default: launch_reduce<0>(norm, flat, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, owner, nvec, g, wsd, false, wire16); break;
        }
        if ((rc = launched(who))) return rc;
    }
    if (partial_out) {
        launch_finalize(static_cast<double*>(ws), S > 0 ? grid : 0, partial_out, stream);
        if ((rc = launched(who))) return rc;
    }
    return GSZ_OK;
}

}  // namespace

extern "C" int gsz_shard_reduce_mean(const gsz_plan* p, int32_t owner,
                                     const uint16_t* const* contrib, int32_t layout, float* g,
                                     double* partial_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, ws_bytes, stream, false, false, "gsz_shard_reduce_mean");
}

extern "C" int gsz_shard_reduce_mean_f32(const gsz_plan* p, int32_t owner,
                                         const float* const* contrib, int32_t layout, float* g,
                                         double* partial_out, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, ws_bytes, stream, false, true, "gsz_shard_reduce_mean_f32");
}

extern "C" int gsz_shard_reduce_mean_bf16_wire(const gsz_plan* p, int32_t owner,
                                               const uint16_t* const* contrib, int32_t layout,
                                               float* g, double* partial_out, void* ws,
                                               size_t ws_bytes, hipStream_t stream) {
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, ws_bytes, stream, true, false,
                       "gsz_shard_reduce_mean_bf16_wire");
}

extern "C" int gsz_shard_grad_sqnorm(const float* g, int64_t n, double* partial_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
    const char* who = "gsz_shard_grad_sqnorm";
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (n < 0 || !partial_out || (n > 0 && !g)) { set_error("%s: bad arguments", who); return GSZ_ERR_INVALID_ARG; }
    size_t need = 0;
    gsz_workspace_bytes(n, &need);
    if (!ws || ws_bytes < need) { set_error("%s: workspace of %zu bytes required", who, need); return GSZ_ERR_SIZE; }
    if (misaligned(ws) || (n > 0 && misaligned(g))) { set_error("%s: misaligned pointer", who); return GSZ_ERR_MISALIGNED; }
    int grid = 0;
    if (n > 0) {
        grid = flat_grid((n + kRedTile - 1) / kRedTile);
        hipLaunchKernelGGL(k_sqnorm, dim3(grid), dim3(kBlock), 0, stream, g, n, static_cast<double*>(ws));
        if ((rc = launched(who))) return rc;
    }
    launch_finalize(static_cast<double*>(ws), grid, partial_out, stream);
    return launched(who);
}

extern "C" int gsz_clip_coef(const double* partials, int32_t n_partials, float max_norm,
                             float* coef_out, float* norm_out, double* total_out,
                             hipStream_t stream) {
    const char* who = "gsz_clip_coef";
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (n_partials < 0 || (n_partials > 0 && !partials) || !coef_out) {
        set_error("%s: bad arguments", who); return GSZ_ERR_INVALID_ARG;
    }
    hipLaunchKernelGGL(k_clip, dim3(1), dim3(64), 0, stream, partials, n_partials, max_norm,
                       coef_out, norm_out, total_out);
    return launched(who);
}

extern "C" int gsz_shard_adamw_step(const gsz_plan* p, int32_t owner, float* master, float* m,
                                    float* v, const float* g, const float* coef,
                                    const gsz_adamw_hp* hp, uint16_t* gathered,
                                    uint16_t* shard_bf16, hipStream_t stream) {
    const char* who = "gsz_shard_adamw_step";
    int rc = check_plan(p, who);
    if (rc) return rc;
    if ((rc = check_owner(p, owner, who))) return rc;
    if (!hp || !coef) { set_error("%s: NULL hyperparameters or coefficient", who); return GSZ_ERR_INVALID_ARG; }
    if (hp->step < 1) { set_error("%s: step must be >= 1", who); return GSZ_ERR_INVALID_ARG; }
    if (!gathered && !shard_bf16) { set_error("%s: need gathered and/or shard_bf16 output", who); return GSZ_ERR_INVALID_ARG; }
    const int64_t S = p->shard_len;
    if (S == 0) return GSZ_OK;
    if (!master || !m || !v || !g) { set_error("%s: NULL state buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(master) || misaligned(m) || misaligned(v) || misaligned(g) ||
        (gathered && misaligned(gathered)) || (shard_bf16 && misaligned(shard_bf16))) {
        set_error("%s: a buffer is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED;
    }
    const AdamScalars s = adam_scalars(*hp);
    const int64_t ntile = (S + 511) / 512;
    int64_t blocks = (ntile + kAdamBlock / 64 - 1) / (kAdamBlock / 64);
    if (blocks > kMaxFlatGrid) blocks = kMaxFlatGrid;
    const dim3 grid((unsigned)blocks);
    const int nseg = (int)p->buckets.size();
    if (gathered && shard_bf16)
        hipLaunchKernelGGL((k_adamw<true, true>), grid, dim3(kAdamBlock), 0, stream, master, m, v, g, coef, s, p->d_seg, nseg, (int64_t)owner, S, gathered, shard_bf16);
    else if (gathered)
        hipLaunchKernelGGL((k_adamw<true, false>), grid, dim3(kAdamBlock), 0, stream, master, m, v, g, coef, s, p->d_seg, nseg, (int64_t)owner, S, gathered, shard_bf16);
    else
        hipLaunchKernelGGL((k_adamw<false, true>), grid, dim3(kAdamBlock), 0, stream, master, m, v, g, coef, s, p->d_seg, nseg, (int64_t)owner, S, gathered, shard_bf16);
    return launched(who);
}

extern "C" int gsz_allgather_layout_write(const gsz_plan* p, int32_t owner,
                                          const uint16_t* shard_bf16, uint16_t* gathered,
                                          hipStream_t stream) {
    const char* who = "gsz_allgather_layout_write";
    int rc = check_plan(p, who);
    if (rc) return rc;
    if ((rc = check_owner(p, owner, who))) return rc;
    const int64_t S = p->shard_len;
    if (S == 0) return GSZ_OK;
    if (!shard_bf16 || !gathered) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(shard_bf16) || misaligned(gathered)) { set_error("%s: misaligned buffer", who); return GSZ_ERR_MISALIGNED; }
    const int64_t nvec = S / 8;
    hipLaunchKernelGGL(k_ag_write, dim3(flat_grid((nvec + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream, shard_bf16,
                       p->d_seg, (int)p->buckets.size(), (int64_t)owner, nvec, gathered);
    return launched(who);
}

extern "C" int gsz_bucket_unpack(const gsz_plan* p, const uint16_t* flat, uint16_t* const* params,
                                 hipStream_t stream) {
    return run_pack(p, const_cast<const uint16_t* const*>(params), const_cast<uint16_t*>(flat),
                    kUnpack, stream, "gsz_bucket_unpack");
}

extern "C" int gsz_allreduce_mean(const gsz_plan* p, const uint16_t* const* contrib, float* g_flat,
                                  double* partials, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* who = "gsz_allreduce_mean";
    int rc = check_plan(p, who);
    if (rc) return rc;
    const int P = p->P;
    const int64_t S = p->shard_len;
    if (partials) {
        size_t need = 0;
        gsz_workspace_bytes(S, &need);
        if (!ws || ws_bytes < need) { set_error("%s: workspace of %zu bytes required", who, need); return GSZ_ERR_SIZE; }
        if (misaligned(ws)) { set_error("%s: workspace is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    }
    if (S == 0) {
        if (partials)
            for (int c = 0; c < P; ++c) {
                launch_finalize(static_cast<double*>(ws), 0, partials + c, stream);
                if ((rc = launched(who))) return rc;
            }
        return GSZ_OK;
    }
    if (!g_flat || !contrib) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(g_flat)) { set_error("%s: g_flat is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    for (int q = 0; q < P; ++q) {
        if (!contrib[q]) { set_error("%s: contribution %d is NULL", who, q); return GSZ_ERR_INVALID_ARG; }
        if (misaligned(contrib[q])) { set_error("%s: contribution %d is not 16-byte aligned", who, q); return GSZ_ERR_MISALIGNED; }
    }
    const int64_t nvec = S / 8;
    const int grid = flat_grid((S + kRedTile - 1) / kRedTile);
    const dim3 gr(grid);
    const int pow2 = (P & (P - 1)) == 0;
    const float invP = pow2 ? 1.0f / (float)P : 0.0f;
    const int nseg = (int)p->buckets.size();
    const bool norm = partials != nullptr;
    double* wsd = static_cast<double*>(ws);
    // chunk c of every bucket, summed in ring order ending at rank c; its norm
    // partial is finalized before the next launch reuses the workspace (stream order)
    for (int c = 0; c < P; ++c) {
        RankPtrs rp{};
        for (int k = 0; k < P; ++k) rp.p[k] = contrib[(c + 1 + k) % P];
        switch (P) {
            case 2: launch_reduce<2>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
            case 4: launch_reduce<4>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
            case 8: launch_reduce<8>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
            case 16: launch_reduce<16>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
            case 32: launch_reduce<32>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
            case 64: launch_reduce<64>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
            default: launch_reduce<0>(norm, true, gr, stream, rp, P, invP, pow2, p->d_seg, nseg, c, nvec, g_flat, wsd, true); break;
        }
        if ((rc = launched(who))) return rc;
        if (norm) {
            launch_finalize(wsd, grid, partials + c, stream);
            if ((rc = launched(who))) return rc;
        }
    }
    return GSZ_OK;
}

extern "C" int gsz_adamw_step(float* master, float* m, float* v, const float* g, int64_t n,
                              const float* coef, const gsz_adamw_hp* hp, uint16_t* out_bf16,
                              hipStream_t stream) {
    const char* who = "gsz_adamw_step";
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (!hp || !coef || n < 0) { set_error("%s: bad arguments", who); return GSZ_ERR_INVALID_ARG; }
    if (hp->step < 1) { set_error("%s: step must be >= 1", who); return GSZ_ERR_INVALID_ARG; }
    if (n % 8 != 0) { set_error("%s: n must be a multiple of 8 (got %lld)", who, (long long)n); return GSZ_ERR_SIZE; }
    if (n == 0) return GSZ_OK;
    if (!master || !m || !v || !g || !out_bf16) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(master) || misaligned(m) || misaligned(v) || misaligned(g) || misaligned(out_bf16)) {
        set_error("%s: a buffer is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED;
    }
    const AdamScalars s = adam_scalars(*hp);
    const int64_t ntile = (n + 511) / 512;
    int64_t blocks = (ntile + kAdamBlock / 64 - 1) / (kAdamBlock / 64);
    if (blocks > kMaxFlatGrid) blocks = kMaxFlatGrid;
    hipLaunchKernelGGL((k_adamw<false, true>), dim3((unsigned)blocks), dim3(kAdamBlock), 0, stream, master, m, v, g,
                       coef, s, nullptr, 0, (int64_t)0, n, nullptr, out_bf16);
    return launched(who);
}
