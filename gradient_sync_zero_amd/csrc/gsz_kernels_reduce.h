// Reduction kernels: the ring-order mean of P contributions (bf16 or fp32, with
// the fused norm partial), the standalone squared norm, the fixed-order
// finalize and the clip coefficient.  Pages cited (title, section): see gsz.h.
#pragma once

#include "gsz_device.h"

#pragma clang fp contract(off)

namespace {

// Loads per group for a compile-time P: the largest divisor of PS up to cap, so
// that the groups read contributions 0..PS-1 and none past them.
constexpr int load_group(int ps, int cap) {
    for (int g = cap < ps ? cap : ps; g > 1; --g)
        if (ps % g == 0) return g;
    return 1;
}

// ---------------------------------------------------------- reduce-mean --

// Contribution layouts as the reduce kernels see them: bucket-flat (the
// owner's chunks read through the plan's segments), shard-compact (index i of
// every contribution), or rank-interleaved (one receive buffer in which rank
// q's values for shard elements [512t, 512t + 512) sit at (t*P + q)*512; the
// host passes p[k] = buffer + q_k * 512, so index i reads p[k] + ilv_index(i)).
// kLayFlatWide is bucket-flat for a plan whose tiles span 2^31 bytes or more
// of a contribution (see k_reduce_mean_lc); kernels other than the
// lane-contiguous one treat it as kLayFlat.
constexpr int kLayFlat = 0, kLayCompact = 1, kLayInterleaved = 2, kLayFlatWide = 3;
constexpr int64_t kIlvPiece = 512;
static_assert(kIlvPiece == GSZ_INTERLEAVE_PIECE, "the header's piece size");

__device__ __forceinline__ int64_t ilv_index(int64_t i, int P) {
    return (i >> 9) * ((int64_t)P << 9) + (i & (kIlvPiece - 1));
}

template <int LAY>
__device__ __forceinline__ int64_t contrib_index(SegCursor& cur, int64_t i, int P) {
    if constexpr (LAY == kLayFlat || LAY == kLayFlatWide) return cur.map(i);
    else if constexpr (LAY == kLayInterleaved) return ilv_index(i, P);
    else return i;
}

// a[0..8) = the ring-order mean of the 8 consecutive elements at offset off of
// every contribution: (((c0 + c1) + c2) + ... + c_{P-1}) / P with rp.p[k] the
// contribution of rank (owner+1+k) mod P, so the owner's own value is added
// last.  PS > 0 fixes P at compile time; loads are issued in groups of up to
// 32 ranks before their adds so many 16-byte requests are in flight.  W16: the
// partial sum is rounded to bf16 after every addition (a ring whose wire
// carries bf16 partial sums); the final division stays fp32.  RG: loads in
// flight per group of the runtime-P loop: 8, one contribution at a time for the
// last (P-1) mod 8; or (where few waves share a CU) 32, then 8, then the rest as
// one group.
template <int PS, bool W16, int RG = 8>
__device__ __forceinline__ void ring_mean8(const RankPtrs& rp, int P, float invP, int pow2,
                                           int64_t off, float a[8]) {
    if constexpr (PS > 0) {
        // up to 32 loads before their adds (at P = 64 that measured 1.4% faster than 16)
        constexpr int G = load_group(PS, 32);
        static_assert(PS % G == 0, "the groups cover exactly the P contributions");
#pragma unroll
        for (int k0 = 0; k0 < PS; k0 += G) {
            u32x4 w[G];
#pragma unroll
            for (int j = 0; j < G; ++j) w[j] = ld16_nt(rp.p[k0 + j] + off);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (k0 + j == 0) widen8(w[j], a);
                else { add8(w[j], a); if (W16) round8_bf16(a); }
            }
        }
    } else {
        widen8(ld16_nt(rp.p[0] + off), a);
        int k = 1;
        if constexpr (RG >= 32) {
            for (; k + 32 <= P; k += 32) {
                u32x4 w[32];
#pragma unroll
                for (int j = 0; j < 32; ++j) w[j] = ld16_nt(rp.p[k + j] + off);
#pragma unroll
                for (int j = 0; j < 32; ++j) { add8(w[j], a); if (W16) round8_bf16(a); }
            }
        }
        for (; k + 8 <= P; k += 8) {
            u32x4 w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = ld16_nt(rp.p[k + j] + off);
#pragma unroll
            for (int j = 0; j < 8; ++j) { add8(w[j], a); if (W16) round8_bf16(a); }
        }
        if constexpr (RG >= 32) {
            // The last (P-1) mod 8 contributions as one group: slots past P
            // reload contribution k (in bounds, the same lines) and are not
            // added.  k and P are wave-uniform, so nothing diverges.
            if (k < P) {
                u32x4 w[7];
#pragma unroll
                for (int j = 0; j < 7; ++j) w[j] = ld16_nt(rp.p[k + j < P ? k + j : k] + off);
#pragma unroll
                for (int j = 0; j < 7; ++j)
                    if (k + j < P) { add8(w[j], a); if (W16) round8_bf16(a); }
            }
        } else {
            for (; k < P; ++k) { add8(ld16_nt(rp.p[k] + off), a); if (W16) round8_bf16(a); }
        }
    }
    if (PS > 0 ? ((PS & (PS - 1)) == 0) : pow2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = a[j] * invP;   // exact: invP is a power of two
    } else {
        const float fP = (float)P;
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = a[j] / fP;
    }
}

// g[i] = ring_mean8 of element i, one tile of kRedTile shard elements per
// block.  Each lane handles 8 consecutive shard elements per iteration (one
// 16-byte load per rank).  With OUTFLAT (bucket-flat input only) g is indexed
// by flat position instead of shard index: P launches, one per chunk owner,
// give the all-reduce result.  Loads and stores are nontemporal (2% faster at
// P = 8, 5% at P = 64 than plain ones).  This kernel serves P > 16 on shards
// below the burst kernel's size and on the bf16 wire (compile-time P for 24,
// 32, 64 and 96, its runtime-P loop for the others) and the all-reduce;
// P <= 16 runs k_reduce_mean_lc below.  LAY is one of the layouts above
// (kLayFlat for OUTFLAT).
template <int PS, bool NORM, int LAY, bool OUTFLAT = false, bool W16 = false>
__global__ __launch_bounds__(kBlock) void k_reduce_mean(RankPtrs rp, int P, float invP, int pow2,
                                                        const int64_t* __restrict__ seg,
                                                        const uint64_t* __restrict__ slut, int sshift,
                                                        int64_t owner, int64_t nvec,
                                                        float* __restrict__ g,
                                                        double* __restrict__ ws) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    const int64_t bx = xcd_remap(blockIdx.x, gridDim.x);      // logical block: tile bx
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr bool FLAT = LAY == kLayFlat;
    static_assert(!OUTFLAT || FLAT, "the all-gather-position output reads bucket-flat input");
    // The results reach HBM as whole-line stores: each wave's 512 results pass
    // through LDS so that one store instruction writes 1 KiB contiguous (lane l
    // writes what lane l/2 computed).  A lane storing 32 contiguous bytes as two
    // 16-byte stores makes each instruction cover half of every line, and such
    // nontemporal half-line stores reached HBM as 9% more write bytes.  So the
    // loop is wave-uniform: lanes past the end stay in it, load position 0 of
    // every contribution (in bounds) and discard the result.
    __shared__ float stage[OUTFLAT ? 1 : kBlock * 8];
    double sq = 0.0;
    SegCursor cur{seg, owner, 0, 0, 0};
    const int64_t S = nvec * 8;
    if (FLAT && bx * kRedTile < S) cur.seek(bx * kRedTile, slut, sshift);  // uniform: scalar loads
    for (int64_t v0 = bx * kBlock + wave * 64; v0 < nvec; v0 += stride) {
        const int64_t v = v0 + lane;
        const bool ok = v < nvec;
        const int64_t i = v * 8;
        const int64_t off = ok ? contrib_index<LAY>(cur, i, PS > 0 ? PS : P) : 0;
        float a[8];
        ring_mean8<PS, W16>(rp, P, invP, pow2, off, a);
        if constexpr (OUTFLAT) {
            if (ok) {                           // all-reduce output: the flat position
                stf4_nt(g + off, f32x4{a[0], a[1], a[2], a[3]});
                stf4_nt(g + off + 4, f32x4{a[4], a[5], a[6], a[7]});
            }
        } else {
            float* st = stage + wave * 512;
            *reinterpret_cast<f32x4*>(st + 8 * lane) = f32x4{a[0], a[1], a[2], a[3]};
            *reinterpret_cast<f32x4*>(st + 8 * lane + 4) = f32x4{a[4], a[5], a[6], a[7]};
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            const f32x4 lo = *reinterpret_cast<const f32x4*>(st + 4 * lane);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(st + 256 + 4 * lane);
            const int64_t e0 = v0 * 8 + 4 * lane, e1 = e0 + 256;
            if (e0 < S) stf4_nt(g + e0, lo);
            if (e1 < S) stf4_nt(g + e1, hi);
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();  // the next iteration's writes come after these reads
        }
        if (NORM && ok) {
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

// ------------------------------------------------------ burst reduce-mean --

// The same g as k_reduce_mean, for large shards at P > 16, with g reaching HBM
// in bursts.  Stores of g scattered among the contribution reads cost the
// read stream far more than their bytes (without its stores the one-tile
// kernel takes 14-23% less time, and writing half as many g lines costs 82%
// as much time as writing all of them).  So one block per CU (its 128 KiB of
// LDS admit no second one) walks chunks of kBurstElems shard elements (wave w
// takes a chunk's 512-element rows w, w + 4, ...) and keeps the rows it
// reduces in LDS, to write them in one of two ways (`chunked`, chosen by the
// host from P and S):
//  - chunk writes: once a chunk is reduced, the whole block writes its 128 KiB
//    as one run (3-5% faster than the one-tile-per-block launch at P = 64);
//  - clock windows: each wave keeps its rows in its own ring of kRingRows rows
//    and writes what it holds, each row as two whole-line stores per lane,
//    when the chip-wide 100 MHz constant clock is in a write window (clock &
//    pmask below `window`) or when the ring is full.  All CUs read the same
//    clock, so their writes fall in the same windows and the DRAM sees a few
//    long write runs between long read runs: 1.5-7% faster than chunk writes
//    on large shards at P = 24-128.  The clock is read as a row starts, so
//    that its latency hides under the row's loads (read as a row ended and
//    taken modulo a period that was no power of two, it made the kernel 4%
//    slower at P = 17).
// Chunks go to XCDs in contiguous ranges (burst_work); the norm partials, one
// per block, are summed in block order by the finalize.
constexpr int kBurstRows = 64;
constexpr int64_t kBurstElems = (int64_t)kBurstRows * 512;
constexpr int kRingRows = 16;                                  // per wave: 32 KiB of fp32

// The work of block b in a grid of G blocks over S shard elements.  The blocks
// with b mod 8 == x run on XCD x; that class takes a contiguous share of the
// chunks in proportion to its n_x blocks, and its blocks advance through the
// share together: `rounds` times, block b takes chunk first + i * n_x.  What
// is left of the share after the last round in which every block of the class
// has a whole chunk (fewer than n_x chunks) is split into n_x pieces of whole
// 512-element rows, [tail0, tail1) for this block, so that the blocks of a
// class finish together instead of half of them idling for a chunk's time.
// Every element goes to exactly one block; a piece has at most kBurstRows rows.
struct BurstWork { int64_t first, rounds, step, tail0, tail1; };

__device__ __forceinline__ BurstWork burst_work(int64_t S, int64_t G, int64_t b) {
    const int64_t chunks = (S + kBurstElems - 1) / kBurstElems;
    const int64_t x = b % kXcds, kb = b / kXcds;
    int64_t before = 0;                                  // blocks in the classes below x
    for (int64_t y = 0; y < x; ++y) before += (G - y + kXcds - 1) / kXcds;
    const int64_t nx = (G - x + kXcds - 1) / kXcds;      // blocks in class x (>= 1: b is one)
    const int64_t c0 = chunks * before / G, c1 = chunks * (before + nx) / G;
    BurstWork w;
    w.first = c0 + kb;
    w.step = nx;
    w.rounds = (c1 - c0) / nx;
    const int64_t e0 = (c0 + w.rounds * nx) * kBurstElems;
    const int64_t e1 = c1 * kBurstElems < S ? c1 * kBurstElems : S;
    const int64_t rows = e1 > e0 ? (e1 - e0 + 511) / 512 : 0;  // fewer than n_x chunks' rows
    const int64_t t0 = e0 + rows * kb / nx * 512, t1 = e0 + rows * (kb + 1) / nx * 512;
    w.tail0 = t0 < e1 ? t0 : e1;
    w.tail1 = t1 < e1 ? t1 : e1;
    return w;
}

template <int PS, bool NORM, int LAY, bool W16 = false>
__global__ __launch_bounds__(kBlock) void k_reduce_burst(RankPtrs rp, int P, float invP, int pow2,
                                                         const int64_t* __restrict__ seg,
                                                         const uint64_t* __restrict__ slut, int sshift,
                                                         int64_t owner, int64_t S,
                                                         float* __restrict__ g,
                                                         double* __restrict__ ws,
                                                         int chunked, uint32_t pmask,
                                                         uint32_t window) {
    // Per wave a ring of kRingRows rows; with chunk writes the same 128 KiB
    // hold one chunk, row r at r * 512.
    __shared__ float lds[kBurstElems];
    __shared__ int64_t row_all[kBlock / 64][kRingRows];
    static_assert(kBlock / 64 * kRingRows * 512 == kBurstElems, "rings fill the chunk buffer");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float* const chunk = lds;
    float* const ring = lds + wave * kRingRows * 512;
    int64_t* const row_at = row_all[wave];  // shard index of each held row's first element
    const BurstWork w = burst_work(S, gridDim.x, blockIdx.x);
    double sq = 0.0;
    SegCursor cur{seg, owner, 0, 0, 0};
    int head = 0, held = 0;                // wave-uniform: slots [head - held, head) are held
    // Writes the held rows: lane l stores elements 4l..4l+3 and 256+4l.. of
    // each (whole lines per instruction), those below S.
    auto flush = [&]() {
        for (int k = 0; k < held; ++k) {
            const int slot = (head - held + k + kRingRows) % kRingRows;
            const float* src = ring + slot * 512;
            const int64_t e0 = row_at[slot] + 4 * lane, e1 = e0 + 256;
            if (e0 < S) stf4_nt(g + e0, *reinterpret_cast<const f32x4*>(src + 4 * lane));
            if (e1 < S) stf4_nt(g + e1, *reinterpret_cast<const f32x4*>(src + 256 + 4 * lane));
        }
        held = 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();   // a slot is reused only after every lane read it
    };
    // Elements [base, base + n) of the shard, 0 < n <= kBurstElems, n and base
    // multiples of 8.
    auto piece = [&](int64_t base, int64_t n) {
        if (LAY == kLayFlat) cur.seek(base, slut, sshift);                   // uniform: scalar loads
        double csq = 0.0;          // this piece's squares, added to sq once: shorter fp64 sums
        // Lanes past n load position 0 of every contribution (in bounds;
        // unconditional loads keep them in flight together) and their results
        // are never stored to g.
        for (int r = wave; (int64_t)r * 512 < n; r += kBlock / 64) {
            // Read before the row's loads, so that the clock's latency hides under theirs.
            const uint32_t t = chunked ? 0u : (uint32_t)__builtin_amdgcn_s_memrealtime() & pmask;
            const int j = r * 512 + 8 * lane;
            const bool ok = j < n;
            const int64_t off = ok ? contrib_index<LAY>(cur, base + j, PS > 0 ? PS : P) : 0;
            float a[8];
            ring_mean8<PS, W16, 32>(rp, P, invP, pow2, off, a);
            float* st = chunked ? chunk + r * 512 : ring + head * 512;
            *reinterpret_cast<f32x4*>(st + 8 * lane) = f32x4{a[0], a[1], a[2], a[3]};
            *reinterpret_cast<f32x4*>(st + 8 * lane + 4) = f32x4{a[4], a[5], a[6], a[7]};
            if (NORM && ok) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const double d = (double)a[k];
                    csq = __fma_rn(d, d, csq);                      // d*d is exact in fp64
                }
            }
            if (chunked) continue;
            if (lane == 0) row_at[head] = base + r * 512;
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();   // the row is in LDS before any lane reads it
            head = (head + 1) % kRingRows;
            ++held;
            if (held == kRingRows || t < window) flush();
        }
        sq = sq + csq;
        if (chunked) {                     // the whole block writes the piece's n elements
            __syncthreads();
            for (int e = 4 * threadIdx.x; e < n; e += 4 * kBlock)
                stf4_nt(g + base + e, *reinterpret_cast<const f32x4*>(chunk + e));
            __syncthreads();
        }
    };
    for (int64_t i = 0; i < w.rounds; ++i) {
        const int64_t base = (w.first + i * w.step) * kBurstElems;
        piece(base, S - base < kBurstElems ? S - base : kBurstElems);
    }
    if (w.tail1 > w.tail0) piece(w.tail0, w.tail1 - w.tail0);
    flush();
    if (NORM) {
        const double s = block_sum(sq);
        if (threadIdx.x == 0) ws[blockIdx.x] = s;
    }
}

// The same ring-order mean in a lane-contiguous layout, for fp32 contributions
// (fp32 accumulation buckets, fp32 on the ring's wire) and for bf16 ones at
// small P.  A wave owns 512 shard elements of its block's tile as two groups of
// 256; lane l handles elements 4l..4l+3 of each (an 8-byte bf16 or 16-byte
// fp32 load per contribution and group), so every 16-byte fp32 store of a wave
// covers whole lines.  With nontemporal stores that matters: k_reduce_mean's
// lanes store 32 contiguous bytes as two half-line stores, which reach HBM as
// 9% more write bytes, and this layout is 4-5% faster at P = 8-16.  At P = 64
// its twice as many (half-size) bf16 loads make it 6-7% slower, so the larger
// P keep k_reduce_mean.  OUTFLAT and W16 as there; blocks, XCD order and norm
// partials as there; LAY as there.
//
// Contributions are read through buffer descriptors based at the tile's first
// position in each contribution (clen elements per contribution buffer), and g
// is written through one based at the tile's first g element (sc1 stores).  A
// lane's offsets are relative to the tile, so they stay below 2^31 bytes for
// every layout except a bucket-flat plan whose tiles span more (a bucket of
// over 2^29 elements next to a chunk boundary): the host passes kLayFlatWide
// for that, and the kernel reads through 64-bit addresses instead.
template <typename T, int PS, bool NORM, int LAY, bool OUTFLAT = false, bool W16 = false>
__global__ __launch_bounds__(kBlock) void k_reduce_mean_lc(RankPtrsT<T> rp, int P, float invP, int pow2,
                                                           const int64_t* __restrict__ seg,
                                                           const uint64_t* __restrict__ slut, int sshift,
                                                           int64_t owner, int64_t S, int64_t clen,
                                                           float* __restrict__ g,
                                                           double* __restrict__ ws) {
    constexpr bool FLAT = LAY == kLayFlat || LAY == kLayFlatWide;
    constexpr bool BUF = LAY != kLayFlatWide;
    static_assert(!OUTFLAT || FLAT, "the all-gather-position output reads bucket-flat input");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t bx = xcd_remap(blockIdx.x, gridDim.x);
    double sq = 0.0;
    SegCursor cur{seg, owner, 0, 0, 0};
    int64_t t = bx * kRedTile;
    if (FLAT && t < S) cur.seek(t, slut, sshift);                     // uniform: scalar loads
    const float fP = (float)P;
    const f32x4 zero = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (; t < S; t += (int64_t)gridDim.x * kRedTile) {
        const int64_t i0 = t + 512 * wave + 4 * lane, i1 = i0 + 256;
        const bool ok0 = i0 < S, ok1 = i1 < S;               // S and i are multiples of 4
        // Past the end a lane reads the tile's first position of each
        // contribution (in bounds) and discards the result: loads under a
        // condition became one branch and one full wait per load, serialising them.
        // tb: the contribution index of the tile's first element (the same in
        // every lane; the cursor only moves forward, so mapping t first is fine).
        const int64_t tb = uniform64(contrib_index<LAY>(cur, t, PS > 0 ? PS : P));
        const int64_t off0 = ok0 ? contrib_index<LAY>(cur, i0, PS > 0 ? PS : P) : tb;
        const int64_t off1 = ok1 ? contrib_index<LAY>(cur, i1, PS > 0 ? PS : P) : tb;
        const int r0 = (int)(off0 - tb) * (int)sizeof(T), r1 = (int)(off1 - tb) * (int)sizeof(T);
        const int64_t rbytes = (clen - tb) * (int64_t)sizeof(T);
        auto ld = [&](int k, bool second) -> f32x4 {
            if constexpr (BUF) return bld4f(buf_res(rp.p[k] + tb, rbytes), second ? r1 : r0, rp.p[k]);
            else return ld4f_nt(rp.p[k] + (second ? off1 : off0));
        };
        f32x4 a = zero, b = zero;
        if constexpr (PS > 0) {
            constexpr int G = load_group(PS, 16);
            static_assert(PS % G == 0, "the groups cover exactly the P contributions");
#pragma unroll
            for (int k0 = 0; k0 < PS; k0 += G) {
                f32x4 w0[G], w1[G];
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    w0[j] = ld(k0 + j, false);
                    w1[j] = ld(k0 + j, true);
                }
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if (k0 + j == 0) { a = w0[j]; b = w1[j]; continue; }
                    a = add4(a, w0[j]);
                    b = add4(b, w1[j]);
                    if (W16) { a = round4_bf16(a); b = round4_bf16(b); }
                }
            }
        } else {
            a = ld(0, false);
            b = ld(0, true);
            int k = 1;
            for (; k + 8 <= P; k += 8) {                      // 16 loads in flight, then the adds
                f32x4 w0[8], w1[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    w0[j] = ld(k + j, false);
                    w1[j] = ld(k + j, true);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    a = add4(a, w0[j]);
                    b = add4(b, w1[j]);
                    if (W16) { a = round4_bf16(a); b = round4_bf16(b); }
                }
            }
            for (; k < P; ++k) {
                a = add4(a, ld(k, false));
                b = add4(b, ld(k, true));
                if (W16) { a = round4_bf16(a); b = round4_bf16(b); }
            }
        }
        if (PS > 0 ? ((PS & (PS - 1)) == 0) : pow2) {
            a = f32x4{a.x * invP, a.y * invP, a.z * invP, a.w * invP};   // exact: a power of two
            b = f32x4{b.x * invP, b.y * invP, b.z * invP, b.w * invP};
        } else {
            a = f32x4{a.x / fP, a.y / fP, a.z / fP, a.w / fP};
            b = f32x4{b.x / fP, b.y / fP, b.z / fP, b.w / fP};
        }
        if constexpr (OUTFLAT && BUF) {                      // all-reduce output: the flat position
            const BufRes rg = buf_res(g + tb, (clen - tb) * 4);
            if (ok0) bstf4<kCpSc1>(rg, (int)(off0 - tb) * 4, a);
            if (ok1) bstf4<kCpSc1>(rg, (int)(off1 - tb) * 4, b);
        } else if constexpr (OUTFLAT) {
            if (ok0) stf4_nt(g + off0, a);
            if (ok1) stf4_nt(g + off1, b);
        } else {
            const BufRes rg = buf_res(g + t, (S - t) * 4);
            if (ok0) bstf4<kCpSc1>(rg, (int)(i0 - t) * 4, a);
            if (ok1) bstf4<kCpSc1>(rg, (int)(i1 - t) * 4, b);
        }
        if (NORM) {
            a = ok0 ? a : zero;
            b = ok1 ? b : zero;
            const double d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) sq = __fma_rn(d[j], d[j], sq);
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
                const f32x4 x = ldf4_nt(g + base + h * (4 * kBlock) + 4 * tid);   // 6% faster
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

}  // namespace
