// Pack kernels: bucket pack, unpack and bf16 accumulation, and the fp32
// accumulation buckets.  Pages cited (title, section): see gsz.h.
#pragma once

#include "gsz_device.h"

#pragma clang fp contract(off)

namespace {

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
// tile}; lut maps a tile to its tensor in one load (a binary search over 256
// tensors, eight dependent loads before a block's first data load, cost 7% of
// the copy rate on a 7B model).  One block per tile of kPackTile = 8 *
// kPackBlock elements (one 16-byte vector per lane), the grid covering the
// batch's tiles [t_begin, t_end): short blocks dispatched in address order keep
// the lines in flight close together, which MI355X's HBM rewards over
// long-running grid-stride blocks.  Grids are capped below the dispatch limit;
// blocks then stride over the remaining tiles.
template <int MODE>
__global__ __launch_bounds__(kPackBlock) void k_pack(PackPtrs pp, const int64_t* __restrict__ tab,
                                                 const uint64_t* __restrict__ tlut, int tshift,
                                                 int k0, int nk, int64_t t_begin, int64_t t_end,
                                                 uint16_t* __restrict__ flat) {
    const int tid = threadIdx.x;
    for (int64_t tile = t_begin + blockIdx.x; tile < t_end; tile += gridDim.x) {
        const int k = lut_find(tlut, tshift, tab + 2, 3, tile, k0, k0 + nk - 1);   // block-uniform
        const int64_t n = tab[3 * k + 1];
        const int64_t j0 = (tile - tab[3 * k + 2]) * gsz::kPackTile;
        const int64_t j1 = j0 + gsz::kPackTile < n ? j0 + gsz::kPackTile : n;
        const uint16_t* __restrict__ src = MODE == kUnpack ? flat + tab[3 * k] : pp.p[k - k0];
        uint16_t* __restrict__ dst = MODE == kUnpack ? const_cast<uint16_t*>(pp.p[k - k0]) : flat + tab[3 * k];
        const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
        if (vec && j1 - j0 == gsz::kPackTile) {
            static_assert(gsz::kPackTile == 8 * kPackBlock, "one vector per lane");
            // Nontemporal hints on both sides: the bytes are used once (2-3% faster).
            // Buffer descriptors at the tile, nontemporal loads, nontemporal
            // sc1 stores: 2.6% (pack) and 3.6% (bf16 accumulation) faster than
            // nontemporal 64-bit-address accesses on the 7B share.
            const BufRes rs = buf_res(src + j0, 2 * gsz::kPackTile), rd = buf_res(dst + j0, 2 * gsz::kPackTile);
            u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * tid, 0, kCpNt);
            if (MODE == kAccumulate) w = add_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rd, 16 * tid, 0, kCpNt), w);
            __builtin_amdgcn_raw_buffer_store_b128(w, rd, 16 * tid, 0, kCpNtSc1);
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
// f32(grad_t[j]), one IEEE fp32 addition.  Tiles as k_pack, in blocks of
// kF32Block = 128 lanes: in a full tile lane l takes elements 4l..4l+3 (one
// 8-byte bf16 load), so each 16-byte fp32 load and store of a wave covers
// whole lines; with nontemporal hints on every access this runs 5-6% faster
// than one 16-byte bf16 load per lane widened into two half-line fp32 stores,
// and one group per lane 3% faster than 64 lanes with two groups each.
__device__ __forceinline__ void stf8(float* p, const float a[8]) {
    stf4(p, f32x4{a[0], a[1], a[2], a[3]});
    stf4(p + 4, f32x4{a[4], a[5], a[6], a[7]});
}
template <bool ACC>
__global__ __launch_bounds__(kF32Block) void k_pack_f32(PackPtrs pp, const int64_t* __restrict__ tab,
                                                     const uint64_t* __restrict__ tlut, int tshift,
                                                     int k0, int nk, int64_t t_begin, int64_t t_end,
                                                     float* __restrict__ flat) {
    const int tid = threadIdx.x;
    for (int64_t tile = t_begin + blockIdx.x; tile < t_end; tile += gridDim.x) {
        const int k = lut_find(tlut, tshift, tab + 2, 3, tile, k0, k0 + nk - 1);   // block-uniform
        const int64_t n = tab[3 * k + 1];
        const int64_t j0 = (tile - tab[3 * k + 2]) * gsz::kPackTile;
        const int64_t j1 = j0 + gsz::kPackTile < n ? j0 + gsz::kPackTile : n;
        const uint16_t* __restrict__ src = pp.p[k - k0];
        float* __restrict__ dst = flat + tab[3 * k];
        const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
        if (vec && j1 - j0 == gsz::kPackTile) {
            static_assert(gsz::kPackTile == 4 * kF32Block, "one group of 4 elements per lane");
            // Lane l: elements 4l..4l+3 of the tile.  Buffer descriptors at the
            // tile as in k_pack: 5.9% faster for the fp32 accumulation (7B share).
            const BufRes rs = buf_res(src + j0, 2 * gsz::kPackTile), rd = buf_res(dst + j0, 4 * gsz::kPackTile);
            const u32x2 wa = __builtin_amdgcn_raw_buffer_load_b64(rs, 8 * tid, 0, kCpNt);
            f32x4 xa = f32x4{bf16_lo(wa.x), bf16_hi(wa.x), bf16_lo(wa.y), bf16_hi(wa.y)};
            if (ACC) {
                const f32x4 da = bldf4_nt(rd, 16 * tid);
                xa = f32x4{da.x + xa.x, da.y + xa.y, da.z + xa.z, da.w + xa.w};
            }
            bstf4<kCpNtSc1>(rd, 16 * tid, xa);
        } else if (vec) {
            const int64_t jv = j0 + ((j1 - j0) & ~(int64_t)7);
            for (int64_t j = j0 + 8 * tid; j < jv; j += 8 * kF32Block) {
                float a[8];
                widen8(ld16(src + j), a);
                if (ACC) {
                    const f32x4 d0 = ldf4(dst + j), d1 = ldf4(dst + j + 4);
                    a[0] = d0.x + a[0]; a[1] = d0.y + a[1]; a[2] = d0.z + a[2]; a[3] = d0.w + a[3];
                    a[4] = d1.x + a[4]; a[5] = d1.y + a[5]; a[6] = d1.z + a[6]; a[7] = d1.w + a[7];
                }
                stf8(dst + j, a);
            }
            for (int64_t j = jv + tid; j < j1; j += kF32Block) {
                const float x = __uint_as_float((uint32_t)src[j] << 16);
                dst[j] = ACC ? dst[j] + x : x;
            }
        } else {
            for (int64_t j = j0 + tid; j < j1; j += kF32Block) {
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

}  // namespace
