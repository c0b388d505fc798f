// The fused AdamW update with its bf16 output in all-gather or shard layout, and
// the standalone all-gather layout writer.  Pages cited (title, section): see gsz.h.
#pragma once

#include "gsz_device.h"

#pragma clang fp contract(off)

namespace {

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

// One block (one wave) updates kAdamTile = 256 consecutive shard elements per
// iteration; lane l takes elements 4l..4l+3, so every 16-byte load and store
// instruction covers 1 KiB of whole 128-byte lines (a lane that loads 32
// contiguous bytes as two 16-byte halves makes each instruction touch half of
// every line, and half-line misses to the same line are fetched twice).  Every
// access goes through a buffer descriptor based at the tile: loads
// nontemporal, stores nontemporal with sc1.  The bf16 result goes out as 8
// bytes per lane, in shard layout and/or at its all-gather position (glen
// elements in `gathered`); gwide: a tile's all-gather positions may span
// 2^31 bytes or more (a bucket of over 2^30 elements), so those stores take
// 64-bit addresses.
template <bool GATH, bool SHARD>
__global__ __launch_bounds__(kAdamBlock) void k_adamw(float* __restrict__ master, float* __restrict__ m,
                                                      float* __restrict__ v, const float* __restrict__ g,
                                                      const float* __restrict__ coefp, AdamScalars s,
                                                      const int64_t* __restrict__ seg,
                                                      const uint64_t* __restrict__ slut, int sshift,
                                                      int64_t owner, int64_t S,
                                                      uint16_t* __restrict__ gathered, int64_t glen,
                                                      int gwide,
                                                      uint16_t* __restrict__ shard_bf16) {
    static_assert(kAdamBlock == 64 && kAdamTile == 4 * kAdamBlock, "one wave, 4 elements per lane");
    const int lane = threadIdx.x;
    const int64_t ntile = (S + kAdamTile - 1) / kAdamTile;
    const float coef = *coefp;
    int64_t t = blockIdx.x;
    SegCursor cur{seg, owner, 0, 0, 0};
    if (GATH && t < ntile) cur.seek(t * kAdamTile, slut, sshift);   // block-uniform: scalar loads
    for (; t < ntile; t += gridDim.x) {
        const int64_t base = t * kAdamTile;
        const int64_t i = base + 4 * lane;
        const int64_t fb = GATH ? uniform64(cur.map(base)) : 0;    // the tile's first all-gather position
        if (i < S) {                           // S and i are multiples of 4
            const int64_t rem = (S - base) * 4;
            const BufRes rg = buf_res(g + base, rem), rt = buf_res(master + base, rem);
            const BufRes rm = buf_res(m + base, rem), rv = buf_res(v + base, rem);
            const int o = 16 * lane;
            const f32x4 g4 = bldf4_nt(rg, o);
            const f32x4 t4 = bldf4_nt(rt, o), m4 = bldf4_nt(rm, o), v4 = bldf4_nt(rv, o);
            float th[4] = {t4.x, t4.y, t4.z, t4.w};
            float mm[4] = {m4.x, m4.y, m4.z, m4.w};
            float vv[4] = {v4.x, v4.y, v4.z, v4.w};
            const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) adamw1(th[j], mm[j], vv[j], gg[j], coef, s);
            bstf4<kCpNtSc1>(rt, o, f32x4{th[0], th[1], th[2], th[3]});
            bstf4<kCpNtSc1>(rm, o, f32x4{mm[0], mm[1], mm[2], mm[3]});
            bstf4<kCpNtSc1>(rv, o, f32x4{vv[0], vv[1], vv[2], vv[3]});
            const u32x2 p = u32x2{bf16_rne(th[0]) | (bf16_rne(th[1]) << 16),
                                  bf16_rne(th[2]) | (bf16_rne(th[3]) << 16)};
            if (GATH) {
                const int64_t fi = cur.map(i);
                if (gwide) st8_nt(gathered + fi, p);
                else bst8<kCpNtSc1>(buf_res(gathered + fb, (glen - fb) * 2), (int)(fi - fb) * 2, p);
            }
            if (SHARD) bst8<kCpNtSc1>(buf_res(shard_bf16 + base, (S - base) * 2), 8 * lane, p);
        }
    }
}

// gathered[i + delta_b] = shard[i] for shard index i of bucket b.  One block
// per 2048-element tile (grid-striding past the dispatch limit), lane l moving
// elements 8l..8l+7 of its wave's 512 (16 bytes): through buffer descriptors
// based at the tile's first element and its first all-gather position, unless
// gwide (a tile's positions may span 2^31 bytes or more), where the stores take
// 64-bit addresses.  glen: elements in `gathered`.
__global__ __launch_bounds__(kBlock) void k_ag_write(const uint16_t* __restrict__ shard,
                                                     const int64_t* __restrict__ seg,
                                                     const uint64_t* __restrict__ slut, int sshift,
                                                     int64_t owner, int64_t nvec,
                                                     uint16_t* __restrict__ gathered, int64_t glen,
                                                     int gwide) {
    const int64_t S = nvec * 8;
    SegCursor cur{seg, owner, 0, 0, 0};
    int64_t t = (int64_t)blockIdx.x * kRedTile;
    if (t < S) cur.seek(t, slut, sshift);                  // block-uniform: scalar loads
    for (; t < S; t += (int64_t)gridDim.x * kRedTile) {
        const int64_t fb = uniform64(cur.map(t));          // the tile's first all-gather position
        const int64_t i = t + 8 * threadIdx.x;
        if (i < S) {                                       // S and i are multiples of 8
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(buf_res(shard + t, (S - t) * 2),
                                                                  16 * threadIdx.x, 0, kCpNt);
            const int64_t fi = cur.map(i);
            if (gwide) st16_nt(gathered + fi, w);
            else __builtin_amdgcn_raw_buffer_store_b128(w, buf_res(gathered + fb, (glen - fb) * 2),
                                                        (int)(fi - fb) * 2, 0, kCpNtSc1);
        }
    }
}

}  // namespace
