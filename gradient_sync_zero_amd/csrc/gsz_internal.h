// Internal declarations shared by the planner, the C-ABI layer and the kernels.
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "gsz.h"

namespace gsz {

// Elements per pack tile: one block of 64 lanes (one wave) moves one tile,
// 16 bytes a lane.
constexpr int64_t kPackTile = 512;
// Tensor pointers per pack launch (they travel in the kernel argument block).
constexpr int kPackBatch = 256;
// Blocks of the reductions: one per kRedElems elements, at most kMaxRedGrid
// (a launch's grid * 256 work-items stays below 2^32); their partials are summed
// in kFinalBlocks fixed ranges when there are more than kFinalBlocks of them.
constexpr int64_t kRedElems = 2048;
constexpr int64_t kMaxRedGrid = (int64_t)1 << 23;
constexpr int64_t kFinalBlocks = 1024;
inline int64_t red_blocks(int64_t n) {
    int64_t b = (n + kRedElems - 1) / kRedElems;
    if (b > kMaxRedGrid) b = kMaxRedGrid;
    return b < 1 ? 1 : b;
}

struct Bucket {
    int32_t first_tensor;  // forward index of the first tensor in bucket order
    int32_t n_tensors;
    int64_t base, n, padded, chunk, shard_off;
};

// Position -> interval lookup tables, in place of a binary search over every
// interval in the kernels.  The intervals (the pack's tensors by first tile, the
// shard's buckets by shard offset) have non-decreasing starts; positions
// [0, total) are cut into at most 2^kLutCellsLog2 cells of 2^shift positions,
// and cell j holds {lo, hi}: the intervals that contain its first and its last
// position.  A kernel reads the cell of its position; lo == hi is the answer,
// otherwise a search over [lo, hi] (the few intervals that start inside the cell).
constexpr int kLutCellsLog2 = 16;
struct Lut {
    int shift = 0;
    std::vector<int32_t> cells;      // 2 per cell: lo, hi
};
// starts(k) = tab[k * stride + offset] for k in [0, n); starts(0) == 0.
Lut build_lut(const std::vector<int64_t>& tab, int stride, int offset, int64_t n, int64_t total);

void set_error(const char* fmt, ...);

}  // namespace gsz

struct gsz_plan {
    std::vector<int64_t> numel;          // forward order
    int32_t P = 1, align = 64;
    int64_t cap = 0;
    std::vector<gsz::Bucket> buckets;
    std::vector<int64_t> tensor_off;     // forward index -> flat offset
    std::vector<int32_t> tensor_bucket;  // forward index -> bucket
    int64_t flat_len = 0, shard_len = 0, n_params = 0, total_pad = 0;
    uint64_t hash = 0;

    // Host copies of the device tables.
    // seg: (B+1) rows of {shard_off, base, chunk}; the last row is {S, 0, 0}.
    std::vector<int64_t> seg;
    // pack: per bucket-order position k (tensor T-1-k): {dst offset, numel, tile_begin};
    // then one sentinel row {0, 0, total tiles}.
    std::vector<int64_t> pack;
    // pads: per padded bucket {start, length}.
    std::vector<int64_t> pads;
    // Lookup tables: shard index -> bucket (over seg), tile -> bucket-order tensor
    // position (over pack).
    gsz::Lut seg_lut, pack_lut;

    // The device tables as one image of 8-byte slots, built with the plan:
    // seg, pack and pads rows (int64), then the two lookup tables (a {lo, hi}
    // pair of int32 per cell, one slot each), then 2 spare slots.  The caller
    // copies it into device memory it owns (gsz_plan_upload); the plan keeps the
    // image for as long as it lives, so that copy may complete asynchronously.
    std::vector<int64_t> image;

    // Where the image was last uploaded: the device and the caller's buffer.
    std::mutex mu;
    int device = -1;
    const int64_t* d_seg = nullptr;
    const int64_t* d_pack = nullptr;
    const int64_t* d_pads = nullptr;
    const uint64_t* d_seg_lut = nullptr;     // {lo, hi} int32 pairs, one per cell
    const uint64_t* d_pack_lut = nullptr;
};
