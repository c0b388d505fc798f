/*
 * gsz_test.h -- test hooks of libgsz, exported only by the test build
 * (libgsz_test.so: the same sources compiled with GSZ_TEST_HOOKS).  The
 * product library, libgsz.so, has none of this state.  No page defines these
 * calls: they exist so that tests can reach code paths that only very large
 * inputs reach otherwise.
 */
#ifndef GSZ_TEST_H
#define GSZ_TEST_H

#include <stdint.h>

#include "gsz.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Caps the number of blocks of every data-sized launch made after the call,
 * for the whole process and every thread; 0 restores the built-in caps (2^31
 * work-items per launch, reached only by inputs of more than about 17e9
 * elements).  Under a cap each block strides over several tiles: the path
 * that otherwise runs only on such inputs.  Results are bit-identical to
 * uncapped launches except the fp64 norm partials, whose summation grouping
 * follows the grid.  Launches already enqueued keep their grids; workspace
 * sizes do not change.  GSZ_ERR_INVALID_ARG if max_blocks < 0. */
int gsz_test_set_grid_limit(int64_t max_blocks);

/* Chooses the kernel of the bf16 reduce at P > 16 (gsz_shard_reduce_mean, its
 * bf16-wire and no-allocation forms) for every call made after this one, for
 * the whole process: 0 the product's rule (the burst kernel from 2^23 shard
 * elements without the bf16 wire, else the one-tile-per-block kernel), 1
 * always the burst kernel (the bf16 wire too), 2 always the
 * one-tile-per-block kernel.  g is
 * bit-identical either way; the norm partial's fp64 summation grouping
 * follows the kernel and its grid (the burst kernel's grid is one block per
 * compute unit, at most one per 32768 elements, and gsz_test_set_grid_limit
 * caps it as well).
 * GSZ_ERR_INVALID_ARG if path is not 0, 1 or 2. */
int gsz_test_set_reduce_path(int32_t path);

/* Sets how the burst kernel writes g, for every launch made after the call,
 * for the whole process.  period 0 restores the product's choice.  Else
 * period must be a power of two: with window 0 each chunk is written by its
 * block once reduced; with window > 0 each wave writes the g rows it holds
 * when (constant clock, 100 MHz) mod period < window, or when its ring of 16
 * rows is full (window >= period: every row as soon as it is reduced).  Only
 * when g is written changes: g and the norm partials are bit-identical for
 * every setting.  GSZ_ERR_INVALID_ARG if period is not 0 or a power of two. */
int gsz_test_set_burst_window(uint32_t period, uint32_t window);

/* Nonzero: every bucket-flat reduce made after the call (the shard reduce in
 * all its forms and the all-reduce) on P <= 16 bf16 or any fp32
 * contributions reads them through 64-bit addresses, and every
 * gsz_shard_adamw_step and gsz_allgather_layout_write writes its all-gather
 * output through them: the paths the product takes only for plans whose
 * shard tiles (2048 elements for the reduce and the writer, 256 for AdamW)
 * span 2^31 bytes or more of a flat buffer (buckets of over 2^29 elements);
 * 0 restores the product's choice.  For the whole process.  Results are
 * bit-identical either way. */
int gsz_test_set_flat_wide(int32_t on);

/* *out = the largest span (last position - first position + 1) that the
 * owner's shard elements [k * tile, (k + 1) * tile) take in the bucket-flat
 * layout, over every k with k * tile below the shard length (at most tile
 * when no such range crosses a bucket boundary); the quantity the library
 * checks against 32-bit buffer offsets.  Host only.  GSZ_ERR_INVALID_ARG for
 * a NULL plan or out or tile < 1, GSZ_ERR_BAD_RANK for an owner outside
 * [0, P). */
int gsz_test_max_tile_span(const gsz_plan* plan, int32_t owner, int64_t tile, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* GSZ_TEST_H */
