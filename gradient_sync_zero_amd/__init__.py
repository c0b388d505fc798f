"""MI355X (gfx950) data-parallel shard step: bucket pack, ring-order reduce-mean,
clip-norm partial, fused AdamW with all-gather-layout output.

The work runs in libgsz.so (HIP kernels behind a C ABI, include/gsz.h); this
package is its ctypes binding and raises ImportError if the library is not
built.
"""
from ._binding import (AdamWHP, GszError, INTERLEAVE_PIECE, LAYOUT_BUCKET_FLAT,
                       LAYOUT_RANK_INTERLEAVED, LAYOUT_SHARD_COMPACT, LIB_PATH, interleaved_len,
                       MAX_RANKS, Plan, adamw_step, allgather_layout_write, allreduce_mean,
                       bucket_accumulate, bucket_accumulate_f32, bucket_pack, bucket_pack_f32,
                       bucket_unpack, clip_coef, load, ledger_bytes_per_param, make_hp, max_tile_span,
                       shard_adamw_step, shard_grad_sqnorm, shard_reduce_mean, shard_reduce_mean_noalloc,
                       set_burst_window, set_flat_wide, set_grid_limit, set_reduce_path, REDUCE_PATH_BURST, REDUCE_PATH_BY_SIZE,
                       REDUCE_PATH_TILE, shard_reduce_mean_f32, test_hooks, workspace_bytes)
from . import _binding

load()

__all__ = ["AdamWHP", "GszError", "INTERLEAVE_PIECE", "LAYOUT_BUCKET_FLAT",
           "LAYOUT_RANK_INTERLEAVED", "LAYOUT_SHARD_COMPACT", "LIB_PATH", "interleaved_len",
           "MAX_RANKS", "Plan", "adamw_step", "allgather_layout_write", "allreduce_mean",
           "bucket_accumulate", "bucket_accumulate_f32", "bucket_pack", "bucket_pack_f32",
           "bucket_unpack", "clip_coef", "ledger_bytes_per_param", "make_hp", "max_tile_span",
           "set_grid_limit",
           "set_burst_window", "set_flat_wide", "set_reduce_path", "REDUCE_PATH_BURST", "REDUCE_PATH_BY_SIZE", "REDUCE_PATH_TILE",
           "shard_adamw_step", "shard_grad_sqnorm", "shard_reduce_mean", "shard_reduce_mean_f32",
           "shard_reduce_mean_noalloc",
           "test_hooks", "workspace_bytes"]
