"""Bucket plan: which gradient goes in which bucket, and which rank owns what.

Followed passages:
  * "Data parallelism in depth" §4.2 (The Bucket mechanism): the buckets are
    filled in the opposite of the order in which the forward pass computes the
    tensors, about 25 MB by default, and a bucket's collective starts once all
    of its gradients exist.
  * "Data Parallelism: DDP, ZeRO and FSDP", section "DDP, and why it works":
    the same ~25 MB buckets in the backward (last layer first) order, and the
    order must agree across ranks.
  * "Data Parallelism: From Parameter Server to Ring All-Reduce" §5: the buffer
    is cut into N equal chunks; when the reduce-scatter ends, each rank holds
    the complete sum of exactly one of them.
  * "Data Parallelism: DDP, ZeRO and FSDP", section "The three stages": under
    ZeRO-1/2 a rank updates only its own shard, after the reduce-scatter.

Readings where the pages are silent:
  * reverse order = the forward tensor list reversed (also inside a block);
  * a bucket holds whole tensors; a tensor is appended, then the bucket closes
    as soon as its byte size reaches the cap; the last bucket holds the rest;
  * a bucket of n elements is zero-padded to L = the next multiple of P*align,
    so its P chunks have equal length C = L/P (align = 64 elements);
  * rank r owns chunk r of every bucket; its shard is the concatenation of its
    chunks in bucket order.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List


@dataclass(frozen=True)
class Bucket:
    tensors: tuple        # tensor indices in bucket (reverse-forward) order
    base: int             # flat offset of the bucket
    n: int                # gradient elements (before padding)
    padded: int           # L: padded length, a multiple of P*align
    chunk: int            # C = L / P
    shard_off: int        # offset of this bucket's chunk inside every shard


@dataclass(frozen=True)
class Plan:
    numel: tuple
    world_size: int
    bucket_cap_bytes: int
    align: int
    buckets: tuple
    tensor_offset: tuple  # flat offset of each tensor (forward index)
    tensor_bucket: tuple  # bucket of each tensor (forward index)
    flat_len: int
    shard_len: int

    def chunk_range(self, b: int, r: int):
        """Flat [start, end) of rank r's chunk of bucket b."""
        bk = self.buckets[b]
        s = bk.base + r * bk.chunk
        return s, s + bk.chunk


def make_plan(numel: List[int], bucket_cap_bytes: int, world_size: int,
              align: int = 64, elem_bytes: int = 2) -> Plan:
    if world_size < 1 or align < 1 or bucket_cap_bytes < 1:
        raise ValueError("bad plan parameters")
    if any(n < 0 for n in numel):
        raise ValueError("negative tensor size")
    groups = []
    cur, cur_elems = [], 0
    for t in reversed(range(len(numel))):
        cur.append(t)
        cur_elems += numel[t]
        if cur_elems * elem_bytes >= bucket_cap_bytes:
            groups.append(cur)
            cur, cur_elems = [], 0
    if cur:
        groups.append(cur)

    gran = world_size * align
    buckets, offs, owner = [], [0] * len(numel), [0] * len(numel)
    base = shard_off = 0
    for b, g in enumerate(groups):
        pos = base
        for t in g:
            offs[t] = pos
            owner[t] = b
            pos += numel[t]
        n = pos - base
        padded = -(-n // gran) * gran
        chunk = padded // world_size
        buckets.append(Bucket(tuple(g), base, n, padded, chunk, shard_off))
        base += padded
        shard_off += chunk
    return Plan(tuple(numel), world_size, bucket_cap_bytes, align, tuple(buckets),
                tuple(offs), tuple(owner), base, shard_off)
