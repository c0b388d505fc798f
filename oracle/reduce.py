"""Mean of P rank gradients for the chunks one rank owns, in ring order.

Followed passages:
  * "Data parallelism in depth" §2 (Mathematical foundation): the synchronised
    gradient is the average (1/N) sum_k g_k of the per-rank gradients, not
    their sum (a sum would scale the learning rate by N).
  * "Data Parallelism: From Parameter Server to Ring All-Reduce" §1 (The
    Contract): every rank ends with the same G, the sum of the N rank
    gradients divided by N; §5 (Ring All-Reduce = Reduce-Scatter +
    All-Gather): the buffer is cut into N chunks; chunk c's fp32 partial sum
    starts at one rank, moves one neighbour per step and takes one addition at
    each hop, so after N-1 steps it is complete at the rank that owns c; the
    all-gather phase then circulates the finished chunks for N-1 more steps.
    Each rank sends (N-1)/N of the buffer per phase, 2(N-1)/N of it in all.
  * "Data parallelism in depth" §5.1-§5.2: AllReduce = ReduceScatter +
    AllGather, per-GPU volume 2*Psi*(N-1)/N.
  * "Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
    section "FSDP1 vs FSDP2 and DTensor": reduce_dtype = fp32.

Readings: the partial sums are fp32, each addition rounded to nearest even; chunk
c enters the ring at rank c+1 and its last addition is the owner's own
contribution, so the owner's sum is ((g_{c+1} + g_{c+2}) + ...) + g_c; the 1/P
is one true division after the sum.
"""
from __future__ import annotations

import numpy as np

from .bf16 import narrow, widen


def as_f32(c) -> np.ndarray:
    """A contribution as fp32: bf16 bits (uint16) are widened exactly; fp32
    contributions (fp32 accumulation buckets) are taken as they are."""
    c = np.asarray(c)
    if c.dtype == np.uint16:
        return widen(c)
    if c.dtype != np.float32:
        raise ValueError(f"contribution dtype {c.dtype}: need bf16 bits (uint16) or float32")
    return c


def reduce_mean(contribs, r: int) -> np.ndarray:
    """contribs[q]: rank q's values for owner r's elements, bf16 bits (uint16)
    or fp32.

    Returns the fp32 mean in ring order ((c[r+1] + c[r+2]) + ...) + c[r], / P.
    """
    P = len(contribs)
    if not 0 <= r < P:
        raise ValueError("owner rank out of range")
    acc = as_f32(contribs[(r + 1) % P]).copy()
    for k in range(2, P + 1):
        acc = acc + as_f32(contribs[(r + k) % P])
    return (acc / np.float32(P)).astype(np.float32)


def ring_allreduce_sim(plan, flats, rs_wire_bytes: int = 4, ag_wire_bytes: int = 4,
                      bf16_partials: bool = False):
    """Message-passing simulation of ring reduce-scatter then all-gather.

    flats[k]: rank k's bucket-major flat buffer (bf16 bits or fp32).  Returns
    (results, rs_sent, ag_sent): results[k] is rank k's fp32 flat buffer after
    the all-reduce (mean); rs_sent[k] / ag_sent[k] count the bytes rank k sent
    in each phase (elements times the wire dtype's size).  With bf16_partials
    every partial sum is rounded to bf16 before it is sent on (and the owner's
    final sum too), as a ring with a bf16 wire does.
    """
    P = plan.world_size
    if len(flats) != P:
        raise ValueError("need one flat buffer per rank")
    results = [np.zeros(plan.flat_len, dtype=np.float32) for _ in range(P)]
    rs_sent = [0] * P
    ag_sent = [0] * P
    for bk in plan.buckets:
        C = bk.chunk
        # buf[k][c]: rank k's current fp32 values of chunk c of this bucket.
        buf = [[as_f32(flats[k][bk.base + c * C: bk.base + (c + 1) * C]).copy()
                for c in range(P)] for k in range(P)]
        for s in range(P - 1):                       # reduce-scatter
            msgs = []
            for k in range(P):
                c = (k - 1 - s) % P
                msgs.append((k, c, buf[k][c].copy()))
                rs_sent[k] += C * rs_wire_bytes
            for k, c, m in msgs:
                dst = (k + 1) % P
                buf[dst][c] = m + buf[dst][c]
                if bf16_partials:
                    buf[dst][c] = widen(narrow(buf[dst][c]))
        for c in range(P):                           # owner c divides its sum
            buf[c][c] = (buf[c][c] / np.float32(P)).astype(np.float32)
        for s in range(P - 1):                       # all-gather
            msgs = []
            for k in range(P):
                c = (k - s) % P
                msgs.append((k, c, buf[k][c].copy()))
                ag_sent[k] += C * ag_wire_bytes
            for k, c, m in msgs:
                buf[(k + 1) % P][c] = m
        for k in range(P):
            for c in range(P):
                results[k][bk.base + c * C: bk.base + (c + 1) * C] = buf[k][c]
    return results, rs_sent, ag_sent


def central_gather_sim(plan, flats, wire_bytes: int = 4):
    """Contrast from "Data parallelism in depth" §5.3: every rank sends its
    gradients to a primary (rank 0), which sums them and sends the result back.
    Returns (result, primary_bytes) where primary_bytes = sent + received by
    rank 0."""
    P = plan.world_size
    acc = widen(flats[0]).copy()
    recv = 0
    for k in range(1, P):
        acc = acc + widen(flats[k])
        recv += plan.flat_len * wire_bytes
    result = (acc / np.float32(P)).astype(np.float32)
    sent = (P - 1) * plan.flat_len * wire_bytes
    return result, sent + recv


def reduce_mean_bf16_wire(contribs, r: int) -> np.ndarray:
    """The same ring, with bf16 partial sums on the wire.

    "Data Parallelism: From Parameter Server to Ring All-Reduce" §8: the
    gradient dtype of the communication changes both bandwidth and numerical
    behaviour.  Reading: each hop adds the received bf16 partial sum to the
    rank's own bf16 value in fp32 and rounds the result to bf16 (round to
    nearest even) before sending it on; the owner's final sum is widened and
    divided by P in fp32.  Returns fp32.
    """
    P = len(contribs)
    if not 0 <= r < P:
        raise ValueError("owner rank out of range")
    acc = np.asarray(contribs[(r + 1) % P], dtype=np.uint16).copy()
    for k in range(2, P + 1):
        acc = narrow(widen(acc) + widen(contribs[(r + k) % P]))
    return (widen(acc) / np.float32(P)).astype(np.float32)
