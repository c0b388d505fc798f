"""Comparison helpers for the parity tests (bit-exact and ulp distances)."""
from __future__ import annotations

import numpy as np


def host(t):
    """Device tensor -> NumPy (bf16 kept as uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.uint16)
    if t.dtype == torch.uint16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def ordered(x: np.ndarray) -> np.ndarray:
    """fp32 bits mapped to integers whose order is the float order (+0 == -0)."""
    i = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(i & 0x7FFFFFFF), i)


def max_ulp(a, b) -> int:
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    if a.size == 0:
        return 0
    nan = np.isnan(a) | np.isnan(b)
    if (np.isnan(a) != np.isnan(b)).any():
        return 1 << 40
    return int(np.abs(ordered(a[~nan]) - ordered(b[~nan])).max(initial=0))


def max_bf16_ulp(a, b) -> int:
    a = np.asarray(a, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return int(np.abs(oa - ob).max(initial=0))


def assert_bits(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.dtype == np.float32:
        bad = gpu.view(np.uint32) != ref.astype(np.float32).view(np.uint32)
        both_nan = np.isnan(gpu) & np.isnan(ref)
        bad &= ~both_nan
    else:
        bad = gpu != ref
    n = int(bad.sum())
    if n:
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {n} of {bad.size} elements differ; first at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r}")


def bf16_wire_bound(contribs_fp64_abs_sum, P):
    """Rigorous bound on |fp32 ring mean - bf16-wire ring mean|, elementwise.

    Both are recursive sums of the same P values, compared with the exact
    mean E: |a - b| <= |a - E| + |E - b|.  A recursive sum whose every
    partial sum is rounded with relative error at most u is off by at most
    (P-1) * u * (1+u)^(P-1) * sum|c| (each of the P-1 rounded partial sums is
    at most (1+u)^(P-1) * sum|c| in magnitude).  The fp32 sum rounds once per
    addition: u = 2^-24.  The bf16 wire rounds each partial sum twice, the
    fp32 addition and then to bf16: |bf16(fl32(x)) - x| <= (2^-8 + 2^-24 +
    2^-32)|x|.  Division by P is exact for P a power of two (no underflow at
    these magnitudes).  The bound is evaluated in fp64; the caller allows a
    relative 1e-12 for that evaluation and nothing else."""
    import numpy as np
    u32 = 2.0 ** -24
    u16 = 2.0 ** -8 + 2.0 ** -24 + 2.0 ** -32
    k = P - 1
    coef = k * (u16 * (1 + u16) ** k + u32 * (1 + u32) ** k)
    return coef * np.asarray(contribs_fp64_abs_sum, dtype=np.float64) / P
