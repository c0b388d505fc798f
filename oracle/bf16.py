"""bf16 codec on uint16 bit patterns.

Parameters and gradients are bf16, 2 bytes each ("Data Parallelism: DDP, ZeRO
and FSDP", section "The memory ledger"); the reduction runs in fp32
("Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
section "FSDP1 vs FSDP2 and DTensor": param_dtype=bf16, reduce_dtype=fp32).

bf16 is the upper half of an IEEE binary32, so widening is a 16-bit shift and
is exact.  Narrowing rounds to nearest, ties to even, on the 16 dropped bits;
NaN stays NaN (quiet bit set).
"""
import numpy as np


def widen(b: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float32, exact."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def narrow(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits (uint16), round to nearest even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    q = ((u >> 16) | 0x0040).astype(np.uint16)
    return np.where(is_nan, q, r).astype(np.uint16)
