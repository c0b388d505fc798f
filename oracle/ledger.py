"""Model-state bytes per parameter per rank.

"Data Parallelism: DDP, ZeRO and FSDP", sections "The memory ledger" and "The
three stages": bf16 parameters 2, bf16 gradients 2, fp32 master 4, Adam first
moment 4, second moment 4 (16 in total, 12 of them optimizer state); ZeRO-1
shards the optimizer state (4 + 12/P), ZeRO-2 also the gradients (2 + 14/P),
ZeRO-3 everything (16/P).  "Data parallelism in depth" §6.1 and §7 give the
same table.
"""
from __future__ import annotations

PARAM = 2
GRAD = 2
MASTER = 4
EXP_AVG = 4
EXP_AVG_SQ = 4


def bytes_per_param(P: int, zero_stage: int) -> float:
    """zero_stage 0 = DDP (nothing sharded), 1, 2, 3."""
    opt = MASTER + EXP_AVG + EXP_AVG_SQ
    if zero_stage == 0:
        return float(PARAM + GRAD + opt)
    if zero_stage == 1:
        return PARAM + GRAD + opt / P
    if zero_stage == 2:
        return PARAM + (GRAD + opt) / P
    if zero_stage == 3:
        return (PARAM + GRAD + opt) / P
    raise ValueError("zero_stage must be 0..3")


def model_state_bytes(psi: int, P: int, zero_stage: int) -> float:
    return psi * bytes_per_param(P, zero_stage)


def optimizer_share() -> float:
    return (MASTER + EXP_AVG + EXP_AVG_SQ) / (PARAM + GRAD + MASTER + EXP_AVG + EXP_AVG_SQ)
