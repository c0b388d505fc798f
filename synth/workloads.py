"""Synthetic workloads for the data-parallel shard step.

This module only *describes* inputs: the per-parameter tensor sizes of each
model shape (in forward / compute order), the number of simulated ranks P, the
bucket cap, the AdamW and clipping hyperparameters, the value distributions and
the seeds.  It holds none of the method's arithmetic (no bucketing, no
reduction, no optimizer step); both the CPU oracle and the HIP path consume
what it describes.

Sources of the workload shapes:
  * "Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
    section "Inside DDP: Bucketed All-Reduce, Gradient Synchronization and
    Overlap": AdamW(lr=2e-4, weight_decay=0.1), clip_grad_norm_(..., 1.0),
    default 25 MB buckets.
  * "Data Parallelism: DDP, ZeRO and FSDP", section "The memory ledger":
    bf16 parameters and gradients, fp32 master / first / second moment.
  * The model shapes are public architectures (GPT-2 small, a GPT-style 1.3B,
    Llama-7B, Llama-70B with grouped-query attention); values are synthetic.

Readings taken where the sources are silent (each is also listed in the
design notes):
  * Linear layers carry no bias and GPT models have no learned position table,
    so GPT-2 small has 123,570,432 parameters; the 1.3B model ties its output
    head to the embedding; the Llama models keep an untied output head.
  * "MB" for the bucket cap is MiB (2**20 bytes), the unit of PyTorch's
    bucket_cap_mb.
  * N(0, s) names a normal distribution with standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

MIB = 1 << 20
SEED = 2026

# Generator stream kinds (the "kind" field of the counter-based generator key).
KIND_GRAD = 1
KIND_MASTER = 2
KIND_EXP_AVG = 3
KIND_EXP_AVG_SQ = 4

# Value distributions (standard deviations).
GRAD_STD = 1e-3
MASTER_STD = 0.02
EXP_AVG_STD = 1e-4
EXP_AVG_SQ_STD = 1e-6  # v is |N(0, 1e-6)|


@dataclass(frozen=True)
class AdamWHP:
    lr: float = 2e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    step: int = 10          # exponent t used in the bias corrections of this update
    max_norm: float = 1.0   # clip threshold on the global L2 norm


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    tensors: Tuple[Tuple[str, Tuple[int, ...]], ...]   # forward (compute) order
    world_size: int                                   # P simulated ranks
    bucket_cap_bytes: int
    grad_std: float = GRAD_STD
    hp: AdamWHP = field(default_factory=AdamWHP)

    @property
    def numel(self) -> List[int]:
        out = []
        for _, shape in self.tensors:
            n = 1
            for d in shape:
                n *= d
            out.append(n)
        return out

    @property
    def n_params(self) -> int:
        return sum(self.numel)


# Sixteen tensor sizes between 64 and 131072 elements whose sum is 2**20:
# eight pairs (a, 131072 - a), the first a = 64 and the others drawn once,
# uniformly from [64, 131008], then shuffled.  Ten of them are odd or not a
# multiple of 8, so bucket offsets are unaligned and tail paths are exercised.
TINY_SIZES = (81520, 66812, 11457, 37473, 131008, 110103, 64260, 119615,
              93599, 24215, 49552, 106857, 120999, 64, 10073, 20969)


def _tiny() -> Workload:
    tensors = tuple((f"t{i}", (n,)) for i, n in enumerate(TINY_SIZES))
    return Workload(0, "tiny-1M-P4", tensors, 4, 1 * MIB)


def _gpt(cfg_id, name, vocab, hidden, mlp, blocks, P) -> Workload:
    t = [("wte", (vocab, hidden))]
    for b in range(blocks):
        t += [(f"h{b}.ln1.w", (hidden,)), (f"h{b}.ln1.b", (hidden,)),
              (f"h{b}.attn.qkv", (hidden, 3 * hidden)),
              (f"h{b}.attn.proj", (hidden, hidden)),
              (f"h{b}.ln2.w", (hidden,)), (f"h{b}.ln2.b", (hidden,)),
              (f"h{b}.mlp.fc", (hidden, mlp)),
              (f"h{b}.mlp.proj", (mlp, hidden))]
    t += [("lnf.w", (hidden,)), ("lnf.b", (hidden,))]
    return Workload(cfg_id, name, tuple(t), P, 25 * MIB)


def _llama(cfg_id, name, vocab, hidden, mlp, blocks, kv_dim, P) -> Workload:
    t = [("embed", (vocab, hidden))]
    for b in range(blocks):
        t += [(f"l{b}.attn_norm", (hidden,)),
              (f"l{b}.q", (hidden, hidden)), (f"l{b}.k", (kv_dim, hidden)),
              (f"l{b}.v", (kv_dim, hidden)), (f"l{b}.o", (hidden, hidden)),
              (f"l{b}.mlp_norm", (hidden,)),
              (f"l{b}.gate", (mlp, hidden)), (f"l{b}.up", (mlp, hidden)),
              (f"l{b}.down", (hidden, mlp))]
    t += [("norm", (hidden,)), ("lm_head", (vocab, hidden))]
    return Workload(cfg_id, name, tuple(t), P, 25 * MIB)


def tiny() -> Workload:
    return _tiny()


def tiny_clip() -> Workload:
    """Tiny with gradients of std 0.1, so the global norm is far above 1.0."""
    w = _tiny()
    return Workload(5, "tiny-1M-P4-clip", w.tensors, 4, 1 * MIB, grad_std=0.1)


def gpt2_small() -> Workload:
    return _gpt(1, "gpt2-small-124M-P8", 50257, 768, 3072, 12, 8)


def gpt_1p3b() -> Workload:
    return _gpt(2, "gpt-1.3B-P8", 50304, 2048, 8192, 24, 8)


def llama_7b() -> Workload:
    return _llama(3, "llama-7B-share-P8", 32000, 4096, 11008, 32, 4096, 8)


def llama_70b() -> Workload:
    return _llama(4, "llama-70B-share-P64", 32000, 8192, 28672, 80, 1024, 64)


WORKLOADS = {w.cfg_id: w for w in (tiny(), gpt2_small(), gpt_1p3b(), llama_7b(),
                                   llama_70b(), tiny_clip())}


def by_id(cfg_id: int) -> Workload:
    return WORKLOADS[cfg_id]


def lsq_problem():
    """Least-squares model for the gradient-mean invariant.

    4 features, 64 samples split into 4 equal shards of 16.  Integer data
    x in {-1,0,1}, theta in {-1,0,1}, y in {-2..2} drawn from a fixed seed, so
    every shard gradient is an integer over 16 and is exact in bf16.
    Returns (x[64,4] int, theta[4] int, y[64] int).
    """
    import numpy as np
    rng = np.random.default_rng([SEED, 99])
    x = rng.integers(-1, 2, size=(64, 4))
    theta = rng.integers(-1, 2, size=4)
    y = rng.integers(-2, 3, size=64)
    return x, theta, y
