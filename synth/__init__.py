"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

`workloads` describes the model shapes and hyperparameters; `gen` wraps the
counter-based generator (host implementation in C, device implementation in
HIP) that produces bit-identical values on both sides.  Nothing here performs
any step of the shard-step method.
"""
from . import workloads  # noqa: F401
