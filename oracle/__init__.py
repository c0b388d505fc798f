"""CPU oracle for one rank's share of a synchronous data-parallel step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy implementation used to check the HIP library.  Only the tests, the
smoke entry point and the benchmark's CPU-baseline leg may import it; the
library and its Python binding never do, and it shares no code with them.

It follows four web pages on data-parallel gradient synchronisation:
  [DPD]  "Data parallelism in depth" (infra-guide, chapter 4.1)
  [DTS]  "Distributed Training: Data Parallel, Model Parallel and FSDP Strategies"
  [DZF]  "Data Parallelism: DDP, ZeRO and FSDP"
  [PSR]  "Data Parallelism: From Parameter Server to Ring All-Reduce"
Every function cites the page title and section it follows.

Modules and the step they cover:
  bf16     bf16 <-> fp32 bit codec
  plan     bucket plan: reverse order, ~25 MiB buckets, padding, chunk ownership
  pack     per-tensor gradients -> bucket-major flat buffer, and back
  reduce   fixed ring-order fp32 mean of P contributions; message-passing ring
  norm     squared-norm partials, rank-order total, clip coefficient
  adamw    fp32 AdamW update, fixed operation order
  layout   owned chunks -> all-gather layout
  ledger   bytes per parameter for DDP and the ZeRO stages
  lsq      least-squares model for the gradient-mean equivalence
  step     composed shard step and the unsharded (DDP) reference

Every function here is pinned by a test against something other than itself
(values printed on the pages, closed forms, invariants, library routines,
brute force on tiny inputs).  Parity unpinned: none.
"""
