"""CPU oracle for Gemma-4-style hybrid attention (test infrastructure only).

Plain, slow, float64 definitions of what the HIP library computes. Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import this package; the
library never calls it and shares no code with it.

Modules:
  bf16      -- bf16 round-to-nearest-even straight from float64, and widening.
  prologue  -- per-head RMSNorm followed by (partial) RoPE, one bf16 rounding.
  attention -- causal / sliding-window GQA softmax attention with dense masks,
               the decode row, and the full layer (prologue + attention).
  split     -- the same attention with a row's keys in fixed chunks whose partial
               results are merged in chunk order.
  backward  -- the attention's gradients (float64 autograd of a dense attention).

Every function is pinned by the CPU tests (closed forms, invariants, brute force,
library routines and the bf16 cases the pages print); none is "parity unpinned".
"""
from . import attention, bf16, prologue, split  # noqa: F401
