"""CPU oracle for one rank's share of a Ulysses sequence-parallel attention layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package:
only the tests, the smoke check and the bench's CPU baseline leg use it. It shares
no code with the HIP library (no kernels, headers, helpers or tables).

Parts:
  permute   -- the local halves of the two all-to-alls, as explicit index loops
  attention -- plain masked softmax attention forward and backward in float64
  brute     -- scalar-loop attention and finite differences for tiny inputs
  chunked   -- the headwise-chunked (UPipe) forward as a loop over head chunks
  ring      -- Ring Attention over P ranks: per-hop partial attention and an LSE merge

Every function is pinned by tests under tests/ (test_oracle_*.py) against
brute force, closed forms, invariants and library routines.
"""
from . import permute, attention, brute, chunked, ring  # noqa: F401
