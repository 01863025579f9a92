"""CPU oracle for block-quantized decode GEMV — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 implementation of what the GPU path
computes, written from the block definitions and checked against hand-worked
blocks, brute-force exact sums and invariants (tests/test_oracle_*.py).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product (the C-ABI library and its
Python binding) never imports, links or calls it, and shares no code with it.

Sources (page titles and sections):
* Kinetic docs, "What makes it fast": decode reads every weight once per
  token; several guessed tokens are checked in one pass over the weights;
  several requests can share one pass; a mixture of experts reads only the
  experts in use.
* Kipp README, "How fast" (footnote to the 4-bit row): affine4 gs32 carries a
  per-group scale and bias, Q4_0 is scale-only; and "What it is": every GPU
  kernel is gated against a scalar CPU oracle.
* The per-format byte definitions (Q8_0, Q4_0, affine4 gs32) stated with the
  workloads; each function below restates the one it follows.
* Kinetic docs, "What makes it fast" (the Shortlist paragraph): an exact
  argmax over an output layer that computes exact scores only for the rows
  a bound from a small copy cannot rule out (shortlist.py).
"""
from . import formats, ref, shortlist  # noqa: F401
