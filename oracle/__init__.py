"""CPU fp64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this package.  The HIP library never imports it, and this package
imports nothing from the library: the two share no code.

What it computes is standard attention written out as its definition
(bornlex.github.io "Flash Attention", section "Standard Attention": S = QK^T,
P = row softmax of S, O = PV; FlashAttention reading guide, xyznot.com,
"Masalah dan Motivasi"), with a caller-given scale and the masks described in
``attention.allowed``.  FlashAttention returns exactly this result (datacamp
"Penjelasan Flash Attention", section "Apa Itu Flash Attention?"), so the
definition is the oracle.  Everything is float64; inputs are the same
(already dtype-rounded) values the GPU receives and nothing is rounded here.

Modules:
  attention  dense definition, forward and backward (chain rule)
  sparse     the same result computed only over allowed 128x128 cells
             (exact because exp(-inf) = 0), for the large workloads
  online     the incremental softmax statistics and the tiled forward as the
             pages state them -- used by the pin tests to show exactness
  visits     the expected set of visited (query cell, key cell) pairs
  dropout    the definition with dropout on P (Philox4x32-10 random bytes),
             forward and backward
  fp8        the definition on the real values of OCP E4M3 inputs with
             per-tensor descale factors
"""
from . import attention, dropout, fp8, online, sparse, visits  # noqa: F401
