"""CPU oracle for the MFMA fragment-layout library — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct fp64 reference implementations of everything
the GPU path computes.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the product path
never calls it and shares no code with it (no kernels, headers, tables or
helpers).  It imports numpy only.

Modules
  formats    fp32 -> fp16 / bf16 round-to-nearest-even, hi/lo split.
  layouts    accumulator-fragment maps, the brute-force ownership enumerator,
             the mixed-radix numeral of the cuda-oxide m16n8k16 example.
  reference  fp64 matmul on quantised inputs, block-repeat, split-precision
             expansion, attention, the normwise error.

Every function cites the passage of the pages it follows.  Functions whose
result is not pinned by anything but the hardware say so in their docstring.
"""
from . import formats, layouts, reference  # noqa: F401
