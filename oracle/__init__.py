"""CPU oracle for the JSSA decode path — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy restatement of what the method computes, written from
the pages (the paper summary page "Summary (Overview)" of arXiv 2610.19026 and
the official-implementation README page of jiwonsong-dev/JSSA).  Only the
tests, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product library never does, and the oracle imports nothing from the
product library.

Modules
  fp8        OCP FP8 E4M3FN codec (round to nearest even, saturating)
  calibrate  second moments, unit-trace normalisation, Eq. 3/4/5
  gqa        projected-key store, group-mean projected score, top-B, attention
  mla        the same steps for the MLA scoring representation

Every function is pinned by tests/test_oracle_*.py against closed forms,
special cases that reduce to textbook/library routines, or brute force; the
one result with no pin is the sparse-vs-dense accuracy gap, which is only
reported ("parity unpinned").
"""
from . import fp8, calibrate, gqa, mla  # noqa: F401
