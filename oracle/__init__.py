"""CPU oracle for the OSCAR hot path — test infrastructure, not product code.

A plain, slow float64 NumPy restatement of what the method computes, written
from the OSCAR pages' descriptions:

  [TS] "Technical Summary: OSCAR - Offline Spectral Covariance-Aware Rotation
       for 2-bit KV Cache Quantization" (gist.science), sections 2.1, 2.2.A,
       2.2.B and 4;
  [AB] the arXiv abstract on the mlsanity.com page of the same paper.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(the page layout is re-implemented here from the prose definition in
``include/oscar.h``, not from its code); the only module both sides use is the
seeded input generator ``int2_rotated_kv_oscar_amd.synth``.

Modules: ``rotation`` (calibration targets, eigenbases, Hadamard, bit reversal,
composite rotation, clip threshold), ``quant`` (rotate, clip, asymmetric INT2
per token and group, and the 16-level INT4 variant), ``layout`` (INT2, INT4
and BF16 page images), ``cache`` (filling pages, the decode-step update),
``attention`` (decode attention over the mixed cache, chunked-prefill
"extend" attention over it, the split/merge formula, plain attention).  Every function is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force or an independent library routine.
"""
