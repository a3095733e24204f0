"""Float64 CPU oracle for exact tiled attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(the HIP library and its Python binding) never imports it and shares no code
with it; the two meet only on inputs made by ``workloads``.

What it computes (all in float64, on the exact values the device receives):

* ``dense``   -- the plain definition: masked softmax(c Q K^T) V, its
  logsumexp statistic, and the hand-derived vector-Jacobian product written
  in the rowsum(P o dP) form (the form the D_i = dY_i . Y_i identity
  replaces, HarshvardhanJ/FlashAttention README, backward section).  Also
  row- and column-sampled evaluations of the same definition for problems
  too large to materialise.
* ``tiled``   -- the forward and reverse procedures of "Exact tiled softmax
  attention with block-recomputed vector-Jacobian products" (alphabetamath
  page, forward procedure steps 1-4 and reverse procedure), with the
  summary/merge convention read as stated in each function.
* ``tilemap`` -- the empty / partial / full classification of (query tile,
  key tile) pairs from the allowed-key sets, which decides which tiles a
  blocked implementation may skip (ob1 page, part 3 on block causal
  masking; alphabetamath page, forward step 2 "skip this block").

Pinning: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, invariants, a library softmax, central finite
differences and block-size independence -- never against the HIP path.
"""

from . import dense, tiled, tilemap  # noqa: F401
