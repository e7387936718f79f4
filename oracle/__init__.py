"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the Mamba-2 SSD forward.

Only tests/, the smoke check and the bench's CPU-baseline leg may import
this package.  It shares no code with the HIP library, and the HIP library
never imports it.

Three independent formulations, all fp64:
  recurrence.ssd_recurrence  the per-token state recurrence, plain C
                             (ssd_recurrence.c), the oracle proper
  dual.ssd_dual              the quadratic masked-attention (dual) form,
                             numpy, tiny inputs only
  chunked.ssd_chunked        the chunked scan written out stage by stage,
                             numpy; also returns every intermediate

Parity pins (tests/test_oracle.py) tie each of them to things other than
itself: the dual form, closed forms, a library IIR filter, hand-derived
fixtures, invariants.  No function here is "parity unpinned".
"""
