"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package.  Only the test suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark may use it.  It shares no code
with the HIP library: it is a plain, slow, token-by-token NumPy restatement of
what the method computes, in float64.

Modules
-------
kda      token-by-token recurrence: prefill (fixed / varlen), decode, verify
         (causal conv + chain / tree), commit.
chunked  the chunked (WY / UT) form of the same recurrence, in float64, used
         only to pin the chunk algebra against the recurrence.

Every function is pinned by a CPU test against something other than itself
(closed forms, invariants, brute force, textbook routines); none is marked
"parity unpinned".
"""

from . import kda, chunked  # noqa: F401
