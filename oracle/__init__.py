"""CPU oracle for SubSpec-style self-speculative decoding with a W4A16 draft.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path never
calls it and shares no code with it.

Plain, slow, obviously correct: NumPy in float64 for every floating-point
quantity that is not a decision, bfloat16 rounding emulated at the storage
points, Python loops where they make the steps easier to check.  Where
floating point decides an integer (a 4-bit code, a sampled token, an
accept/reject) the oracle takes that decision in float32 exactly as the
definition below states, so that it is taken in the same precision as on the
GPU; sums that feed a decision are exact (integers).

Sources (cited by page title and section):
  [SD]   "How speculative decoding makes LLMs go brrr" (digest), overall flow
         and pseudo-code, Module 2 (parallel verify), Module 3 (rejection
         sampling and losslessness), Module 4 (benefit model).
  [SSN]  "SubSpec: Speculate Deep and Accurate" (paper note), Method details:
         substitute layers, resident-layer sharing, KV-cache sharing.
  [SSR]  "SubSpec: the target's own low-bit shadow as the draft" (report),
         sections 2.1-2.2, 3.2-3.7 (Tables 1, 3, 5) and the back-solved
         denominators that follow section 7.1.
  [SSL]  "The second ledger of speculative decoding" (SparseSpec-L blog),
         sections 1, 2, 3.1-3.3.

Parity status of each part is listed in the module docstrings.  Every part
has pins; the sparse-KV draft (sparse.py) is pinned by properties, special
cases and brute force only, since the pages print no worked example of it.
"""
