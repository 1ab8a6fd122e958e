"""CPU oracle for long-context causal attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy statement of what the HIP library computes. Only the tests, the smoke check in
__graft_entry__ and the cpu_baseline leg of bench.py may import it; the library and its Python binding never do,
and the oracle shares no code with them (inputs come from the separate `workloads` generator module).

Contents
  attention.causal_attention   exact causal softmax attention with GQA head grouping (dense prefill)
  attention.masked_attention   the same, restricted to the key blocks a block mask keeps (block-sparse prefill)
  attention.paged_decode       q_len = 1 attention over a paged KV cache, unsplit
  attention.split_decode / lse_combine
                               the split-KV form and its log-sum-exp reduce (used for the split == unsplit pin)
  block_mask.*                 the selection pre-pass: centroids, radii, radius quantiles, the two branches and
                               their OR

Every function is pinned by tests under tests/test_oracle_*.py against brute force, closed forms, invariants and
library routines (see each function's docstring for the passage it follows). There is no "parity unpinned"
function in this package.
"""
from . import attention, block_mask  # noqa: F401
