"""CPU oracle for the verify / select / sparse-draft attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
run this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
kernels or their binding; it imports nothing but NumPy (and the standard
library in ``brute``).

Modules
-------
``attention``  dense verify attention with Collect-2-Query logits, and sparse
               attention over token lists, per-KV-head lists or block lists.
``select``     the selector: head-summed two-row scores, sink / recent windows
               and top-k, in fp64 and in the pinned fp32 order that the GPU
               must reproduce bit for bit.
``nsa``        the NSA branches of sparse speculative verification: block-mean
               compression of the cache, and the gated sum of the compression,
               selection and sliding-window branches (exact or approximate
               grouping of the verifier rows' block sets).
``speedup``    the speculative speedup identity and its derivative.
``brute``      pure-Python loops for tiny inputs, used to pin ``attention``.

Every function names the passage of the pages it follows.  "Vegas page" is the
Pith review of *Vegas: Self-Speculative Decoding with Verification-Guided
Sparse Attention*; "Sparse Glimpse page" the review of *A Sparse Glimpse of the
Whole: Train-Free Self-Speculative Decoding*; "SSV page" the review of *SSV:
Sparse Speculative Verification for Efficient LLM Inference*.

Pinning status: every public function is pinned by a non-GPU test against
something other than itself (brute force, a library routine, closed forms,
invariants or pairwise enumeration); see ``tests/test_oracle_*.py``.  That
includes ``attention.attention_one`` (brute force, a verify row, closed form),
``attention.sparse_attn`` with a different list per KV head (brute force) and
``select.select`` in block mode (rank enumeration over each group's block
maxima, or block log-sum-exps) and every function of ``nsa`` (brute force per
branch, linearity in the gates, hand-worked bf16 rounding).
"""
