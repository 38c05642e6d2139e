"""CPU oracle for exact softmax attention (fp64, numpy). TEST INFRASTRUCTURE ONLY.

This package is the independent definition that the HIP library is checked
against. Only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it. The library under
``memory_efficient_exact_amd`` never imports, links or calls anything here, and
nothing here imports that library: the two share no code.

Sources (web pages; cited by title and section throughout):

* "Self-attention Does Not Need O(n^2) Memory" (arXiv 2112.05682), as given by
  two digests: a Chinese one (sections 方法论, 方法详解, and the original
  English abstract, 原文摘要) and an English one (the method bullet list).
* "Fast and memory-efficient exact attention 分析", section 数学表达形式
  (the attention formula softmax(QK^T / sqrt(d_k)) V).
* "当注意力成为瓶颈：从O(n²)困境到线性复杂度的技术突围", sections
  平方级的诅咒 (S = QK^T, P = softmax(S) row-wise, O = PV) and IO感知 (the
  two-block merge equations for m, l and O).

Every function works in float64 on whatever values it is given; callers pass
the exact bf16/fp32 input values upcast to float64.

Parity status of each function (what pins it, see tests/test_oracle.py):

* ``naive_fwd``   - pinned: brute-force pure-Python loops, closed forms,
  torch fp64 SDPA, invariants (n=1, equal keys, permutation, shift, V=1,
  argmax limit).
* ``chunked_fwd`` - pinned: agrees with ``naive_fwd`` and with the brute force;
  same invariants.
* ``single_query`` - pinned: brute force and closed forms.
* ``naive_bwd``   - pinned: central finite differences of ``naive_fwd``,
  torch fp64 autograd, exact sum identities, special cases.
* ``row_stats``   - pinned: brute force (max and sum definitions).
* ``gqa_fwd`` / ``kv_head_of`` - pinned: per-group constant values fix the
  head mapping in closed form; brute force per query head; torch fp64 SDPA on
  explicitly repeated key/value heads.
* ``gqa_bwd``     - pinned: central finite differences of ``gqa_fwd`` (the
  shared key/value heads included); torch fp64 autograd.
* ``block_summary`` / ``merge_summaries`` / ``split_fwd`` - pinned: brute
  force, ``naive_fwd`` for every split count, order independence of the
  merge, one-key blocks against the plain definition, 1e4-scale scores.
"""

from .attention import (  # noqa: F401
    naive_fwd,
    chunked_fwd,
    single_query,
    naive_bwd,
    row_stats,
    softmax_scale,
    kv_head_of,
    gqa_fwd,
    gqa_bwd,
    block_summary,
    merge_summaries,
    split_ranges,
    split_fwd,
)

__all__ = ["naive_fwd", "chunked_fwd", "single_query", "naive_bwd", "row_stats", "softmax_scale",
           "kv_head_of", "gqa_fwd", "gqa_bwd", "block_summary", "merge_summaries", "split_ranges",
           "split_fwd"]
