"""fp64 CPU oracle for exact blockwise softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package; only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library and never imports it.

What it computes is the plain definition of the result every blockwise method
on the source pages reaches exactly: softmax(c * Q K^T) V with a natural-log row
log-sum-exp, the log-sum-exp weighted merge of partial results over disjoint
key sets, and the analytic gradients of sum(dO * O).  Every function is pinned
by CPU tests against closed forms, invariants, finite differences, brute-force
scalar loops and library routines (see ``tests/test_oracle_*.py``).

Sources (page title, section):

* "BurstAttention: An Efficient Distributed Attention Framework for Extremely
  Long Sequences", abstract and method section: each device computes attention
  on its local share and a global step aggregates the local results.
* "Effiziente verteilte Aufmerksamkeit für das Training von LLMs mit langem
  Kontext" (DistFlashAttn digest), Core Concepts and Abstract: the distributed
  attention is exact, and the backward needs no re-run of the forward and
  introduces no numerical difference.
* "Tree Attention: Topology-aware Decoding for Long-Context Attention on GPU
  clusters", Technical Explanation and the Tree Attention and Lean Attention
  abstracts under Related Papers: partial results over sequence chunks are
  reduced as a tree; the softmax reduction is associative.
"""

from .attention import (  # noqa: F401
    attention,
    attention_backward,
    attention_backward_head,
    attention_head,
    decode,
    merge,
    merge_tree,
    visible_mask,
)
