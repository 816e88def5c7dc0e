"""CPU float64 oracle for DualKV shared-prompt attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package. The product path (the
HIP library and its Python binding) never imports it, and this package never
imports the product path: the two share no code. Inputs are plain numpy arrays.

Two independent formulations of the same definition live here:

* ``replicated`` -- the literal one. The shared prompt is copied into N ordinary
  causal sequences [prompt; response_n], each is run through textbook softmax
  attention and its textbook backward, and the results are gathered back into
  the packed layout, summing the N copies' prompt gradients. This is what the
  DualKV pages (the arXiv abstract; the research-map summary, section
  Approach) say the fused kernels are
  exactly equivalent to.
* ``sampled`` -- the packed definition written out per query row and per key:
  row t attends A(t) = {0..t} for a prompt row and {0..P-1} u {o_n..t} for a row
  of response n. It evaluates selected rows/keys at full workload sizes, where
  the literal replication is too slow to run whole.

``groups`` extends both to several shared-prompt groups packed back to back
(independent groups; each row attends only its own group). ``layer`` is a
float64 decoder layer run on the replicated sequences (for the packed-layer
check); ``tree`` runs every root-to-leaf path of a multi-level prefix forest
as its own causal sequence.

Every function in these modules has a pin in tests/test_oracle.py against
something other than itself (library attention + autograd, closed forms,
finite differences, invariants).
"""
from .replicated import oracle_fwd_bwd, causal_attention_fwd, causal_attention_bwd  # noqa: F401
from .sampled import attended_keys, rows_fwd_bwd, keys_dkdv  # noqa: F401
from .groups import attended_keys_groups, group_starts, oracle_groups_fwd_bwd  # noqa: F401
from .layer import layer64, replicated_layer, rms_norm64, rope64  # noqa: F401
from .tree import attended_keys_tree, leaf_paths, oracle_tree_fwd_bwd, segment_starts  # noqa: F401
