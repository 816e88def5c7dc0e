"""MI355X (gfx950) shared-prompt attention: packed prompt + N responses.

The forward and backward passes are HIP kernels in libdualkv.so behind the C
ABI of include/dualkv.h; this package is the thin Python binding over it
(`fwd`, `bwd`, `DualKVAttention`; `fwd_groups`, `bwd_groups` for several
prompt groups per call; `fwd_tree`, `bwd_tree` for multi-level prefixes), plus seeded workload inputs and work/FLOP accounting
used by the tests and the benchmark.
"""
from .binding import (DualKVAttention, DualKVError, GroupPacking, Packing, TreePacking,  # noqa: F401
                      bwd, bwd_groups, bwd_tree, bwd_workspace_bytes, fwd, fwd_groups, fwd_tree,
                      fwd_workspace_bytes, load)
