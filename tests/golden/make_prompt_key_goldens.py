"""Write the stored expected values for prompt-key dK/dV at full workload sizes.

    python tests/golden/make_prompt_key_goldens.py [workload ...]

A prompt key is attended by every later row of the packed batch, so its key
gradients need the softmax of every row: too slow to recompute inside a GPU
test. This script evaluates them once with the CPU float64 oracle only
(oracle.keys_dkdv, the packed definition of the DualKV mask) on the seeded
workload inputs, and stores them with the sha256 of those inputs, so a test can
prove it regenerated the very same inputs before comparing.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from exact_shared_prefix_amd.inputs import WORKLOADS, workload_inputs  # noqa: E402
from oracle import keys_dkdv  # noqa: E402

FULL_SIZE = ["qwen3_8b_p4k_r4k_n8", "rollout_p8k_r4k_n32", "longprompt_p32k_r2k_n16",
             "ragged_p64k_n16_r256_2048"]


def prompt_keys(P: int) -> list[int]:
    """First, last, tile-edge and interior prompt keys."""
    ks = {0, 1, 127, 128, P // 2 + 3, P - 129, P - 2, P - 1}
    return sorted(k for k in ks if 0 <= k < P)


def path_for(name: str) -> str:
    return os.path.join(HERE, f"prompt_keys_{name}.npz")


def make(name: str) -> str:
    t0 = time.time()
    inp = workload_inputs(name)
    q = inp.q.float().numpy()
    k = inp.k.float().numpy()
    v = inp.v.float().numpy()
    do = inp.do.float().numpy()
    keys = prompt_keys(inp.P)
    out = keys_dkdv(q, k, v, do, inp.P, inp.lengths, inp.scale, keys, kv_head=0, row_block=256)
    p = path_for(name)
    np.savez_compressed(p, digest=np.array(inp.digest()), keys=np.array(keys), kv_head=np.array(0),
                        dK=out["dK"], dV=out["dV"], lengths=np.array(inp.lengths),
                        P=np.array(inp.P))
    print(f"{name}: {len(keys)} keys, {time.time() - t0:.1f} s -> {p}", flush=True)
    return p


if __name__ == "__main__":
    names = sys.argv[1:] or FULL_SIZE
    for n in names:
        assert n in WORKLOADS, n
        make(n)
