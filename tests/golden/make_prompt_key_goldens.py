"""Write the stored expected values for prompt-key dK/dV at full workload sizes.

    python tests/golden/make_prompt_key_goldens.py [workload ...]

A prompt key is attended by every later row of the packed batch, so its key
gradients need the softmax of every row: too slow to recompute inside a GPU
test. This script evaluates them once with the CPU float64 oracle only
(oracle.keys_dkdv, the packed definition of the DualKV mask) on the seeded
workload inputs, for the first and the last KV head, and stores them with the
sha256 of those inputs, so a test can prove it regenerated the very same
inputs before comparing.
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

KEY_TILE = 256      # keys per backward key tile
WAVE_KEYS = 32      # keys per 32-key block inside a tile
ROW_CHUNK = 2048    # rows per backward row chunk: keys at chunk edges are chosen too


def prompt_keys(P: int, n_tiles: int = 16) -> list[int]:
    """At least 64 prompt keys: the first and last key of n_tiles 256-key tiles
    spread over the prompt, in each of them the keys on both sides of its
    first 32-key block edge and one interior key, the keys on both sides of
    the first four and the last two 2048-row chunk edges, and a few more."""
    tiles = (P + KEY_TILE - 1) // KEY_TILE
    pick = sorted(set(int(round(x)) for x in np.linspace(0, tiles - 1, min(n_tiles, tiles))))
    ks = set()
    for j, t in enumerate(pick):
        a, b = t * KEY_TILE, min(P, (t + 1) * KEY_TILE) - 1
        ks |= {a, b, a + WAVE_KEYS - 1, a + WAVE_KEYS, a + 5 * WAVE_KEYS + 17 + j}
    edges = list(range(ROW_CHUNK, P, ROW_CHUNK))
    for e in edges[:4] + edges[-2:]:
        ks |= {e - 1, e}
    ks |= {1, P // 2 + 3, P - 129, P - 2}
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
    heads = sorted({0, inp.Hkv - 1})
    dK = np.zeros((len(heads), len(keys), inp.d))
    dV = np.zeros((len(heads), len(keys), inp.d))
    for i, g in enumerate(heads):
        out = keys_dkdv(q, k, v, do, inp.P, inp.lengths, inp.scale, keys, kv_head=g, row_block=256)
        dK[i], dV[i] = out["dK"], out["dV"]
        print(f"{name}: kv head {g}: {len(keys)} keys, {time.time() - t0:.1f} s", flush=True)
    p = path_for(name)
    np.savez_compressed(p, digest=np.array(inp.digest()), keys=np.array(keys),
                        kv_heads=np.array(heads), dK=dK, dV=dV, lengths=np.array(inp.lengths),
                        P=np.array(inp.P))
    print(f"{name}: {len(keys)} keys x {len(heads)} kv heads, {time.time() - t0:.1f} s -> {p}", flush=True)
    return p


if __name__ == "__main__":
    names = sys.argv[1:] or FULL_SIZE
    for n in names:
        assert n in WORKLOADS, n
        make(n)
