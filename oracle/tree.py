"""Multi-level shared prefixes (float64). TEST INFRASTRUCTURE ONLY.

The DualKV summary page lists as a limitation that a single shared prefix per
group is assumed and tree-structured prefixes are not handled
("Limitations"). Reading taken here for that extension: the packed rows form
a forest of segments in depth-first order; segment i has node_len[i] rows
(right after segment i - 1) and parent node_parent[i] (-1 for a root). Every
root-to-leaf path is one ordinary causal sequence (the concatenation of its
segments), and the packed layout stores each segment once. So the oracle runs
textbook causal attention on every path and folds the results back: outputs
of a segment's rows from any path through it, gradients summed over the paths,
and the packed upstream gradient of a segment's rows split equally over the
L(v) paths that contain it (L(v) = number of leaves in its subtree).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .replicated import causal_attention_bwd, causal_attention_fwd


def segment_starts(node_len: Sequence[int]) -> list[int]:
    s = [0]
    for x in node_len:
        s.append(s[-1] + int(x))
    return s


def leaf_paths(node_parent: Sequence[int]) -> list[list[int]]:
    """Root-to-leaf segment lists, one per leaf (a segment with no children)."""
    n = len(node_parent)
    has_child = [False] * n
    for p in node_parent:
        if p >= 0:
            has_child[p] = True
    paths = []
    for v in range(n):
        if not has_child[v]:
            path = [v]
            while node_parent[path[-1]] >= 0:
                path.append(node_parent[path[-1]])
            paths.append(path[::-1])
    return paths


def attended_keys_tree(t: int, node_len: Sequence[int], node_parent: Sequence[int]) -> np.ndarray:
    """Packed key indices row t attends: every key of its segment's proper
    ancestors, then its own segment's keys up to t."""
    s = segment_starts(node_len)
    if t < 0 or t >= s[-1]:
        raise IndexError(t)
    v = int(np.searchsorted(s, t, side="right") - 1)
    while node_len[v] == 0:   # searchsorted lands on the last of equal starts; empty segments hold no rows
        v -= 1
    anc = []
    a = node_parent[v]
    while a >= 0:
        anc.append(a)
        a = node_parent[a]
    parts = [np.arange(s[a], s[a + 1]) for a in anc[::-1]] + [np.arange(s[v], t + 1)]
    return np.concatenate(parts).astype(np.int64)


def oracle_tree_fwd_bwd(q, k, v, do, node_len: Sequence[int], node_parent: Sequence[int],
                        scale: float, block: int = 256) -> dict:
    """O [T,Hq,d], LSE [Hq,T], dQ [T,Hq,d], dK, dV [T,Hkv,d] (float64)."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    s = segment_starts(node_len)
    if s[-1] != T:
        raise ValueError("segment lengths do not add up to T")
    paths = leaf_paths(node_parent)
    n_paths = [0] * len(node_len)
    for path in paths:
        for seg in path:
            n_paths[seg] += 1
    O = np.full((T, Hq, d), np.nan)
    LSE = np.full((Hq, T), np.nan)
    dQ = np.zeros((T, Hq, d))
    dK = np.zeros((T, Hkv, d))
    dV = np.zeros((T, Hkv, d))
    for path in paths:
        idx = np.concatenate([np.arange(s[x], s[x + 1]) for x in path]).astype(np.int64)
        if idx.size == 0:
            continue
        share = np.concatenate([np.full(s[x + 1] - s[x], 1.0 / n_paths[x]) for x in path])
        for g in range(Hkv):
            kg = np.asarray(k[idx, g], dtype=np.float64)
            vg = np.asarray(v[idx, g], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                qh = np.asarray(q[idx, h], dtype=np.float64)
                On, lsen = causal_attention_fwd(qh, kg, vg, scale, block)
                O[idx, h] = On
                LSE[h, idx] = lsen
                don = np.asarray(do[idx, h], dtype=np.float64) * share[:, None]
                dqn, dkn, dvn = causal_attention_bwd(qh, kg, vg, don, scale, block)
                np.add.at(dQ[:, h], idx, dqn)
                np.add.at(dK[:, g], idx, dkn)
                np.add.at(dV[:, g], idx, dvn)
    return {"O": O, "LSE": LSE, "dQ": dQ, "dK": dK, "dV": dV}
