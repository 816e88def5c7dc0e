"""Several shared-prompt groups packed back to back (float64). TEST INFRASTRUCTURE ONLY.

A training micro-batch can hold more than one prompt group (the DualKV summary
page quotes its GRPO results at a micro-batch size of 8, "Key results", and
assumes one shared prefix per micro-batch group, "Limitations"). Reading taken
here: the groups are independent packed micro-batches stored one after the
other in the same [T, H, d] tensors; a row attends only keys of its own group,
by the single-group rule. So the oracle is the single-group replicated oracle
run on each group's rows, and the per-row definition is the single-group A(t)
shifted to the group's first row.

groups: sequence of (P_b, [R_b0, R_b1, ...]).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .replicated import oracle_fwd_bwd
from .sampled import attended_keys


def group_starts(groups: Sequence) -> list[int]:
    """First packed row of each group, plus the total row count at the end."""
    s = [0]
    for P, L in groups:
        s.append(s[-1] + int(P) + sum(int(x) for x in L))
    return s


def attended_keys_groups(t: int, groups: Sequence) -> np.ndarray:
    """A(t) for packed row t of a multi-group batch, as absolute key indices."""
    s = group_starts(groups)
    if t < 0 or t >= s[-1]:
        raise IndexError(t)
    b = int(np.searchsorted(s, t, side="right") - 1)
    P, L = groups[b]
    return s[b] + attended_keys(t - s[b], int(P), [int(x) for x in L])


def oracle_groups_fwd_bwd(q, k, v, do, groups: Sequence, scale: float,
                          backward: bool = True) -> dict:
    """O [T,Hq,d], LSE [Hq,T], dQ [T,Hq,d], dK, dV [T,Hkv,d] (float64): the
    single-group oracle on each group's rows, placed at the group's rows."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    s = group_starts(groups)
    if s[-1] != T:
        raise ValueError("group sizes do not add up to T")
    out = {"O": np.full((T, Hq, d), np.nan), "LSE": np.full((Hq, T), np.nan),
           "dQ": np.full((T, Hq, d), np.nan), "dK": np.full((T, Hkv, d), np.nan),
           "dV": np.full((T, Hkv, d), np.nan)}
    for b, (P, L) in enumerate(groups):
        a, e = s[b], s[b + 1]
        if a == e:
            continue
        r = oracle_fwd_bwd(q[a:e], k[a:e], v[a:e], do[a:e], int(P), [int(x) for x in L], scale,
                           backward=backward)
        out["O"][a:e] = r["O"]
        out["LSE"][:, a:e] = r["LSE"]
        if backward:
            out["dQ"][a:e] = r["dQ"]
            out["dK"][a:e] = r["dK"]
            out["dV"][a:e] = r["dV"]
    return out
