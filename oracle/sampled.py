"""Packed-definition oracle for selected rows and keys (float64). TEST INFRASTRUCTURE ONLY.

At full workload sizes the literal replication is too slow to run whole, so
this module evaluates the same definition directly on the packed layout for a
chosen set of query rows or keys. The definition (the DualKV research-map
summary, section Approach, and the arXiv abstract): a prompt row t attends the prompt keys 0..t; a row t of
response n (o_n <= t < o_{n+1}) attends every prompt key and the keys o_n..t of
its own response; nothing else. The loss is L = sum_{t,h} <dO_{t,h}, O_{t,h}>.

Readings (the same as the replicated oracle): diagonal included, GQA head
h -> h // G, scale inside the exponent, natural-log LSE.

Rows are independent, so work is spread over a thread pool by (head, row
block); partial key gradients are summed in a fixed order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Sequence

import numpy as np


def _offsets(P: int, lengths: Sequence[int]) -> np.ndarray:
    return np.concatenate([[P], P + np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def _segment_of(t: int, P: int, o: np.ndarray) -> int:
    """-1 for a prompt row, else the response index n with o_n <= t < o_{n+1}."""
    if t < P:
        return -1
    return int(np.searchsorted(o, t, side="right") - 1)


def attended_keys(t: int, P: int, lengths: Sequence[int]) -> np.ndarray:
    """A(t): the packed key indices row t attends, in increasing order."""
    o = _offsets(P, lengths)
    if t < 0 or t >= o[-1]:
        raise IndexError(t)
    n = _segment_of(t, P, o)
    if n < 0:
        return np.arange(0, t + 1)
    return np.concatenate([np.arange(0, P), np.arange(o[n], t + 1)])


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


def rows_fwd_bwd(q, k, v, do, P: int, lengths: Sequence[int], scale: float,
                 rows: Sequence[int]) -> dict:
    """O, LSE and dQ of the selected packed rows, every query head.

    Each row's softmax, output and query gradient depend on that row alone:
    S = scale * q_t K_A^T, Pm = softmax(S), O_t = Pm V_A, LSE_t = logsumexp(S),
    dPm = dO_t V_A^T, dS = Pm * (dPm - rowsum(Pm * dPm)), dQ_t = scale * dS K_A.
    Returns arrays O [n,Hq,d], LSE [Hq,n], dQ [n,Hq,d] for n = len(rows).
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = [int(t) for t in rows]
    O = np.zeros((len(rows), Hq, d))
    LSE = np.zeros((Hq, len(rows)))
    dQ = np.zeros((len(rows), Hq, d))

    def one(i: int) -> None:
        t = rows[i]
        A = attended_keys(t, P, lengths)
        for g in range(Hkv):
            KA = np.asarray(k[A, g], dtype=np.float64)
            VA = np.asarray(v[A, g], dtype=np.float64)
            hs = slice(g * G, (g + 1) * G)
            qt = np.asarray(q[t, hs], dtype=np.float64)     # [G, d]
            dot = np.asarray(do[t, hs], dtype=np.float64)   # [G, d]
            S = scale * (qt @ KA.T)                          # [G, |A|]
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            Pm = E / l
            O[i, hs] = Pm @ VA
            LSE[hs, i] = (m + np.log(l))[:, 0]
            dPm = dot @ VA.T
            dS = Pm * (dPm - (Pm * dPm).sum(axis=1, keepdims=True))
            dQ[i, hs] = scale * (dS @ KA)

    with ThreadPoolExecutor(_threads()) as pool:
        list(pool.map(one, range(len(rows))))
    return {"O": O, "LSE": LSE, "dQ": dQ}


def keys_dkdv(q, k, v, do, P: int, lengths: Sequence[int], scale: float,
              keys: Sequence[int], kv_head: int, row_block: int = 512) -> dict:
    """dK and dV of KV head kv_head at the selected packed keys.

    dV_j = sum over rows t with j in A(t) and query heads h of the group of
    Pm_tj dO_t;  dK_j = scale * sum of dS_tj q_t. Pm_tj and dS_tj need row t's
    whole softmax, so every row attending any selected key is evaluated in full
    (rows in blocks, all of a block in one segment so they share a key list).
    Returns dK, dV of shape [len(keys), d].
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    N = len(lengths)
    o = _offsets(P, lengths)
    keys = np.asarray([int(j) for j in keys], dtype=np.int64)
    if keys.size and (keys.min() < 0 or keys.max() >= T):
        raise IndexError("key out of range")
    kg = k[:, kv_head]
    vg = v[:, kv_head]

    # which rows attend any selected key, per segment
    prompt_keys = keys[keys < P]
    tasks = []  # (segment, row0, row1)
    if prompt_keys.size:
        lo = int(prompt_keys.min())
        tasks += [(-1, r, min(P, r + row_block)) for r in range(lo, P, row_block)]
    for n in range(N):
        a, b = int(o[n]), int(o[n + 1])
        if a == b:
            continue
        if prompt_keys.size:
            lo = a
        else:
            own = keys[(keys >= a) & (keys < b)]
            if not own.size:
                continue
            lo = int(own.min())
        tasks += [(n, r, min(b, r + row_block)) for r in range(lo, b, row_block)]
    work = [(h, t) for h in range(kv_head * G, (kv_head + 1) * G) for t in tasks]

    def one(item):
        h, (n, r0, r1) = item
        if n < 0:
            kidx = np.arange(0, r1)
        else:
            kidx = np.concatenate([np.arange(0, P), np.arange(o[n], r1)])
        KA = np.asarray(kg[kidx], dtype=np.float64)
        VA = np.asarray(vg[kidx], dtype=np.float64)
        Qb = np.asarray(q[r0:r1, h], dtype=np.float64)
        dOb = np.asarray(do[r0:r1, h], dtype=np.float64)
        S = scale * (Qb @ KA.T)
        t = np.arange(r0, r1)[:, None]
        allowed = kidx[None, :] <= t   # prompt keys < P <= t for response rows
        S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        Pm = E / E.sum(axis=1, keepdims=True)
        dPm = dOb @ VA.T
        dS = Pm * (dPm - (Pm * dPm).sum(axis=1, keepdims=True))
        # columns of the selected keys inside this block's key list
        pos = np.searchsorted(kidx, keys)
        hit = (pos < kidx.size) & (kidx[np.minimum(pos, kidx.size - 1)] == keys)
        dk = np.zeros((keys.size, d))
        dv = np.zeros((keys.size, d))
        if hit.any():
            cols = pos[hit]
            dv[hit] = Pm[:, cols].T @ dOb
            dk[hit] = scale * (dS[:, cols].T @ Qb)
        return dk, dv

    dK = np.zeros((keys.size, d))
    dV = np.zeros((keys.size, d))
    with ThreadPoolExecutor(_threads()) as pool:
        for dk, dv in pool.map(one, work):   # map keeps submission order
            dK += dk
            dV += dv
    return {"dK": dK, "dV": dV}
