"""Literal replicated-prompt oracle (float64, numpy). TEST INFRASTRUCTURE ONLY.

Follows the DualKV pages: the method is exactly standard attention on N
separate sequences [prompt; response_n] (the arXiv abstract of "DualKV":
no approximation against standard attention, N(P+R) tokens packed into P+NR;
the research-map summary of the same paper, section Approach: two disjoint KV
regions, shared-prompt gradients accumulated across the N sequences). The oracle therefore does the replicated computation
literally and only then folds it back to the packed layout.

Readings taken where the pages are silent:
* causal masks include the diagonal; a response's local position r sits at
  position P + r of its replicated sequence;
* query head h uses KV head h // G with G = Hq / Hkv (contiguous GQA groups);
* the scale multiplies q.k inside the exponent; LSE is the natural-log
  log-sum-exp of the scaled scores;
* the packed upstream gradient of a prompt row is split equally over the N
  copies (dO_prompt / N each), so that the copies' gradients sum to the packed
  gradient of L = sum_t <dO_t, O_t>.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np


def _offsets(P: int, lengths: Sequence[int]) -> list[int]:
    o = [P]
    for r in lengths:
        o.append(o[-1] + int(r))
    return o


def causal_attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                         block: int = 256):
    """Textbook causal softmax attention of one sequence, one head.

    q, k, v: [L, d] float64. Returns O [L, d] and LSE [L] (natural log of the
    row's sum of exp(scale * q.k) over keys j <= i). Rows are processed in
    blocks of complete rows, so each row's softmax is formed in one piece.
    """
    L, d = q.shape
    O = np.zeros((L, v.shape[1]))
    lse = np.zeros(L)
    for r0 in range(0, L, block):
        r1 = min(L, r0 + block)
        S = scale * (q[r0:r1] @ k[:r1].T)
        i = np.arange(r0, r1)[:, None]
        j = np.arange(r1)[None, :]
        S = np.where(j <= i, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        Pm = E / l
        O[r0:r1] = Pm @ v[:r1]
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return O, lse


def causal_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dO: np.ndarray,
                         scale: float, block: int = 256):
    """Textbook backward of causal_attention_fwd for L = sum <dO, O>.

    The softmax is recomputed per block from scratch; its Jacobian is applied
    in the form dS = Pm * (dPm - rowsum(Pm * dPm)).
    Returns dq [L, d], dk [L, d], dv [L, d].
    """
    L, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, L, block):
        r1 = min(L, r0 + block)
        S = scale * (q[r0:r1] @ k[:r1].T)
        i = np.arange(r0, r1)[:, None]
        j = np.arange(r1)[None, :]
        S = np.where(j <= i, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        Pm = E / E.sum(axis=1, keepdims=True)
        g = dO[r0:r1]
        dv[:r1] += Pm.T @ g
        dPm = g @ v[:r1].T
        dS = Pm * (dPm - (Pm * dPm).sum(axis=1, keepdims=True))
        dq[r0:r1] = scale * (dS @ k[:r1])
        dk[:r1] += scale * (dS.T @ q[r0:r1])
    return dq, dk, dv


def oracle_fwd_bwd(q, k, v, do, P: int, lengths: Sequence[int], scale: float,
                   kv_heads: Optional[Iterable[int]] = None, backward: bool = True,
                   block: int = 256) -> dict:
    """Shared-prompt attention forward and backward by literal replication.

    q, do: [T, Hq, d]; k, v: [T, Hkv, d] (any float dtype, packed layout
    [prompt][resp_0]...[resp_{N-1}], T = P + sum(lengths)).
    kv_heads: restrict to these KV heads and their query heads (heads are
    independent); the other heads' entries are left NaN.

    Returns float64 arrays in the packed layout: O [T,Hq,d], LSE [Hq,T],
    dQ [T,Hq,d], dK, dV [T,Hkv,d], plus "prompt_replica_maxdiff", the largest
    difference between replicas' prompt-row O/LSE (zero by prompt invariance).
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    N = len(lengths)
    o = _offsets(P, lengths)
    if o[-1] != T:
        raise ValueError("P + sum(lengths) != T")
    kv_list = list(range(Hkv)) if kv_heads is None else sorted(set(int(x) for x in kv_heads))

    O = np.full((T, Hq, d), np.nan)
    LSE = np.full((Hq, T), np.nan)
    dQ = np.full((T, Hq, d), np.nan)
    dK = np.full((T, Hkv, d), np.nan)
    dV = np.full((T, Hkv, d), np.nan)
    maxdiff = 0.0

    for g in kv_list:
        dK[:, g] = 0.0
        dV[:, g] = 0.0
        kg = np.asarray(k[:, g], dtype=np.float64)
        vg = np.asarray(v[:, g], dtype=np.float64)
        for h in range(g * G, (g + 1) * G):
            qh = np.asarray(q[:, h], dtype=np.float64)
            doh = np.asarray(do[:, h], dtype=np.float64)
            dQ[:, h] = 0.0
            for n in range(N):
                seg = slice(o[n], o[n + 1])
                qn = np.concatenate([qh[:P], qh[seg]])
                if qn.shape[0] == 0:
                    continue
                kn = np.concatenate([kg[:P], kg[seg]])
                vn = np.concatenate([vg[:P], vg[seg]])
                On, lsen = causal_attention_fwd(qn, kn, vn, scale, block)
                if n == 0:
                    O[:P, h] = On[:P]
                    LSE[h, :P] = lsen[:P]
                elif P:
                    maxdiff = max(maxdiff, float(np.max(np.abs(On[:P] - O[:P, h]))),
                                  float(np.max(np.abs(lsen[:P] - LSE[h, :P]))))
                O[seg, h] = On[P:]
                LSE[h, seg] = lsen[P:]
                if not backward:
                    continue
                don = np.concatenate([doh[:P] / N, doh[seg]])
                dqn, dkn, dvn = causal_attention_bwd(qn, kn, vn, don, scale, block)
                dQ[:P, h] += dqn[:P]
                dQ[seg, h] = dqn[P:]
                dK[:P, g] += dkn[:P]
                dV[:P, g] += dvn[:P]
                dK[seg, g] += dkn[P:]
                dV[seg, g] += dvn[P:]
    out = {"O": O, "LSE": LSE, "prompt_replica_maxdiff": maxdiff, "kv_heads": kv_list}
    if backward:
        out.update(dQ=dQ, dK=dK, dV=dV)
    return out
