"""Work and traffic accounting for the packed shared-prompt layout.

pairs: number of attended (query, key) pairs per query head under the packed
mask (prompt rows causal within the prompt; response rows see the whole
prompt plus their own response causally):
    pairs = P(P+1)/2 + sum_n [R_n P + R_n(R_n+1)/2]   (PP, RP, RR blocks).
Useful FLOPs count 4 d per pair forward (two matrix products) and 10 d per pair
backward (five), times Hq; masked tile waste and recomputation are excluded.
"""
from __future__ import annotations

from typing import Sequence

BF16 = 2
FP32 = 4


def pair_blocks(P: int, lengths: Sequence[int]) -> dict:
    pp = P * (P + 1) // 2
    rp = sum(int(r) * P for r in lengths)
    rr = sum(int(r) * (int(r) + 1) // 2 for r in lengths)
    return {"PP": pp, "RP": rp, "RR": rr, "total": pp + rp + rr}


def pairs(P: int, lengths: Sequence[int]) -> int:
    return pair_blocks(P, lengths)["total"]


def tree_pairs(node_len: Sequence[int], node_parent: Sequence[int]) -> int:
    """Attended pairs per query head of a prefix forest (segments in
    depth-first order): a row at offset i of segment v sees every key of v's
    ancestors and keys 0 .. i of v."""
    depth_keys = []
    total = 0
    for ln, par in zip(node_len, node_parent):
        anc = 0 if par < 0 else depth_keys[par] + int(node_len[par])
        depth_keys.append(anc)
        ln = int(ln)
        total += ln * anc + ln * (ln + 1) // 2
    return total


def replicated_pairs(P: int, lengths: Sequence[int]) -> int:
    """Pairs of the same batch with the prompt copied into every sequence."""
    return sum((P + int(r)) * (P + int(r) + 1) // 2 for r in lengths)


def useful_flops(P: int, lengths: Sequence[int], Hq: int, d: int) -> dict:
    n = pairs(P, lengths)
    return {"fwd": 4 * d * Hq * n, "bwd": 10 * d * Hq * n, "total": 14 * d * Hq * n}


def kernel_flops(P: int, lengths: Sequence[int], Hq: int, d: int) -> dict:
    """FLOPs each kernel executes on attended pairs: the forward (S, PV), the
    key-stationary dK/dV pass (S, dP, dV, dK) and the query-stationary dQ pass
    (S and dP recomputed, dQ)."""
    n = pairs(P, lengths)
    return {"fwd_kernel": 4 * d * Hq * n, "dkv_kernel": 8 * d * Hq * n, "dq_kernel": 6 * d * Hq * n}


def kernel_useful_flops(P: int, lengths: Sequence[int], Hq: int, d: int) -> dict:
    """The part of each kernel's work that counts toward the useful 14 d per
    pair: all of the forward (4 d) and of the dK/dV pass (8 d: the backward's
    S, dP, dV, dK products), and only the dQ product (2 d) of the dQ pass, whose
    S and dP are the dK/dV pass's products computed a second time."""
    n = pairs(P, lengths)
    return {"fwd_kernel": 4 * d * Hq * n, "dkv_kernel": 8 * d * Hq * n, "dq_kernel": 2 * d * Hq * n}


def tokens(P: int, lengths: Sequence[int]) -> tuple[int, int]:
    """(packed, replicated) token counts; their ratio is rho = N(P+R)/(P+NR)."""
    return P + sum(lengths), sum(P + int(r) for r in lengths)


def min_hbm_bytes(P: int, lengths: Sequence[int], Hq: int, Hkv: int, d: int) -> dict:
    """Compulsory HBM bytes: each input read once, each output written once.

    forward: read q, k, v; write o, lse.
    backward: read q, k, v, o, dO, lse; write dQ, dK, dV.
    """
    T = P + sum(lengths)
    xq = T * Hq * d * BF16
    xk = T * Hkv * d * BF16
    lse = T * Hq * FP32
    fwd = xq + 2 * xk + xq + lse
    bwd = 3 * xq + 2 * xk + lse + xq + 2 * xk
    return {"fwd": fwd, "bwd": bwd, "total": fwd + bwd}
