"""Seeded synthetic inputs for shared-prompt attention workloads.

This module only describes workloads and draws random numbers. It holds none of
the attention arithmetic, so both the CPU oracle (test infrastructure) and the
HIP path can consume what it produces without sharing any computation.

Workloads follow the packed micro-batch of the DualKV pages (the arXiv abstract:
one shared prompt of P tokens followed by N responses, P+NR tokens instead of
N(P+R)); the head shapes are the Qwen3-8B ones the pages' GRPO runs use.

Random numbers: every tensor is split into fixed-size chunks; chunk c of tensor
number i under seed s is drawn from numpy's Philox bit generator seeded with
SeedSequence([s, i, c]) as float64 standard normals, multiplied by the
workload's input scale, rounded to float32 and then to bfloat16 (round to
nearest even). The draw is integer-exact up to the final rounding, so the same
seed gives the same bf16 bits on any x86 host with this numpy/torch. Ragged
response lengths are drawn first, as integers uniform on [lo, hi] inclusive,
from SeedSequence([s, 0, 0]).
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

_CHUNK = 1 << 22  # elements per independently seeded chunk

# tensor ids in the seed sequence (0 is reserved for the length draw)
_TID = {"q": 1, "k": 2, "v": 3, "do": 4}


@dataclass(frozen=True)
class Workload:
    """One packed shared-prompt micro-batch shape.

    R is either an int (uniform response length) or a (lo, hi) pair, meaning
    ragged lengths drawn uniformly from [lo, hi].
    """

    name: str
    P: int
    R: object
    N: int
    Hq: int
    Hkv: int
    d: int
    qkv_scale: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def ragged(self) -> bool:
        return not isinstance(self.R, int)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_p128_r64_n4_gqa2_d64", 128, 64, 4, 4, 2, 64, 1.0, 1,
                 "tiny correctness case, 384 packed tokens"),
        Workload("qwen3_8b_p4k_r4k_n8", 4096, 4096, 8, 32, 8, 128, 0.5, 2,
                 "one attention layer with Qwen3-8B heads, Q/K/V x0.5"),
        Workload("rollout_p8k_r4k_n32", 8192, 4096, 32, 32, 8, 128, 1.0, 3,
                 "large-rollout regime, 139264 packed vs 393216 replicated tokens"),
        Workload("longprompt_p32k_r2k_n16", 32768, 2048, 16, 32, 8, 128, 1.0, 4,
                 "long prompt, short responses, 65536 packed vs 557056 replicated"),
        Workload("ragged_p64k_n16_r256_2048", 65536, (256, 2048), 16, 32, 4, 128, 1.0, 5,
                 "very long prompt, ragged responses packed by offsets"),
    ]
}

# the workload the headline throughput is quoted on
HEADLINE = "rollout_p8k_r4k_n32"


@dataclass(frozen=True)
class GroupWorkload:
    """Several shared-prompt groups packed back to back in one call: B groups
    of P prompt tokens and N responses of R tokens each (Qwen3-8B heads)."""

    name: str
    B: int
    P: int
    R: int
    N: int
    Hq: int
    Hkv: int
    d: int
    seed: int = 0
    note: str = ""

    @property
    def groups(self) -> list:
        return [(self.P, [self.R] * self.N) for _ in range(self.B)]

    @property
    def T(self) -> int:
        return self.B * (self.P + self.N * self.R)


GROUP_WORKLOADS = {
    w.name: w
    for w in [
        GroupWorkload("microbatch_g8_p2k_r1k_n8", 8, 2048, 1024, 8, 32, 8, 128, 6,
                      "8 prompt groups in one call, 81920 packed vs 196608 replicated tokens"),
    ]
}


def group_workload_inputs(w: GroupWorkload | str) -> Inputs:
    """Inputs of a multi-group workload: the [T, H, d] tensors are drawn like
    a single packing of T rows (P = 0, one segment); the grouping is
    w.groups."""
    if isinstance(w, str):
        w = GROUP_WORKLOADS[w]
    inp = make_inputs(0, [w.T], w.Hq, w.Hkv, w.d, seed=w.seed)
    inp.meta["workload"] = w.name
    inp.meta["groups"] = w.groups
    return inp


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def response_lengths(w: Workload) -> list[int]:
    """Per-response token counts R_n, n = 0..N-1 (drawn first for ragged)."""
    if not w.ragged:
        return [int(w.R)] * w.N
    lo, hi = w.R
    g = np.random.Generator(np.random.Philox(np.random.SeedSequence([w.seed, 0, 0])))
    return [int(x) for x in g.integers(lo, hi, size=w.N, endpoint=True)]


def _normal_bf16(seed: int, tid: int, shape: Sequence[int], scale: float,
                 pool: ThreadPoolExecutor) -> torch.Tensor:
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=torch.bfloat16)

    def one(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, tid, c])))
        x = g.standard_normal(hi - lo, dtype=np.float64)
        if scale != 1.0:
            x *= scale
        out[lo:hi] = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)

    list(pool.map(one, range((n + _CHUNK - 1) // _CHUNK)))
    return out.view(*shape)


@dataclass
class Inputs:
    """bf16 CPU tensors in the packed [T, H, d] layout plus the shape data."""

    P: int
    lengths: list
    Hq: int
    Hkv: int
    d: int
    scale: float  # softmax scale
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def T(self) -> int:
        return self.P + sum(self.lengths)

    def digest(self) -> str:
        """sha256 over the raw bf16 bytes of q, k, v, dO (input identity)."""
        h = hashlib.sha256()
        for t in (self.q, self.k, self.v, self.do):
            h.update(t.contiguous().view(torch.int16).numpy().tobytes())
        return h.hexdigest()


def make_inputs(P: int, lengths: Sequence[int], Hq: int, Hkv: int, d: int, *,
                seed: int, qkv_scale: float = 1.0, scale: Optional[float] = None,
                const_v: bool = False) -> Inputs:
    """Draw q, k, v, dO for an explicit packing (P, response lengths).

    const_v replaces every V row of a KV head by that head's first prompt row
    (or first row if P == 0), a degenerate case whose attention output is known.
    """
    lengths = [int(x) for x in lengths]
    T = P + sum(lengths)
    with ThreadPoolExecutor(_threads()) as pool:
        q = _normal_bf16(seed, _TID["q"], (T, Hq, d), qkv_scale, pool)
        k = _normal_bf16(seed, _TID["k"], (T, Hkv, d), qkv_scale, pool)
        v = _normal_bf16(seed, _TID["v"], (T, Hkv, d), qkv_scale, pool)
        do = _normal_bf16(seed, _TID["do"], (T, Hq, d), 1.0, pool)
    if const_v and T > 0:
        v = v[0:1].expand(T, Hkv, d).contiguous()
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    return Inputs(P, lengths, Hq, Hkv, d, float(scale), q, k, v, do,
                  {"seed": seed, "qkv_scale": qkv_scale, "const_v": const_v})


def workload_inputs(w: Workload | str) -> Inputs:
    if isinstance(w, str):
        w = WORKLOADS[w]
    inp = make_inputs(w.P, response_lengths(w), w.Hq, w.Hkv, w.d,
                      seed=w.seed, qkv_scale=w.qkv_scale)
    inp.meta["workload"] = w.name
    return inp
