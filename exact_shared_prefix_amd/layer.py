"""A packed decoder layer around the shared-prompt attention (random weights).

The DualKV arXiv abstract extends the token saving from attention to the whole
model: in a decoder-only model causal masking makes the prompt's hidden states
identical across the N sequences at every layer, so the per-token operations
(norms, projections, MLP) can process the prompt once, on P + sum(R_n) packed
tokens instead of N(P+R) (ratio rho = N(P+R)/(P+NR)). This module is one such
layer with Qwen3-8B-like shapes: RMSNorm, Q/K/V projections, rotary position
embedding with per-sequence positions (a response token at offset r of its
response sits at position P + r of its own sequence), the shared-prompt
attention of this package (its HIP kernels, forward and backward), the output
projection, RMSNorm and a SwiGLU MLP, with residual connections.

The projections and the MLP are plain dense matrix products (torch / hipBLASLt);
the attention is the package's C ABI. Weights are random (seeded): the layer
measures cost and checks exactness of the packing, it is not a trained model.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from .binding import DualKVAttention, Packing


@dataclass(frozen=True)
class LayerConfig:
    hidden: int = 4096
    Hq: int = 32
    Hkv: int = 8
    d: int = 128
    inter: int = 12288
    eps: float = 1e-6
    rope_theta: float = 1.0e6


def init_weights(cfg: LayerConfig, seed: int, device, dtype=torch.bfloat16) -> dict:
    """Seeded random weights (normal, std 0.02; norm gains 1)."""
    g = torch.Generator(device="cpu").manual_seed(seed)

    def rnd(*shape):
        return (torch.randn(*shape, generator=g, dtype=torch.float32) * 0.02).to(device=device, dtype=dtype)

    h, d = cfg.hidden, cfg.d
    return {
        "ln1": torch.ones(h, device=device, dtype=dtype),
        "wq": rnd(cfg.Hq * d, h), "wk": rnd(cfg.Hkv * d, h), "wv": rnd(cfg.Hkv * d, h),
        "wo": rnd(h, cfg.Hq * d),
        "ln2": torch.ones(h, device=device, dtype=dtype),
        "wg": rnd(cfg.inter, h), "wu": rnd(cfg.inter, h), "wd": rnd(h, cfg.inter),
    }


def packed_positions(P: int, lengths: Sequence[int]) -> torch.Tensor:
    """Position of each packed token inside its own sequence [prompt; response]:
    prompt token i -> i, token r of a response -> P + r."""
    parts = [torch.arange(P)] + [P + torch.arange(int(r)) for r in lengths]
    return torch.cat(parts).to(torch.int64)


def rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float) -> torch.Tensor:
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype) * w


def rope(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotary embedding, rotate-half form, x [T, H, d], pos [T]."""
    d = x.shape[-1]
    inv = theta ** (-torch.arange(0, d, 2, device=x.device, dtype=torch.float32) / d)
    ang = pos.to(x.device, torch.float32)[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[:, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[:, None, :]
    xf = x.float()
    x1, x2 = xf[..., : d // 2], xf[..., d // 2:]
    rot = torch.cat([-x2, x1], -1)
    return (xf * cos + rot * sin).to(x.dtype)


def layer_forward(x: torch.Tensor, w: dict, cfg: LayerConfig, pk: Packing,
                  pos: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decoder layer on packed tokens x [T, hidden] (bf16, on the GPU)."""
    T = x.shape[0]
    if pos is None:
        pos = packed_positions(pk.P, pk.lengths)
    h = rms_norm(x, w["ln1"], cfg.eps)
    q = (h @ w["wq"].T).view(T, cfg.Hq, cfg.d)
    k = (h @ w["wk"].T).view(T, cfg.Hkv, cfg.d)
    v = (h @ w["wv"].T).view(T, cfg.Hkv, cfg.d).contiguous()
    q = rope(q, pos, cfg.rope_theta).contiguous()
    k = rope(k, pos, cfg.rope_theta).contiguous()
    a = DualKVAttention.apply(q, k, v, pk, cfg.d ** -0.5)
    x = x + a.reshape(T, cfg.Hq * cfg.d) @ w["wo"].T
    h = rms_norm(x, w["ln2"], cfg.eps)
    return x + (torch.nn.functional.silu(h @ w["wg"].T) * (h @ w["wu"].T)) @ w["wd"].T
