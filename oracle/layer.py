"""Float64 reference of one decoder layer on replicated sequences. TEST
INFRASTRUCTURE ONLY.

The DualKV arXiv abstract: in a decoder-only model causal masking makes the
prompt's hidden states identical across the N sequences at every layer, so
every per-token operation can run on the packed P + sum(R_n) tokens. The
reference here does the opposite, literally: it runs the layer on each
sequence [prompt; response_n] separately (positions 0 .. P + R_n - 1, plain
causal attention from the library's scaled_dot_product_attention) and folds
the results back to the packed layout (prompt outputs from any replica;
prompt input gradients and all weight gradients summed over replicas, the
packed prompt rows' upstream gradient split equally over the N copies).

Layer (Qwen3-8B-like shapes, random weights): RMSNorm -> Q/K/V projections ->
rotary position embedding (rotate-half form, base theta) -> causal attention
with grouped KV heads -> output projection + residual -> RMSNorm -> SwiGLU MLP
+ residual.
"""
from __future__ import annotations

from typing import Sequence

import torch
import torch.nn.functional as F


def rms_norm64(x, w, eps):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * w


def rope64(x, pos, theta):
    """x [L, H, d] float64, pos [L]: rotate the pair (x_i, x_{i + d/2}) by the
    angle pos * theta^(-2i/d)."""
    d = x.shape[-1]
    half = d // 2
    freq = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    ang = pos.to(torch.float64)[:, None, None] * freq[None, None, :]
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * torch.cos(ang) - b * torch.sin(ang), b * torch.cos(ang) + a * torch.sin(ang)], -1)


def layer64(x, w, cfg, pos, mask=None):
    """x [L, hidden] float64; causal attention over the L tokens, or the given
    boolean mask [L, L] (True = attended)."""
    L = x.shape[0]
    Hq, Hkv, d = cfg["Hq"], cfg["Hkv"], cfg["d"]
    h = rms_norm64(x, w["ln1"], cfg["eps"])
    q = rope64((h @ w["wq"].T).view(L, Hq, d), pos, cfg["rope_theta"])
    k = rope64((h @ w["wk"].T).view(L, Hkv, d), pos, cfg["rope_theta"])
    v = (h @ w["wv"].T).view(L, Hkv, d)
    G = Hq // Hkv
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    qh, kh, vh = (t.transpose(0, 1).contiguous() for t in (q, k, v))   # [H, L, d]
    if mask is None:
        a = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True, scale=d ** -0.5)
    else:
        a = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=d ** -0.5)
    x = x + a.transpose(0, 1).reshape(L, Hq * d) @ w["wo"].T
    h = rms_norm64(x, w["ln2"], cfg["eps"])
    return x + (F.silu(h @ w["wg"].T) * (h @ w["wu"].T)) @ w["wd"].T


def replicated_layer(x, w, cfg, P: int, lengths: Sequence[int], dy):
    """Outputs and gradients of sum <dy, y> for the packed batch, computed on
    the N replicated sequences. x, dy: packed [T, hidden]; w: dict of weights.
    Returns (y [T, hidden], dx [T, hidden], dw dict), all float64."""
    N = len(lengths)
    xl = x.detach().to(torch.float64).requires_grad_(True)
    wl = {kk: t.detach().to(torch.float64).requires_grad_(True) for kk, t in w.items()}
    dy = dy.to(torch.float64)
    T = xl.shape[0]
    y = torch.zeros(T, xl.shape[1], dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    o = P
    for n, r in enumerate(lengths):
        r = int(r)
        xn = torch.cat([xl[:P], xl[o:o + r]])
        if xn.shape[0]:
            yn = layer64(xn, wl, cfg, torch.arange(P + r))
            dyn = torch.cat([dy[:P] / N, dy[o:o + r]])
            loss = loss + (yn * dyn).sum()
            if n == 0:
                y[:P] = yn[:P].detach()
            y[o:o + r] = yn[P:].detach()
        o += r
    loss.backward()
    return y, xl.grad, {kk: t.grad for kk, t in wl.items()}
