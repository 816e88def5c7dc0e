"""Packed decoder layer (shared-prompt attention inside a full layer).

CPU pins for the float64 reference (oracle/layer.py): rotary embedding
properties, RMSNorm, and the packing identity itself (the layer on packed
tokens with packed positions and the packed attention mask equals the layer
run on each replicated sequence). GPU: the product layer (bf16 projections and
MLP, the library's attention kernels) against that reference.
"""
import numpy as np
import pytest
import torch

from oracle import layer64, replicated_layer, rms_norm64, rope64

CFG = dict(hidden=64, Hq=4, Hkv=2, d=16, inter=96, eps=1e-6, rope_theta=10000.0)


def _weights(cfg, seed, scale=0.2):
    g = torch.Generator().manual_seed(seed)
    h, d = cfg["hidden"], cfg["d"]
    rnd = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64) * scale  # noqa: E731
    return {"ln1": 1 + 0.1 * rnd(h), "wq": rnd(cfg["Hq"] * d, h), "wk": rnd(cfg["Hkv"] * d, h),
            "wv": rnd(cfg["Hkv"] * d, h), "wo": rnd(h, cfg["Hq"] * d), "ln2": 1 + 0.1 * rnd(h),
            "wg": rnd(cfg["inter"], h), "wu": rnd(cfg["inter"], h), "wd": rnd(h, cfg["inter"])}


def test_rope_preserves_norm_and_depends_on_relative_position():
    g = torch.Generator().manual_seed(1)
    q = torch.randn(1, 1, 16, generator=g, dtype=torch.float64)
    k = torch.randn(1, 1, 16, generator=g, dtype=torch.float64)
    for m in (0, 3, 250):
        assert torch.allclose(rope64(q, torch.tensor([m]), 1e4).norm(), q.norm(), rtol=1e-12)

    def dot(m, n):
        return float((rope64(q, torch.tensor([m]), 1e4) * rope64(k, torch.tensor([n]), 1e4)).sum())
    assert abs(dot(7, 3) - dot(107, 103)) < 1e-10
    assert abs(dot(7, 3) - dot(3, 7)) > 1e-6   # not symmetric: it is a rotation by m - n
    assert torch.equal(rope64(q, torch.tensor([0]), 1e4), q)


def test_rope_frequency_schedule_closed_form():
    """Rotary frequencies of the RoFormer / rotate-half convention: pair i of a
    d-wide head (elements i and i + d/2) turns by pos * theta^(-2i/d). Pinned by
    values with closed forms at theta = 10^4, d = 16: pair 0 turns by pos
    radians, pair 1 by pos * 10^-0.5 (= pos / sqrt(10)), pair 7 = d/2 - 1 by
    pos * 10^-3.5. A unit vector on element i must come out as
    cos(a) e_i + sin(a) e_(i + d/2); theta^(-i/d) or theta^(-2(i+1)/d) would
    move pair 1 to 10^-0.25 or 10^-1."""
    d, theta = 16, 1.0e4
    expect = {0: 1.0, 1: 1.0 / np.sqrt(10.0), 7: 10.0 ** -3.5}
    for pos in (1, 3):
        for i, f in expect.items():
            x = torch.zeros(1, 1, d, dtype=torch.float64)
            x[0, 0, i] = 1.0
            y = rope64(x, torch.tensor([pos]), theta)[0, 0]
            want = torch.zeros(d, dtype=torch.float64)
            want[i] = np.cos(pos * f)
            want[i + d // 2] = np.sin(pos * f)
            assert torch.allclose(y, want, rtol=0, atol=1e-14), (pos, i, y, want)
            # the partner element rotates the other way: e_(i + d/2) -> -sin e_i + cos e_(i + d/2)
            x2 = torch.zeros(1, 1, d, dtype=torch.float64)
            x2[0, 0, i + d // 2] = 1.0
            y2 = rope64(x2, torch.tensor([pos]), theta)[0, 0]
            want2 = torch.zeros(d, dtype=torch.float64)
            want2[i] = -np.sin(pos * f)
            want2[i + d // 2] = np.cos(pos * f)
            assert torch.allclose(y2, want2, rtol=0, atol=1e-14), (pos, i)


def test_rms_norm_unit_rms():
    x = torch.randn(5, 32, dtype=torch.float64) * 7
    y = rms_norm64(x, torch.ones(32, dtype=torch.float64), 0.0)
    assert torch.allclose(y.pow(2).mean(-1), torch.ones(5, dtype=torch.float64), rtol=1e-12)


def test_rms_norm_weight_closed_form():
    """x = 2 * (1, -1, 1, -1) has root mean square 2, so with eps = 0 the
    normalised row is (1, -1, 1, -1) and the weight multiplies it elementwise;
    eps = 12 makes the denominator sqrt(4 + 12) = 4."""
    x = torch.tensor([[2.0, -2.0, 2.0, -2.0]], dtype=torch.float64)
    w = torch.tensor([1.0, 2.0, 3.0, 4.0], dtype=torch.float64)
    assert torch.equal(rms_norm64(x, w, 0.0), torch.tensor([[1.0, -2.0, 3.0, -4.0]], dtype=torch.float64))
    assert torch.allclose(rms_norm64(x, w, 12.0), torch.tensor([[0.5, -1.0, 1.5, -2.0]], dtype=torch.float64),
                          rtol=0, atol=1e-15)


def _packed_mask(P, lengths):
    T = P + sum(lengths)
    M = torch.zeros(T, T, dtype=torch.bool)
    for t in range(P):
        M[t, : t + 1] = True
    o = P
    for r in lengths:
        for i in range(r):
            M[o + i, :P] = True
            M[o + i, o: o + i + 1] = True
        o += r
    return M


@pytest.mark.parametrize("P,lengths", [(6, [3, 0, 5]), (0, [4, 2]), (9, [1])])
def test_packed_layer_equals_replicated_layer(P, lengths):
    """The packing identity, in float64: one layer on the packed tokens (packed
    positions, packed attention mask, loss sum <dy, y>) gives the replicated
    layer's outputs, input gradients and weight gradients."""
    g = torch.Generator().manual_seed(3 + P)
    T = P + sum(lengths)
    x = torch.randn(T, CFG["hidden"], generator=g, dtype=torch.float64)
    dy = torch.randn(T, CFG["hidden"], generator=g, dtype=torch.float64)
    w = _weights(CFG, 5)
    y_rep, dx_rep, dw_rep = replicated_layer(x, w, CFG, P, lengths, dy)
    pos = torch.cat([torch.arange(P)] + [P + torch.arange(r) for r in lengths])
    xl = x.clone().requires_grad_(True)
    wl = {k: t.clone().requires_grad_(True) for k, t in w.items()}
    y = layer64(xl, wl, CFG, pos, mask=_packed_mask(P, lengths))
    (y * dy).sum().backward()
    assert torch.allclose(y.detach(), y_rep, rtol=1e-10, atol=1e-10)
    assert torch.allclose(xl.grad, dx_rep, rtol=1e-9, atol=1e-9)
    for k in w:
        assert torch.allclose(wl[k].grad, dw_rep[k], rtol=1e-9, atol=1e-9), k


@pytest.mark.gpu
def test_gpu_packed_layer_against_replicated_reference():
    from exact_shared_prefix_amd import Packing
    from exact_shared_prefix_amd.layer import LayerConfig, layer_forward

    cfg = LayerConfig(hidden=256, Hq=4, Hkv=2, d=64, inter=512, eps=1e-6, rope_theta=1.0e4)
    P, lengths = 70, [33, 0, 91, 5]
    T = P + sum(lengths)
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(11)
    x = torch.randn(T, cfg.hidden, generator=g).to(torch.bfloat16)
    dy = torch.randn(T, cfg.hidden, generator=g).to(torch.bfloat16)
    h = cfg.hidden
    wcpu = {"ln1": (1 + 0.1 * torch.randn(h, generator=g)), "wq": torch.randn(cfg.Hq * cfg.d, h, generator=g) * 0.06,
            "wk": torch.randn(cfg.Hkv * cfg.d, h, generator=g) * 0.06,
            "wv": torch.randn(cfg.Hkv * cfg.d, h, generator=g) * 0.06,
            "wo": torch.randn(h, cfg.Hq * cfg.d, generator=g) * 0.06, "ln2": (1 + 0.1 * torch.randn(h, generator=g)),
            "wg": torch.randn(cfg.inter, h, generator=g) * 0.06, "wu": torch.randn(cfg.inter, h, generator=g) * 0.06,
            "wd": torch.randn(h, cfg.inter, generator=g) * 0.06}
    wcpu = {k: t.to(torch.bfloat16) for k, t in wcpu.items()}
    xg = x.to(dev).requires_grad_(True)
    wg = {k: t.to(dev).requires_grad_(True) for k, t in wcpu.items()}
    y = layer_forward(xg, wg, cfg, Packing(P, lengths))
    y.backward(dy.to(dev))
    torch.cuda.synchronize()
    ref_cfg = dict(hidden=h, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, inter=cfg.inter, eps=cfg.eps,
                   rope_theta=cfg.rope_theta)
    y_ref, dx_ref, dw_ref = replicated_layer(x.double(), {k: t.double() for k, t in wcpu.items()},
                                             ref_cfg, P, lengths, dy.double())

    def rel(a, b):
        a, b = a.detach().double().cpu(), b.double()
        return float((a - b).norm() / b.norm())

    errs = {"y": rel(y, y_ref), "dx": rel(xg.grad, dx_ref)}
    errs.update({f"d{k}": rel(wg[k].grad, dw_ref[k]) for k in wcpu})
    print(errs, flush=True)
    for k, e in errs.items():
        assert e <= 2e-2, (k, e)
