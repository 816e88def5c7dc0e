"""Pins for the CPU oracle: each check ties it to something other than itself.

* library attention (torch scaled_dot_product_attention in float64) plus
  autograd through a prompt that is shared by concatenation N times;
* central finite differences of the packed loss L = sum <dO, O>;
* the closed form at scale 0 (uniform attention over A(t));
* constant V (O = that row, zero query/key gradients);
* prompt invariance, locality and response-permutation invariants;
* the two oracle formulations (literal replication, packed per-row/per-key)
  against each other.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from exact_shared_prefix_amd.inputs import make_inputs, response_lengths, WORKLOADS
from oracle import oracle_fwd_bwd, rows_fwd_bwd, keys_dkdv, attended_keys
from tests.conftest import to_np


def _attended(t, P, lengths):
    """A(t) written out independently of the oracle: a prompt row sees prompt
    keys 0..t; a row of response n sees the whole prompt and its own response
    up to itself."""
    if t < P:
        return list(range(t + 1))
    start = P
    for r in lengths:
        if t < start + r:
            return list(range(P)) + list(range(start, t + 1))
        start += r
    raise IndexError(t)


def _inputs_np(inp):
    return tuple(to_np(x).astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))


def _offsets(P, lengths):
    o = [P]
    for r in lengths:
        o.append(o[-1] + r)
    return o


def _torch_reference(q, k, v, do, P, lengths, scale):
    """Replicated attention built from the library SDPA, gradients by autograd.

    The prompt rows enter every sequence through torch.cat of the same leaf
    tensors, so autograd itself sums the N copies' prompt gradients.
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    N = len(lengths)
    o = _offsets(P, lengths)
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    dot = torch.tensor(do, dtype=torch.float64)
    O = torch.zeros(T, Hq, d, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for n in range(N):
        a, b = o[n], o[n + 1]
        qn = torch.cat([qt[:P], qt[a:b]])
        if qn.shape[0] == 0:
            continue
        kn = torch.cat([kt[:P], kt[a:b]]).repeat_interleave(G, dim=1)
        vn = torch.cat([vt[:P], vt[a:b]]).repeat_interleave(G, dim=1)
        On = F.scaled_dot_product_attention(
            qn.transpose(0, 1)[None], kn.transpose(0, 1)[None], vn.transpose(0, 1)[None],
            is_causal=True, scale=scale)[0].transpose(0, 1)
        dOn = torch.cat([dot[:P] / N, dot[a:b]])
        loss = loss + (On * dOn).sum()
        with torch.no_grad():
            if n == 0:
                O[:P] = On[:P]
            O[a:b] = On[P:]
    loss.backward()
    return O.numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


SMALL_CASES = [
    # P, lengths, Hq, Hkv, d
    (7, [5, 0, 9], 4, 2, 8),
    (16, [3, 11], 2, 2, 4),       # MHA
    (0, [6, 4, 1], 4, 1, 8),      # no prompt (replicated layout)
    (12, [10], 3, 1, 8),          # N = 1
]


@pytest.mark.parametrize("case", SMALL_CASES)
def test_oracle_matches_library_attention_and_autograd(case):
    P, lengths, Hq, Hkv, d = case
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=11)
    q, k, v, do = _inputs_np(inp)
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=4)
    O, dq, dk, dv = _torch_reference(q, k, v, do, P, lengths, inp.scale)
    assert _rel(ref["O"], O) < 1e-12
    assert _rel(ref["dQ"], dq) < 1e-12
    assert _rel(ref["dK"], dk) < 1e-12
    assert _rel(ref["dV"], dv) < 1e-12
    assert ref["prompt_replica_maxdiff"] < 1e-12


def test_n1_is_ordinary_causal_attention():
    P, R, Hq, Hkv, d = 20, 13, 2, 1, 16
    inp = make_inputs(P, [R], Hq, Hkv, d, seed=3)
    q, k, v, do = _inputs_np(inp)
    ref = oracle_fwd_bwd(q, k, v, do, P, [R], inp.scale, block=8)
    # plain causal attention over the whole P + R sequence
    qt = torch.tensor(q, dtype=torch.float64).transpose(0, 1)[None]
    kt = torch.tensor(k, dtype=torch.float64).repeat_interleave(2, 1).transpose(0, 1)[None]
    vt = torch.tensor(v, dtype=torch.float64).repeat_interleave(2, 1).transpose(0, 1)[None]
    O = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=inp.scale)
    assert _rel(ref["O"], O[0].transpose(0, 1).numpy()) < 1e-12


def test_lse_against_softmax_output_with_identity_v():
    """With V = I (one-hot rows), O_t is the softmax row, so
    LSE_t = scale * q_t.k_j - log O_tj for every attended key j."""
    P, lengths = 6, [4, 5]
    T = P + sum(lengths)
    Hq, Hkv, d = 2, 1, T
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=5)
    q, k, _, do = (x.astype(np.float64) for x in _inputs_np(inp))
    v = np.eye(T)[:, None, :].astype(np.float64)
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, backward=False, block=3)
    for h in range(Hq):
        for t in range(T):
            for j in _attended(t, P, lengths):
                want = inp.scale * float(q[t, h] @ k[j, 0]) - math.log(ref["O"][t, h, j])
                assert abs(ref["LSE"][h, t] - want) < 1e-12
            # and keys outside A(t) get exactly zero weight
            outside = np.setdiff1d(np.arange(T), _attended(t, P, lengths))
            assert np.all(ref["O"][t, h, outside] == 0.0)


def _closed_form_scale0(v, do, P, lengths, Hq):
    """scale = 0: uniform attention over A(t) (written with plain loops)."""
    T, Hkv, d = v.shape
    G = Hq // Hkv
    O = np.zeros((T, Hq, d))
    LSE = np.zeros((Hq, T))
    dV = np.zeros((T, Hkv, d))
    for t in range(T):
        A = _attended(t, P, lengths)
        for h in range(Hq):
            g = h // G
            O[t, h] = sum(v[j, g].astype(np.float64) for j in A) / len(A)
            LSE[h, t] = math.log(len(A))
            for j in A:
                dV[j, g] += do[t, h] / len(A)
    return O, LSE, dV


@pytest.mark.parametrize("case", [(9, [7, 0, 3, 12], 4, 2, 8), (0, [5, 8], 2, 1, 4)])
def test_scale_zero_closed_form(case):
    P, lengths, Hq, Hkv, d = case
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=2, scale=0.0)
    q, k, v, do = _inputs_np(inp)
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, 0.0, block=5)
    O, LSE, dV = _closed_form_scale0(v, do, P, lengths, Hq)
    assert np.max(np.abs(ref["O"] - O)) < 1e-12
    assert np.max(np.abs(ref["LSE"] - LSE)) < 1e-12
    assert np.max(np.abs(ref["dV"] - dV)) < 1e-12
    assert np.max(np.abs(ref["dQ"])) == 0.0
    assert np.max(np.abs(ref["dK"])) == 0.0


def test_constant_v():
    P, lengths, Hq, Hkv, d = 10, [6, 9, 2], 4, 2, 8
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=4, const_v=True)
    q, k, v, do = _inputs_np(inp)
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=4)
    G = Hq // Hkv
    for h in range(Hq):
        assert np.max(np.abs(ref["O"][:, h] - v[0, h // G])) < 1e-13
    scale_ref = np.abs(do).max() * np.abs(k).max() * np.abs(q).max()
    assert np.max(np.abs(ref["dQ"])) < 1e-13 * scale_ref
    assert np.max(np.abs(ref["dK"])) < 1e-13 * scale_ref


def _packed_loss(q, k, v, do, P, lengths, scale):
    out = oracle_fwd_bwd(q, k, v, do, P, lengths, scale, backward=False, block=3)
    return float(np.sum(out["O"] * do))


def test_finite_differences_of_packed_loss():
    """Central differences of L = sum_t <dO_t, O_t> on the packed outputs.

    This pins the backward formulas and the split of the prompt's upstream
    gradient over the N copies, independently of the autograd reference."""
    P, lengths, Hq, Hkv, d = 5, [3, 0, 4], 2, 1, 4
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=9)
    q, k, v, do = (x.astype(np.float64) for x in _inputs_np(inp))
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=2)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, arr, grad in (("q", q, ref["dQ"]), ("k", k, ref["dK"]), ("v", v, ref["dV"])):
        T = arr.shape[0]
        picks = [(0, 0, 0), (P - 1, arr.shape[1] - 1, 1), (P, 0, 2), (T - 1, 0, 3)]
        picks += [tuple(int(rng.integers(s)) for s in arr.shape) for _ in range(8)]
        for idx in picks:
            save = arr[idx]
            arr[idx] = save + eps
            lp = _packed_loss(q, k, v, do, P, lengths, inp.scale)
            arr[idx] = save - eps
            lm = _packed_loss(q, k, v, do, P, lengths, inp.scale)
            arr[idx] = save
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


def test_locality_and_prompt_invariance():
    P, lengths, Hq, Hkv, d = 8, [5, 7, 6], 2, 1, 8
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=6)
    q, k, v, do = (x.astype(np.float64) for x in _inputs_np(inp))
    base = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=4)
    o = _offsets(P, lengths)
    # perturb response 1 (rows o1..o2) in q, k, v and dO
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    sl = slice(o[1], o[2])
    rng = np.random.default_rng(1)
    for a in (q2, k2, v2, do2):
        a[sl] += rng.standard_normal(a[sl].shape)
    pert = oracle_fwd_bwd(q2, k2, v2, do2, P, lengths, inp.scale, block=4)
    others = np.r_[0:P, o[0]:o[1], o[2]:o[3]]
    for key in ("O", "dQ"):
        assert np.array_equal(base[key][others], pert[key][others])
    assert np.array_equal(base["LSE"][:, others], pert["LSE"][:, others])
    resp_other = np.r_[o[0]:o[1], o[2]:o[3]]
    for key in ("dK", "dV"):
        assert np.array_equal(base[key][resp_other], pert[key][resp_other])
        # every response attends the prompt, so prompt key gradients change
        assert not np.allclose(base[key][:P], pert[key][:P])


def test_response_permutation():
    P, lengths, Hq, Hkv, d = 6, [4, 7, 2], 2, 1, 8
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=8)
    q, k, v, do = (x.astype(np.float64) for x in _inputs_np(inp))
    base = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=4)
    o = _offsets(P, lengths)
    perm = [2, 0, 1]
    segs = [np.arange(o[n], o[n + 1]) for n in range(3)]
    idx = np.concatenate([np.arange(P)] + [segs[n] for n in perm])
    new_len = [lengths[n] for n in perm]
    out = oracle_fwd_bwd(q[idx], k[idx], v[idx], do[idx], P, new_len, inp.scale, block=4)
    for key in ("O", "dQ", "dK", "dV"):
        assert np.max(np.abs(out[key] - base[key][idx])) < 1e-12
    assert np.max(np.abs(out["LSE"] - base["LSE"][:, idx])) < 1e-12


def test_replica_zero_gradient_split_gives_same_sums():
    """Any split of the prompt's upstream gradient that sums to dO_prompt gives
    the same packed gradients: here all of it goes to copy 0 (autograd)."""
    P, lengths, Hq, Hkv, d = 6, [3, 5], 2, 1, 4
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=10)
    q, k, v, do = (x.astype(np.float64) for x in _inputs_np(inp))
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=4)
    o = _offsets(P, lengths)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    loss = 0
    for n in range(2):
        a, b = o[n], o[n + 1]
        qn = torch.cat([qt[:P], qt[a:b]]).transpose(0, 1)[None]
        kn = torch.cat([kt[:P], kt[a:b]]).repeat_interleave(2, 1).transpose(0, 1)[None]
        vn = torch.cat([vt[:P], vt[a:b]]).repeat_interleave(2, 1).transpose(0, 1)[None]
        On = F.scaled_dot_product_attention(qn, kn, vn, is_causal=True, scale=inp.scale)[0].transpose(0, 1)
        w = torch.tensor(do[:P] if n == 0 else 0 * do[:P])
        loss = loss + (On[:P] * w).sum() + (On[P:] * torch.tensor(do[a:b])).sum()
    loss.backward()
    assert _rel(ref["dQ"], qt.grad.numpy()) < 1e-12
    assert _rel(ref["dK"], kt.grad.numpy()) < 1e-12
    assert _rel(ref["dV"], vt.grad.numpy()) < 1e-12


@pytest.mark.parametrize("case", [(13, [9, 0, 17, 4], 4, 2, 8), (0, [7, 11], 2, 1, 8)])
def test_sampled_oracle_matches_replicated(case):
    P, lengths, Hq, Hkv, d = case
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=12)
    q, k, v, do = _inputs_np(inp)
    T = inp.T
    ref = oracle_fwd_bwd(q, k, v, do, P, lengths, inp.scale, block=5)
    rows = list(range(T))
    s = rows_fwd_bwd(q, k, v, do, P, lengths, inp.scale, rows)
    assert np.max(np.abs(s["O"] - ref["O"])) < 1e-12
    assert np.max(np.abs(s["LSE"] - ref["LSE"])) < 1e-12
    assert np.max(np.abs(s["dQ"] - ref["dQ"])) < 1e-12
    for g in range(Hkv):
        for keys in ([0, T - 1], list(range(T)), [P] if P < T else [0]):
            kk = keys_dkdv(q, k, v, do, P, lengths, inp.scale, keys, g, row_block=3)
            assert np.max(np.abs(kk["dK"] - ref["dK"][keys, g])) < 1e-12
            assert np.max(np.abs(kk["dV"] - ref["dV"][keys, g])) < 1e-12


def test_attended_keys_definition():
    P, lengths = 4, [2, 0, 3]
    assert list(attended_keys(0, P, lengths)) == [0]
    assert list(attended_keys(3, P, lengths)) == [0, 1, 2, 3]
    assert list(attended_keys(4, P, lengths)) == [0, 1, 2, 3, 4]
    assert list(attended_keys(5, P, lengths)) == [0, 1, 2, 3, 4, 5]
    assert list(attended_keys(6, P, lengths)) == [0, 1, 2, 3, 6]
    assert list(attended_keys(8, P, lengths)) == [0, 1, 2, 3, 6, 7, 8]
    with pytest.raises(IndexError):
        attended_keys(9, P, lengths)


def test_attended_keys_against_independent_definition():
    for P, lengths in ((5, [3, 0, 4, 1]), (0, [2, 3]), (9, []), (1, [1, 1])):
        T = P + sum(lengths)
        for t in range(T):
            assert list(attended_keys(t, P, lengths)) == _attended(t, P, lengths)


def test_ragged_lengths_draw():
    w = WORKLOADS["ragged_p64k_n16_r256_2048"]
    lens = response_lengths(w)
    assert len(lens) == 16 and all(256 <= x <= 2048 for x in lens)
    assert lens == response_lengths(w)  # deterministic


# --------------------------------------------------- several prompt groups --
from oracle import attended_keys_groups, group_starts, oracle_groups_fwd_bwd  # noqa: E402


def _groups_attended(t, groups):
    """A(t) of a multi-group batch written out independently: find the group
    holding row t, then the single-group rule inside it, in absolute indices."""
    start = 0
    for P, L in groups:
        size = P + sum(L)
        if t < start + size:
            return [start + j for j in _attended(t - start, P, L)]
        start += size
    raise IndexError(t)


def _dense_masked_reference(q, k, v, do, groups, scale):
    """Dense attention over the whole packed tensor with an explicit boolean
    mask M[t, j] = (j in A(t)), float64, gradients of L = sum <dO, O> by
    autograd: a formulation with no replication and no per-group slicing."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    M = torch.zeros(T, T, dtype=torch.bool)
    for t in range(T):
        M[t, _groups_attended(t, groups)] = True
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    O = torch.zeros(T, Hq, d, dtype=torch.float64)
    LSE = torch.zeros(Hq, T, dtype=torch.float64)
    for h in range(Hq):
        S = scale * (qt[:, h] @ kt[:, h // G].T)
        S = S.masked_fill(~M, float("-inf"))
        LSE[h] = torch.logsumexp(S, dim=1)
        O[:, h] = torch.softmax(S, dim=1) @ vt[:, h // G]
    (O * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return {"O": O.detach().numpy(), "LSE": LSE.detach().numpy(), "dQ": qt.grad.numpy(),
            "dK": kt.grad.numpy(), "dV": vt.grad.numpy()}


GROUP_CASES = [
    # (groups, Hq, Hkv, d)
    ([(5, [3, 0, 4]), (0, [6]), (4, [2, 5])], 4, 2, 8),
    ([(7, [1, 2]), (3, [4]), (6, [0, 3, 2])], 2, 1, 4),
]


@pytest.mark.parametrize("case", range(len(GROUP_CASES)))
def test_group_oracle_matches_dense_masked_attention(case):
    groups, Hq, Hkv, d = GROUP_CASES[case]
    T = group_starts(groups)[-1]
    rng = np.random.default_rng(60 + case)
    q, do = rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hq, d))
    k, v = rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hkv, d))
    scale = 0.7
    got = oracle_groups_fwd_bwd(q, k, v, do, groups, scale)
    ref = _dense_masked_reference(q, k, v, do, groups, scale)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.max(np.abs(got[key] - ref[key])) <= 1e-10, key


def test_group_oracle_one_group_is_the_single_group_oracle():
    inp = make_inputs(6, [3, 0, 5], 4, 2, 8, seed=61)
    q, k, v, do = _inputs_np(inp)
    a = oracle_groups_fwd_bwd(q, k, v, do, [(6, [3, 0, 5])], inp.scale)
    b = oracle_fwd_bwd(q, k, v, do, 6, [3, 0, 5], inp.scale)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[key], b[key]), key


def test_groups_are_isolated():
    """Changing every input of the middle group leaves the other groups'
    outputs and gradients bitwise unchanged."""
    groups = [(4, [2, 3]), (3, [5]), (2, [1, 4])]
    s = group_starts(groups)
    T = s[-1]
    rng = np.random.default_rng(62)
    x = [rng.standard_normal((T, 2, 4)) for _ in range(2)] + [rng.standard_normal((T, 1, 4)) for _ in range(2)]
    q, do, k, v = x
    a = oracle_groups_fwd_bwd(q, k, v, do, groups, 0.5)
    q2, k2, v2, do2 = (t.copy() for t in (q, k, v, do))
    for t in (q2, k2, v2, do2):
        t[s[1]:s[2]] += rng.standard_normal(t[s[1]:s[2]].shape)
    b = oracle_groups_fwd_bwd(q2, k2, v2, do2, groups, 0.5)
    keep = np.r_[0:s[1], s[2]:T]
    for key in ("O", "dQ", "dK", "dV"):
        assert np.array_equal(a[key][keep], b[key][keep]), key
        assert not np.allclose(a[key][s[1]:s[2]], b[key][s[1]:s[2]]), key
    assert np.array_equal(a["LSE"][:, keep], b["LSE"][:, keep])


def test_group_attended_keys_against_independent_definition():
    groups = [(3, [2, 0, 1]), (0, [4]), (5, [2])]
    for t in range(group_starts(groups)[-1]):
        assert list(attended_keys_groups(t, groups)) == _groups_attended(t, groups)


# ------------------------------------------------- multi-level prefix trees --
from oracle import attended_keys_tree, oracle_tree_fwd_bwd, segment_starts  # noqa: E402


def _tree_attended(t, node_len, node_parent):
    """A(t) written out independently: walk the segments to find row t's, then
    list the keys of every ancestor (root first) and its own up to t."""
    start = 0
    for v, n in enumerate(node_len):
        if start <= t < start + n:
            break
        start += n
    else:
        raise IndexError(t)
    starts = [sum(node_len[:i]) for i in range(len(node_len))]
    chain = []
    a = node_parent[v]
    while a != -1:
        chain.insert(0, a)
        a = node_parent[a]
    keys = []
    for a in chain:
        keys += list(range(starts[a], starts[a] + node_len[a]))
    return keys + list(range(starts[v], t + 1))


TREE_CASES = [
    # (node_len, node_parent, Hq, Hkv, d): depth-first order
    ([4, 3, 2, 0, 3, 5, 2, 3], [-1, 0, 1, 1, 0, -1, 5, 5], 4, 2, 8),
    ([3, 2, 2, 1, 4], [-1, 0, 1, 2, 0], 2, 1, 4),   # a chain of four levels and a sibling
]


def _tree_mask_reference(q, k, v, do, node_len, node_parent, scale):
    T = sum(node_len)
    groups_like = None  # noqa: F841
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    M = torch.zeros(T, T, dtype=torch.bool)
    for t in range(T):
        M[t, _tree_attended(t, node_len, node_parent)] = True
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    O = torch.zeros(T, Hq, q.shape[2], dtype=torch.float64)
    LSE = torch.zeros(Hq, T, dtype=torch.float64)
    for h in range(Hq):
        S = (scale * (qt[:, h] @ kt[:, h // G].T)).masked_fill(~M, float("-inf"))
        LSE[h] = torch.logsumexp(S, dim=1)
        O[:, h] = torch.softmax(S, dim=1) @ vt[:, h // G]
    (O * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return {"O": O.detach().numpy(), "LSE": LSE.detach().numpy(), "dQ": qt.grad.numpy(),
            "dK": kt.grad.numpy(), "dV": vt.grad.numpy()}


@pytest.mark.parametrize("case", range(len(TREE_CASES)))
def test_tree_oracle_matches_dense_masked_attention(case):
    node_len, node_parent, Hq, Hkv, d = TREE_CASES[case]
    T = segment_starts(node_len)[-1]
    rng = np.random.default_rng(70 + case)
    q, do = rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hq, d))
    k, v = rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hkv, d))
    got = oracle_tree_fwd_bwd(q, k, v, do, node_len, node_parent, 0.6)
    ref = _tree_mask_reference(q, k, v, do, node_len, node_parent, 0.6)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.max(np.abs(got[key] - ref[key])) <= 1e-10, key


def test_one_level_tree_is_the_single_group_oracle():
    P, L = 6, [3, 0, 5]
    inp = make_inputs(P, L, 4, 2, 8, seed=71)
    q, k, v, do = _inputs_np(inp)
    a = oracle_tree_fwd_bwd(q, k, v, do, [P] + L, [-1] + [0] * len(L), inp.scale)
    b = oracle_fwd_bwd(q, k, v, do, P, L, inp.scale)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.max(np.abs(a[key] - b[key])) <= 1e-12, key


def test_tree_attended_keys_against_independent_definition():
    for node_len, node_parent, *_ in TREE_CASES:
        for t in range(sum(node_len)):
            assert list(attended_keys_tree(t, node_len, node_parent)) == _tree_attended(t, node_len, node_parent)
