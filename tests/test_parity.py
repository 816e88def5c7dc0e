"""GPU parity: the HIP forward/backward against the CPU float64 oracle.

Bar (from the arithmetic: bf16 inputs/outputs, bf16 MFMA operands for P and
dS, fp32 accumulation): per tensor ||X_gpu - X_ref||_F / ||X_ref||_F <= 1e-2
for O, dQ, dK, dV (also per region, prompt vs response rows/keys, so a bad
prompt reduction cannot hide), and max |LSE_gpu - LSE_ref| <= 1e-3.
Where the reference is exactly zero (scale 0; constant V) an absolute bound
is used instead.

* small cases: every element, against the literal replicated oracle;
* full workload sizes, in the launch configuration the benchmark times:
  sampled rows (O, LSE, dQ; every head) and response keys (dK, dV) evaluated
  live by the packed-definition oracle, prompt keys against stored oracle
  values (tests/golden, tied to the inputs by sha256), and sum rules that
  hold at any size.
"""
import os
import sys

import numpy as np
import pytest
import torch

from exact_shared_prefix_amd import binding
from exact_shared_prefix_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from oracle import (group_starts, keys_dkdv, oracle_fwd_bwd, oracle_groups_fwd_bwd, oracle_tree_fwd_bwd,
                    rows_fwd_bwd)

pytestmark = pytest.mark.gpu

REL = 1e-2
LSE_ABS = 1e-3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(inp, deterministic=False):
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
    pk = binding.Packing(inp.P, inp.lengths)
    o, lse = binding.fwd(q, k, v, pk, inp.scale)
    dq, dk, dv = binding.bwd(q, k, v, o, lse, do, pk, inp.scale, deterministic=deterministic)
    torch.cuda.synchronize()
    out = {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}
    res = {kk: t.float().cpu().numpy() for kk, t in out.items()}
    del q, k, v, do, o, lse, dq, dk, dv, out
    torch.cuda.empty_cache()
    return res


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def np64(t):
    return t.float().numpy().astype(np.float64)


def check_all(got, ref, P, tag):
    for key in ("O", "dQ", "dK", "dV"):
        e = rel(got[key], ref[key])
        ep = rel(got[key][:P], ref[key][:P]) if P else 0.0
        er = rel(got[key][P:], ref[key][P:]) if got[key].shape[0] > P else 0.0
        say(f"  {tag} {key}: rel {e:.2e} (prompt {ep:.2e}, response {er:.2e})")
        assert e <= REL and ep <= REL and er <= REL, (tag, key, e, ep, er)
    dl = float(np.max(np.abs(got["LSE"] - ref["LSE"])))
    say(f"  {tag} LSE: max abs {dl:.2e}")
    assert dl <= LSE_ABS
    for key, x in got.items():
        assert np.all(np.isfinite(x)), key


SMALL = {
    "ragged_tails_p300": dict(P=300, lengths=[129, 1, 0, 64, 250], Hq=4, Hkv=2, d=128, seed=21),
    "no_prompt_p0": dict(P=0, lengths=[200, 77], Hq=2, Hkv=1, d=128, seed=22),
    "single_response_mha_d64": dict(P=256, lengths=[100], Hq=2, Hkv=2, d=64, seed=23),
    "gqa8_p192": dict(P=192, lengths=[65, 128], Hq=8, Hkv=1, d=128, seed=24),
    "prompt_tail_empty_responses": dict(P=129, lengths=[0, 0, 31], Hq=2, Hkv=1, d=128, seed=25),
    "peaked_scores_q_x4": dict(P=160, lengths=[96, 33], Hq=4, Hkv=2, d=128, seed=26, qkv_scale=2.0),
    "ragged_d64_many": dict(P=70, lengths=[1, 2, 3, 130, 64, 65], Hq=4, Hkv=1, d=64, seed=27),
    # small N with a long prompt and short responses (the sweep's crossover regime)
    "small_n2_long_prompt": dict(P=1000, lengths=[37, 64], Hq=4, Hkv=2, d=128, seed=28),
    "n1_prompt_only_response": dict(P=777, lengths=[1], Hq=2, Hkv=1, d=128, seed=29),
    # many tiny responses (0 .. 40 tokens): dozens of short regions, work items and tail masks
    "many_tiny_responses_n40": dict(P=96, lengths=[(7 * i) % 41 for i in range(40)], Hq=8, Hkv=2,
                                    d=128, seed=30),
    # every region boundary on a 256-row / 256-key tile edge
    "tile_aligned_p256_r256": dict(P=256, lengths=[256, 256], Hq=2, Hkv=1, d=128, seed=33),
    # head counts that neither divide nor are multiples of 8: the launch's
    # block -> (item, head) map takes its plain form (no XCD grouping)
    "headmap_plain_h12_kv3_d128": dict(P=300, lengths=[200, 57, 0, 130], Hq=12, Hkv=3, d=128, seed=35),
    "headmap_plain_h12_kv3_d64": dict(P=190, lengths=[70, 260, 1], Hq=12, Hkv=3, d=64, seed=36),
}


def test_tiny_workload_elementwise():
    w = WORKLOADS["tiny_p128_r64_n4_gqa2_d64"]
    inp = workload_inputs(w)
    say(f"case {w.name}: P={inp.P} lengths={inp.lengths}")
    got = run_gpu(inp)
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), inp.P, inp.lengths,
                         inp.scale)
    check_all(got, ref, inp.P, w.name)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_cases_elementwise(name):
    kw = dict(SMALL[name])
    P, lengths, Hq, Hkv, d, seed = (kw.pop(x) for x in ("P", "lengths", "Hq", "Hkv", "d", "seed"))
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=seed, **kw)
    say(f"case {name}: P={P} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d}")
    got = run_gpu(inp)
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, inp.scale)
    check_all(got, ref, P, name)


def test_scale_zero_closed_form():
    P, lengths = 150, [70, 3, 0, 129]
    inp = make_inputs(P, lengths, 4, 2, 128, seed=31, scale=0.0)
    say("case scale0")
    got = run_gpu(inp)
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, 0.0)
    for key in ("O", "dV"):
        assert rel(got[key], ref[key]) <= REL, key
    assert float(np.max(np.abs(got["LSE"] - ref["LSE"]))) <= LSE_ABS
    assert np.all(got["dQ"] == 0.0) and np.all(got["dK"] == 0.0)


def test_constant_v():
    P, lengths = 140, [60, 0, 90]
    inp = make_inputs(P, lengths, 4, 2, 128, seed=32, const_v=True)
    say("case constant V")
    got = run_gpu(inp)
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, inp.scale)
    for key in ("O", "dV"):
        assert rel(got[key], ref[key]) <= REL, key
    # reference dQ and dK vanish: bound them against the size of a typical gradient
    typical = float(np.linalg.norm(np64(inp.do))) * float(np.abs(np64(inp.k)).max()) * inp.scale
    for key in ("dQ", "dK"):
        assert float(np.linalg.norm(got[key])) <= 1e-3 * typical, key


def test_repeat_calls_agree_within_tolerance():
    """Atomic accumulation order may differ between runs; results stay within
    float32 rounding of each other and bitwise-equal in the forward."""
    inp = make_inputs(256, [300, 180], 4, 2, 128, seed=33)
    say("case repeat")
    a = run_gpu(inp)
    b = run_gpu(inp)
    for key in ("O", "LSE"):
        assert np.array_equal(a[key], b[key]), key
    for key in ("dQ", "dK", "dV"):
        assert rel(a[key], b[key]) <= 1e-3, key


def test_backward_phase_by_phase_is_the_whole_backward():
    """The four backward phases run one call at a time on one workspace
    (preprocess; dQ before dK/dV, which are independent; finish) give the
    whole backward's bits (deterministic mode, so dK, dV are ordered)."""
    inp = make_inputs(300, [129, 1, 0, 64, 250], 4, 2, 128, seed=61)
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
    pk = binding.Packing(inp.P, inp.lengths)
    o, lse = binding.fwd(q, k, v, pk, inp.scale)
    whole = binding.bwd(q, k, v, o, lse, do, pk, inp.scale, deterministic=True)
    ws = torch.empty(binding.bwd_workspace_bytes(pk, 4, 2, 128, True), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for ph in (binding.PHASE_PRE, binding.PHASE_DQ, binding.PHASE_MAIN, binding.PHASE_FINISH):
        binding.bwd(q, k, v, o, lse, do, pk, inp.scale, dq, dk, dv, workspace=ws, deterministic=True,
                    phases=ph)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), whole, (dq, dk, dv)):
        assert torch.equal(a, b), name


def test_calls_on_a_side_stream_match_the_current_stream():
    """Forward and backward enqueued on another stream (default priority),
    outputs and workspaces allocated by the binding for that stream, give the
    current stream's bits (deterministic backward)."""
    inp = make_inputs(256, [300, 180, 7], 4, 2, 128, seed=62)
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
    pk = binding.Packing(inp.P, inp.lengths)
    o, lse = binding.fwd(q, k, v, pk, inp.scale)
    ref = binding.bwd(q, k, v, o, lse, do, pk, inp.scale, deterministic=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o2, lse2 = binding.fwd(q, k, v, pk, inp.scale, stream=side)
    got = binding.bwd(q, k, v, o2, lse2, do, pk, inp.scale, deterministic=True, stream=side)
    side.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(a, b), name


def test_noalloc_forward_replays_in_a_captured_graph():
    """The allocation-free forward launches only kernels (its work lists are
    built on the device), so it can be captured in a HIP graph: every replay,
    with eager work of the same library between them, gives the eager result."""
    inp = make_inputs(700, [300, 0, 129, 64], 8, 2, 128, seed=63)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    pk = binding.Packing(inp.P, inp.lengths)
    ref_o, ref_lse = binding.fwd(q, k, v, pk, inp.scale)
    o = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_lse)
    binding.fwd_noalloc(q, k, v, pk, inp.scale, out=o, lse=lse)   # first call: scratch address taken
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.fwd_noalloc(q, k, v, pk, inp.scale, out=o, lse=lse)
    other = make_inputs(300, [100, 50], 8, 2, 128, seed=64)
    oq, ok, ov = (x.to(dev) for x in (other.q, other.k, other.v))
    opk = binding.Packing(other.P, other.lengths)
    for r in range(3):
        o.zero_()
        lse.zero_()
        binding.fwd_noalloc(oq, ok, ov, opk, other.scale)   # eager, same scratch array
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse), r


@pytest.mark.parametrize("name", ["ragged_tails_p300", "ragged_d64_many", "gqa8_p192"])
def test_deterministic_mode_parity_and_bitwise_repeat(name):
    """Deterministic mode: same bar against the oracle, and two calls give
    bitwise-identical dQ, dK, dV."""
    kw = dict(SMALL[name])
    P, lengths, Hq, Hkv, d, seed = (kw.pop(x) for x in ("P", "lengths", "Hq", "Hkv", "d", "seed"))
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=seed, **kw)
    say(f"case deterministic {name}: P={P} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d}")
    a = run_gpu(inp, deterministic=True)
    b = run_gpu(inp, deterministic=True)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[key], b[key]), key
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, inp.scale)
    check_all(a, ref, P, name + " det")


def test_deterministic_mode_bitwise_repeat_multi_chunk():
    """Long enough that prompt tiles span several row chunks (so the ordered
    reduction sums many partials); the atomic result agrees to fp32 rounding."""
    inp = make_inputs(4096, [2500, 3000, 1800], 8, 2, 128, seed=34)
    say("case deterministic multi-chunk: P=4096 lengths=[2500, 3000, 1800]")
    a = run_gpu(inp, deterministic=True)
    b = run_gpu(inp, deterministic=True)
    c = run_gpu(inp, deterministic=False)
    for key in ("dQ", "dK", "dV"):
        assert np.array_equal(a[key], b[key]), key
        assert rel(a[key], c[key]) <= 1e-3, key


# ------------------------------------------------------ random packings --
# Seeded random packings (prompt length, number and lengths of responses,
# empty responses, head counts that are not powers of two, d = 64 / 128,
# input scales, both reduction modes), each compared element-wise with the
# replicated oracle. The shapes come from numpy's generator seeded with the
# case number; they are test parameters, not part of the method.
_HEADS = [(2, 1), (4, 2), (4, 4), (6, 3), (8, 2), (3, 1), (5, 5), (12, 4)]


def _random_case(i):
    rng = np.random.default_rng(1000 + i)
    P = int(rng.integers(0, 601))
    n = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(0, 257, size=n)]
    if P + sum(lengths) == 0:
        lengths[0] = 1
    Hq, Hkv = _HEADS[int(rng.integers(0, len(_HEADS)))]
    d = (64, 128)[int(rng.integers(0, 2))]
    qkv_scale = float((0.5, 1.0, 2.0)[int(rng.integers(0, 3))])
    return dict(P=P, lengths=lengths, Hq=Hq, Hkv=Hkv, d=d, qkv_scale=qkv_scale, seed=2000 + i,
                det=bool(i % 2))


@pytest.mark.parametrize("i", range(16))
def test_random_packings_elementwise(i):
    kw = _random_case(i)
    det = kw.pop("det")
    P, lengths, Hq, Hkv, d, seed = (kw.pop(x) for x in ("P", "lengths", "Hq", "Hkv", "d", "seed"))
    inp = make_inputs(P, lengths, Hq, Hkv, d, seed=seed, **kw)
    say(f"case random {i}: P={P} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d} qkv_scale={inp.meta['qkv_scale']} "
        f"deterministic={det}")
    got = run_gpu(inp, deterministic=det)
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, inp.scale)
    check_all(got, ref, P, f"random {i}")


# ------------------------------------------------ across the row-chunk grid --
# The dK/dV pass cuts every key tile's attending rows into row chunks (2048
# rows; 256 to 1024 for problems too small to fill the chip with 2048-row
# chunks, as these); a prompt key tile's gradient is the sum of the partials of
# all its chunks (fp32 atomics, or the ordered sum of the deterministic mode).
# These cases have T > 4096, so prompt tiles span many chunks, and every
# element is compared with the replicated oracle in both modes.
CHUNKED = {
    "chunks_p4096_gqa4_d128": dict(P=4096, lengths=[2500, 3000, 1800], Hq=8, Hkv=2, d=128, seed=34),
    "chunks_p2400_ragged_d64": dict(P=2400, lengths=[1900, 1500, 700, 3], Hq=2, Hkv=1, d=64, seed=37),
}
_ORACLE_CACHE = {}


def _chunked(name):
    if name not in _ORACLE_CACHE:
        kw = dict(CHUNKED[name])
        P, lengths, Hq, Hkv, d, seed = (kw.pop(x) for x in ("P", "lengths", "Hq", "Hkv", "d", "seed"))
        inp = make_inputs(P, lengths, Hq, Hkv, d, seed=seed)
        say(f"case {name}: oracle for P={P} lengths={lengths} Hq={Hq} Hkv={Hkv} d={d}")
        ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, inp.scale)
        _ORACLE_CACHE[name] = (inp, ref)
    return _ORACLE_CACHE[name]


@pytest.mark.parametrize("det", [False, True])
@pytest.mark.parametrize("name", sorted(CHUNKED))
def test_across_row_chunks_elementwise(name, det):
    inp, ref = _chunked(name)
    assert inp.T > 2 * 2048
    say(f"case {name} deterministic={det}: T={inp.T}")
    got = run_gpu(inp, deterministic=det)
    check_all(got, ref, inp.P, f"{name} det={det}")
    # prompt keys per 256-key tile: every tile's multi-chunk sum on its own
    for t0 in range(0, inp.P, 256):
        t1 = min(inp.P, t0 + 256)
        for key in ("dK", "dV"):
            e = rel(got[key][t0:t1], ref[key][t0:t1])
            assert e <= REL, (key, t0, e)


def _plant_reference_moves(inp, plants):
    """Make chosen rows' scores jump far above their first key tile: for
    (row t, key j, alpha) set k_j = alpha * q_t (query head h = first of the
    KV head's group, every KV head), so row t's score on key j is about
    alpha * |q_t|^2 * scale (tens of log2 units for alpha >= 2, d = 128)."""
    G = inp.Hq // inp.Hkv
    k = inp.k.clone()
    for t, j, alpha in plants:
        for g in range(inp.Hkv):
            k[j, g] = (alpha * inp.q[t, g * G].float()).to(torch.bfloat16)
    inp.k = k
    return inp


def test_forward_reference_moves_elementwise():
    """Rows whose scores rise by 20 to 60 log2 units after their first key
    tile, once or twice along the row (inside the prompt region, at the switch
    to the own-response region, and inside it), plus a key ramp that makes
    later keys larger for every row: the forward must move its reference and
    rescale O and the row sum, and the backward must agree."""
    P, lengths = 400, [300, 200, 90]
    inp = make_inputs(P, lengths, 4, 2, 128, seed=38)
    o = [P] + list(P + np.cumsum(lengths))
    plants = [
        (300, 150, 2.0), (300, 290, 4.0),          # prompt row: two moves, in tiles 2 and 4
        (o[0] + 10, 380, 2.5),                     # response row: late prompt tile
        (o[0] + 250, o[0] + 200, 3.0),             # response row: inside its own region
        (o[1] + 150, 70, 2.0), (o[1] + 150, o[1] + 140, 4.0),
        (o[2] + 89, o[2] + 80, 3.5),
    ]
    _plant_reference_moves(inp, plants)
    c = inp.scale * np.log2(np.e)
    for t, j, _ in plants:
        first = np.max(np64(inp.q)[t, 0] @ np64(inp.k)[:64, 0].T) * c
        jump = float(np64(inp.q)[t, 0] @ np64(inp.k)[j, 0]) * c - first
        say(f"  row {t} key {j}: score {jump:.1f} log2 units above its first tile's max")
        assert jump > 20.0
    # ramp: the last keys of every region are scaled up to 2.5x
    ramp = torch.from_numpy(1.0 + 1.5 * (np.arange(inp.T) / inp.T) ** 2).to(torch.float32)
    inp.k = (inp.k.float() * ramp[:, None, None]).to(torch.bfloat16)
    say(f"case reference moves: P={P} lengths={lengths}")
    got = run_gpu(inp)
    ref = oracle_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), P, lengths, inp.scale)
    check_all(got, ref, P, "reference moves")
    rows = sorted({t for t, _, _ in plants})
    e = rel(got["O"][rows], ref["O"][rows])
    say(f"  planted rows O: rel {e:.2e}")
    assert e <= REL
    assert float(np.max(np.abs(got["LSE"][:, rows] - ref["LSE"][:, rows]))) <= LSE_ABS


# ------------------------------------------------- several prompt groups --
GROUPS = {
    # groups: [(P_b, [R_b0, ...]), ...]
    "three_groups_ragged_d128": dict(groups=[(300, [129, 1, 0, 64]), (0, [200]), (129, [31, 0, 250])],
                                     Hq=4, Hkv=2, d=128, seed=41),
    "four_groups_d64_gqa4": dict(groups=[(64, [64, 64]), (70, [1, 2, 3]), (256, [100]), (5, [300])],
                                 Hq=8, Hkv=2, d=64, seed=42),
}


def run_gpu_groups(inp, groups, deterministic=False):
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
    gp = binding.GroupPacking(groups)
    o, lse = binding.fwd_groups(q, k, v, gp, inp.scale)
    dq, dk, dv = binding.bwd_groups(q, k, v, o, lse, do, gp, inp.scale, deterministic=deterministic)
    torch.cuda.synchronize()
    return {kk: t.float().cpu().numpy() for kk, t in
            {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}.items()}


@pytest.mark.parametrize("name", sorted(GROUPS))
@pytest.mark.parametrize("det", [False, True])
def test_groups_elementwise(name, det):
    c = GROUPS[name]
    groups = c["groups"]
    T = group_starts(groups)[-1]
    inp = make_inputs(0, [T], c["Hq"], c["Hkv"], c["d"], seed=c["seed"])
    say(f"case groups {name} det={det}: {groups}")
    got = run_gpu_groups(inp, groups, det)
    ref = oracle_groups_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), groups, inp.scale)
    s = group_starts(groups)
    for b in range(len(groups)):
        a, e = s[b], s[b + 1]
        for key in ("O", "dQ", "dK", "dV"):
            err = rel(got[key][a:e], ref[key][a:e])
            say(f"  group {b} {key}: rel {err:.2e}")
            assert err <= REL, (b, key)
        assert float(np.max(np.abs(got["LSE"][:, a:e] - ref["LSE"][:, a:e]))) <= LSE_ABS, b
    for key, x in got.items():
        assert np.all(np.isfinite(x)), key


def _random_groups(i):
    rng = np.random.default_rng(3000 + i)
    groups = []
    for _ in range(int(rng.integers(1, 5))):
        P = int(rng.integers(0, 300))
        groups.append((P, [int(x) for x in rng.integers(0, 200, size=int(rng.integers(1, 5)))]))
    if group_starts(groups)[-1] == 0:
        groups[0] = (1, groups[0][1])
    Hq, Hkv = _HEADS[int(rng.integers(0, len(_HEADS)))]
    d = (64, 128)[int(rng.integers(0, 2))]
    return groups, Hq, Hkv, d


@pytest.mark.parametrize("i", range(6))
def test_random_groups_elementwise(i):
    """Seeded random multi-group calls (group counts, prompt and response
    lengths including empty ones, head layouts, d), alternating modes."""
    groups, Hq, Hkv, d = _random_groups(i)
    det = bool(i % 2)
    T = group_starts(groups)[-1]
    inp = make_inputs(0, [T], Hq, Hkv, d, seed=3100 + i)
    say(f"case random groups {i}: {groups} Hq={Hq} Hkv={Hkv} d={d} det={det}")
    got = run_gpu_groups(inp, groups, det)
    ref = oracle_groups_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), groups, inp.scale)
    for key in ("O", "dQ", "dK", "dV"):
        err = rel(got[key], ref[key])
        say(f"  {key}: rel {err:.2e}")
        assert err <= REL, key
    assert float(np.max(np.abs(got["LSE"] - ref["LSE"]))) <= LSE_ABS
    for key, x in got.items():
        assert np.all(np.isfinite(x)), key


def test_one_group_call_is_the_single_group_call():
    """B = 1 through the group entry points gives the single-group entry
    points' bits (deterministic backward, so dK, dV are ordered too)."""
    P, L = 300, [129, 1, 0, 64, 250]
    inp = make_inputs(P, L, 4, 2, 128, seed=43)
    a = run_gpu(inp, deterministic=True)
    b = run_gpu_groups(inp, [(P, L)], deterministic=True)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[key], b[key]), key


# ------------------------------------------------- multi-level prefix trees --
TREES = {
    # depth-first (node_len, node_parent)
    "system_prompt_two_levels": dict(node_len=[200, 150, 64, 0, 97, 90, 33, 128], node_parent=[-1, 0, 1, 1, 1, 0, 5, 5],
                                     Hq=4, Hkv=2, d=128, seed=51),
    "four_levels_d64": dict(node_len=[70, 65, 40, 31, 5, 129], node_parent=[-1, 0, 1, 2, 2, 0],
                            Hq=4, Hkv=1, d=64, seed=52),
    "forest_of_trees": dict(node_len=[64, 32, 16, 100, 7, 300, 1], node_parent=[-1, 0, 1, -1, 3, 3, -1],
                            Hq=8, Hkv=2, d=128, seed=53),
}


def run_gpu_tree(inp, node_len, node_parent, deterministic=False):
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
    tp = binding.TreePacking(node_len, node_parent)
    o, lse = binding.fwd_tree(q, k, v, tp, inp.scale)
    dq, dk, dv = binding.bwd_tree(q, k, v, o, lse, do, tp, inp.scale, deterministic=deterministic)
    torch.cuda.synchronize()
    return {kk: t.float().cpu().numpy() for kk, t in
            {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}.items()}


@pytest.mark.parametrize("name", sorted(TREES))
def test_tree_elementwise(name):
    c = TREES[name]
    T = sum(c["node_len"])
    inp = make_inputs(0, [T], c["Hq"], c["Hkv"], c["d"], seed=c["seed"])
    say(f"case tree {name}: {c['node_len']} {c['node_parent']}")
    got = run_gpu_tree(inp, c["node_len"], c["node_parent"])
    ref = oracle_tree_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), c["node_len"],
                              c["node_parent"], inp.scale)
    for key in ("O", "dQ", "dK", "dV"):
        e = rel(got[key], ref[key])
        say(f"  {key}: rel {e:.2e}")
        assert e <= REL, key
    assert float(np.max(np.abs(got["LSE"] - ref["LSE"]))) <= LSE_ABS
    for key, x in got.items():
        assert np.all(np.isfinite(x)), key


def _random_forest(i):
    """A random prefix forest in depth-first order, at most four levels: each
    new segment hangs below a segment on the current root-to-leaf path (or
    starts a new tree)."""
    rng = np.random.default_rng(4000 + i)
    node_len, node_parent, depth, path = [], [], [], []
    for n in range(int(rng.integers(2, 10))):
        choices = [-1] + [x for x in path if depth[x] < 4]
        par = choices[int(rng.integers(0, len(choices)))] if n else -1
        node_len.append(int(rng.integers(0, 160)) if rng.random() > 0.1 else 0)
        node_parent.append(par)
        depth.append(1 if par < 0 else depth[par] + 1)
        path = ([] if par < 0 else path[:path.index(par) + 1]) + [n]
    if sum(node_len) == 0:
        node_len[0] = 1
    Hq, Hkv = _HEADS[int(rng.integers(0, len(_HEADS)))]
    d = (64, 128)[int(rng.integers(0, 2))]
    return node_len, node_parent, Hq, Hkv, d


@pytest.mark.parametrize("i", range(6))
def test_random_trees_elementwise(i):
    node_len, node_parent, Hq, Hkv, d = _random_forest(i)
    T = sum(node_len)
    inp = make_inputs(0, [T], Hq, Hkv, d, seed=4100 + i)
    say(f"case random tree {i}: {node_len} {node_parent} Hq={Hq} Hkv={Hkv} d={d}")
    got = run_gpu_tree(inp, node_len, node_parent, deterministic=bool(i % 2))
    ref = oracle_tree_fwd_bwd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.do), node_len, node_parent,
                              inp.scale)
    for key in ("O", "dQ", "dK", "dV"):
        e = rel(got[key], ref[key])
        say(f"  {key}: rel {e:.2e}")
        assert e <= REL, key
    assert float(np.max(np.abs(got["LSE"] - ref["LSE"]))) <= LSE_ABS
    for key, x in got.items():
        assert np.all(np.isfinite(x)), key


def test_one_level_tree_call_is_the_single_group_call():
    P, L = 300, [129, 1, 0, 64, 250]
    inp = make_inputs(P, L, 4, 2, 128, seed=54)
    a = run_gpu(inp, deterministic=True)
    b = run_gpu_tree(inp, [P] + L, [-1] + [0] * len(L), deterministic=True)
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[key], b[key]), key


# ----------------------------------------------------------- full sizes --
FULL = ["qwen3_8b_p4k_r4k_n8", "rollout_p8k_r4k_n32", "longprompt_p32k_r2k_n16",
        "ragged_p64k_n16_r256_2048"]


def sample_rows(P, lengths, T, seed):
    o = np.concatenate([[P], P + np.cumsum(lengths)])
    rows = {0, 1, T - 1}
    if P:
        rows |= {P - 1, P // 2, min(P, T - 1)}
    for n in (0, 1, len(lengths) // 2, len(lengths) - 1):
        if lengths[n]:
            rows |= {int(o[n]), int(o[n + 1] - 1), int(o[n] + lengths[n] // 2)}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, T, 12))
    return sorted(r for r in rows if 0 <= r < T)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    say(f"case {name}: generating inputs")
    inp = workload_inputs(w)
    say(f"case {name}: T={inp.T} running fwd+bwd on the GPU")
    got = run_gpu(inp)
    for key, x in got.items():
        assert np.all(np.isfinite(x)), key
    q, k, v, do = (t.float().numpy() for t in (inp.q, inp.k, inp.v, inp.do))
    P, L, T = inp.P, inp.lengths, inp.T

    # 1. sampled rows, every head
    rows = sample_rows(P, L, T, w.seed)
    say(f"case {name}: oracle on {len(rows)} rows")
    ref = rows_fwd_bwd(q, k, v, do, P, L, inp.scale, rows)
    for key in ("O", "dQ"):
        e = rel(got[key][rows], ref[key])
        say(f"  rows {key}: rel {e:.2e}")
        assert e <= REL, key
    dl = float(np.max(np.abs(got["LSE"][:, rows] - ref["LSE"])))
    say(f"  rows LSE: max abs {dl:.2e}")
    assert dl <= LSE_ABS

    # 2. response keys near the end of the first and last responses
    o = np.concatenate([[P], P + np.cumsum(L)])
    for n in sorted({0, len(L) - 1}):
        a, b = int(o[n]), int(o[n + 1])
        keys = list(range(max(a, b - 24), b))
        for g in sorted({0, inp.Hkv - 1}):
            say(f"case {name}: oracle response keys n={n} kv_head={g}")
            rk = keys_dkdv(q, k, v, do, P, L, inp.scale, keys, g)
            for key in ("dK", "dV"):
                e = rel(got[key][keys, g], rk[key])
                say(f"  response {key} n={n} g={g}: rel {e:.2e}")
                assert e <= REL, (key, n, g)

    # 3. prompt keys against stored oracle values (first and last KV head; first
    #    and last keys of 16 key tiles, 32-key block edges, row-chunk edges)
    gpath = os.path.join(GOLDEN, f"prompt_keys_{name}.npz")
    gold = np.load(gpath)
    assert str(gold["digest"]) == inp.digest(), "inputs differ from the ones the goldens were made from"
    keys, heads = [int(x) for x in gold["keys"]], [int(x) for x in gold["kv_heads"]]
    assert len(keys) >= 64 and heads == sorted({0, inp.Hkv - 1})
    for i, g in enumerate(heads):
        for key in ("dK", "dV"):
            e = rel(got[key][keys, g], gold[key][i])
            say(f"  prompt {key} kv_head={g} ({len(keys)} keys, stored): rel {e:.2e}")
            assert e <= REL, (key, g)
            worst = max(rel(got[key][j, g], gold[key][i, n]) for n, j in enumerate(keys))
            say(f"    largest single-key rel error {worst:.2e}")

    # 4. sum rules: sum_j dK_j = 0 and sum_j dV_j = sum_{t, h in group} dO_t,h
    G = inp.Hq // inp.Hkv
    for g in range(inp.Hkv):
        sk = got["dK"][:, g].astype(np.float64).sum(0)
        assert np.linalg.norm(sk) <= REL * np.linalg.norm(got["dK"][:, g]), ("sum dK", g)
        sv = got["dV"][:, g].astype(np.float64).sum(0)
        want = do[:, g * G:(g + 1) * G].astype(np.float64).sum((0, 1))
        assert rel(sv, want) <= REL, ("sum dV", g)


def test_qwen3_heads_elementwise_first_and_last_kv_head():
    """The Qwen3-8B-head workload (P = 4096, N = 8 responses of 4096, Q/K/V x0.5)
    in full for KV heads 0 and 7 and their query heads: every element of O,
    LSE and dQ of those query heads and of dK, dV of those KV heads against the
    replicated oracle (heads are independent, so this is the literal check of
    those heads at full sequence length)."""
    name = "qwen3_8b_p4k_r4k_n8"
    w = WORKLOADS[name]
    inp = workload_inputs(w)
    say(f"case {name}: T={inp.T} running fwd+bwd on the GPU")
    got = run_gpu(inp)
    G = inp.Hq // inp.Hkv
    q, k, v, do = (np64(t) for t in (inp.q, inp.k, inp.v, inp.do))
    for g in sorted({0, inp.Hkv - 1}):
        say(f"case {name}: replicated oracle for kv head {g}")
        ref = oracle_fwd_bwd(q, k, v, do, inp.P, inp.lengths, inp.scale, kv_heads=[g])
        hs = slice(g * G, (g + 1) * G)
        sub = {"O": got["O"][:, hs], "dQ": got["dQ"][:, hs], "dK": got["dK"][:, g], "dV": got["dV"][:, g],
               "LSE": got["LSE"][hs]}
        want = {"O": ref["O"][:, hs], "dQ": ref["dQ"][:, hs], "dK": ref["dK"][:, g], "dV": ref["dV"][:, g],
                "LSE": ref["LSE"][hs]}
        check_all(sub, want, inp.P, f"kv head {g}")


def test_tensors_beyond_2_31_elements_sampled():
    """Q, O, dO, dQ with more than 2^31 elements (64 query heads, 262656
    tokens: 1025 responses of 256 after a 256-token prompt). Rows and keys
    whose element offsets lie past 2^31 are checked against the oracle."""
    P, N, R, Hq, Hkv, d = 256, 1025, 256, 64, 8, 128
    L = [R] * N
    T = P + N * R
    assert T * Hq * d > 2 ** 31
    say(f"case beyond 2^31: generating inputs T={T} Hq={Hq}")
    inp = make_inputs(P, L, Hq, Hkv, d, seed=71)
    say("case beyond 2^31: running fwd+bwd on the GPU")
    got = run_gpu(inp)
    first_past = (2 ** 31) // (Hq * d)   # first row whose elements start past 2^31
    rows = sorted({0, P - 1, P, T // 2, first_past - 1, first_past, first_past + 77, T - R, T - 2, T - 1})
    q, k, v, do = (t.float().numpy() for t in (inp.q, inp.k, inp.v, inp.do))
    say(f"case beyond 2^31: oracle on rows {rows}")
    ref = rows_fwd_bwd(q, k, v, do, P, L, inp.scale, rows)
    for key in ("O", "dQ"):
        e = rel(got[key][rows], ref[key])
        say(f"  rows {key}: rel {e:.2e}")
        assert e <= REL, key
    assert float(np.max(np.abs(got["LSE"][:, rows] - ref["LSE"]))) <= LSE_ABS
    keys = list(range(T - R, T - R + 8)) + list(range(T - 8, T))   # last response: its rows lie past 2^31
    for g in (0, Hkv - 1):
        rk = keys_dkdv(q, k, v, do, P, L, inp.scale, keys, g)
        for key in ("dK", "dV"):
            e = rel(got[key][keys, g], rk[key])
            say(f"  last-response {key} g={g}: rel {e:.2e}")
            assert e <= REL, (key, g)

