#!/usr/bin/env python3
"""Forward + backward throughput of packed shared-prompt attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = dualkv_fwd + dualkv_bwd (all of its phases) over the packed batch
[prompt P][N responses], inputs resident in HBM before the timed region.
Prints one JSON line on stdout (progress goes to stderr):

* value: useful TFLOP/s, 14 d Hq pairs per step (pairs = attended (query, key)
  pairs under the packed mask; masked tile waste and recomputation excluded)
  divided by the measured time per step;
* roofline: the dominant kernel (largest share of the step) timed with HIP
  events on the launch stream, its algorithmic FLOPs per launch against the
  MI355X dense bf16 MFMA peak; traffic from committed rocprofv3 counters when
  they were taken on the current kernel source, else null;
* replicated: the same kernels on the unshared layout (P = 0, N sequences of
  P + R_n tokens) and the packed speed-up over it;
* cpu_baseline: the float64 CPU oracle timed on a bounded sample of the same
  workload on the host's cores, scaled to the whole workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "fwd+bwd useful TFLOP/s and % bf16 MFMA peak at P=8K,R=4K,N=32"
PROFILES = os.path.join(ROOT, "profiles")
# a kernel's code depends on its source, the shared headers and the build's
# compiler options
_FRAG = ["exact_shared_prefix_amd/csrc/common.h", "exact_shared_prefix_amd/csrc/frag.h",
         "exact_shared_prefix_amd/build.py"]
KERNEL_SOURCES = {
    "dkv_kernel": ["exact_shared_prefix_amd/csrc/bwd.hip"] + _FRAG,
    "dq_kernel": ["exact_shared_prefix_amd/csrc/bwd.hip"] + _FRAG,
    "fwd_kernel": ["exact_shared_prefix_amd/csrc/fwd.hip"] + _FRAG,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, if they were taken on the current source of the kernel."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None, "no counters committed"
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_digest(kernel):
        return None, "kernel changed since the counters were taken"
    return float(rec["hbm_bytes_per_launch"]), os.path.relpath(path, ROOT)


def replicated_inputs(q, k, v, do, P, lengths):
    import torch
    offs = [P]
    for r in lengths:
        offs.append(offs[-1] + r)
    idx = torch.cat([torch.cat([torch.arange(0, P), torch.arange(offs[n], offs[n + 1])])
                     for n in range(len(lengths))]).to(q.device)
    return (q.index_select(0, idx), k.index_select(0, idx), v.index_select(0, idx),
            do.index_select(0, idx), [P + r for r in lengths])


def time_steps(q, k, v, do, pk, scale, steps, warmup, phase_events=True, deterministic=False,
               queued=False):
    """Run warmup + timed fwd+bwd steps; returns timings in ms. queued: hold
    the GPU in a spin kernel while the host enqueues all timed steps, so the
    timed region is the GPU's own execution with no wait for the host."""
    import torch
    from exact_shared_prefix_amd import binding
    dev = q.device
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((Hq, pk.T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsf = torch.empty(binding.fwd_workspace_bytes(pk, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    wsb = torch.empty(binding.bwd_workspace_bytes(pk, Hq, Hkv, d, deterministic), dtype=torch.uint8,
                      device=dev)
    stream = torch.cuda.current_stream()

    phases = (binding.PHASE_PRE, binding.PHASE_MAIN, binding.PHASE_DQ, binding.PHASE_FINISH)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        binding.fwd(q, k, v, pk, scale, out=o, lse=lse, workspace=wsf)
        for i, ph in enumerate(phases):
            if ev:
                ev[i + 1].record(stream)
            binding.bwd(q, k, v, o, lse, do, pk, scale, dq, dk, dv, workspace=wsb,
                        deterministic=deterministic, phases=ph)
        if ev:
            ev[5].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if queued:
        torch.cuda._sleep(int(2e8))   # ~0.1 s of spinning: longer than enqueueing the steps
    t_all0.record(stream)
    for i in range(steps):
        step(evs[i] if phase_events else None)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3
    total = t_all0.elapsed_time(t_all1)
    res = {"ms_per_step": total / steps, "wall_ms_per_step": wall / steps}
    if phase_events:
        def avg(a, b):
            return sum(e[a].elapsed_time(e[b]) for e in evs) / steps
        per = sorted(e[0].elapsed_time(e[5]) for e in evs)
        res.update(min_ms_per_step=per[0], median_ms_per_step=per[len(per) // 2])
        res.update(fwd_ms=avg(0, 1), bwd_pre_ms=avg(1, 2), bwd_dkv_ms=avg(2, 3),
                   bwd_dq_ms=avg(3, 4), bwd_finish_ms=avg(4, 5), bwd_ms=avg(1, 5))
    del o, lse, dq, dk, dv, wsf, wsb
    return res


def cpu_baseline(inp, budget_s: float) -> dict:
    """The float64 oracle on a bounded sample: whole replicated sequences
    (prompt + response n) for single query heads, fwd + bwd, until about
    budget_s of CPU work; scaled by pair counts to the whole workload."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from exact_shared_prefix_amd import metrics
    from oracle.replicated import causal_attention_bwd, causal_attention_fwd

    cores = len(os.sched_getaffinity(0))
    P, L = inp.P, inp.lengths
    offs = [P]
    for r in L:
        offs.append(offs[-1] + r)
    G = inp.Hq // inp.Hkv
    done_pairs, t_used, samples = 0, 0.0, []
    with threadpool_limits(cores):
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
        order = [(n, h) for h in range(inp.Hq) for n in range(len(L))]
        for n, h in order:
            a, b = offs[n], offs[n + 1]
            sl = np.r_[0:P, a:b]
            qh = inp.q[sl, h].float().numpy().astype(np.float64)
            kh = inp.k[sl, h // G].float().numpy().astype(np.float64)
            vh = inp.v[sl, h // G].float().numpy().astype(np.float64)
            dh = inp.do[sl, h].float().numpy().astype(np.float64)
            t0 = time.perf_counter()
            causal_attention_fwd(qh, kh, vh, inp.scale)
            causal_attention_bwd(qh, kh, vh, dh, inp.scale)
            t_used += time.perf_counter() - t0
            Ln = P + (b - a)
            done_pairs += Ln * (Ln + 1) // 2
            samples.append((n, h, Ln))
            if t_used >= budget_s:
                break
    total_pairs = metrics.replicated_pairs(P, L) * inp.Hq
    est_s = t_used * total_pairs / done_pairs
    useful = metrics.useful_flops(P, L, inp.Hq, inp.d)["total"]
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next(ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {
        "value": useful / est_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(samples)} replicated sequence(s) x query head (first: response "
                   f"{samples[0][0]}, head {samples[0][1]}, {samples[0][2]} tokens), textbook "
                   f"float64 fwd+bwd in {t_used:.1f} s; whole workload extrapolated by replicated "
                   f"pair count ({est_s:.0f} s)"),
        "cpu_model": model,
        "seconds_measured": t_used,
        "seconds_extrapolated": est_s,
    }


def calibrate_copy(nbytes: int) -> None:
    """A plain copy kernel of known size (copy_kernel), for scaling the HBM
    byte counters taken on the attention kernels."""
    import torch
    from exact_shared_prefix_amd import microbench
    torch.cuda.set_device(0)
    print(json.dumps(microbench.copy(nbytes)))


def group_main(args, name: str) -> int:
    """Several prompt groups per call (dualkv_fwd_groups / dualkv_bwd_groups):
    the same JSON line for a multi-group workload. The group entry points have
    no per-phase split, so the roofline is taken over the whole fwd+bwd step on
    its useful FLOPs (14 d per pair and query head), with the executed ones
    (18 d: the dQ pass recomputes S and dP) beside them."""
    import torch

    from exact_shared_prefix_amd import binding, metrics
    from exact_shared_prefix_amd.inputs import GROUP_WORKLOADS, group_workload_inputs

    w = GROUP_WORKLOADS[name]
    log(f"[bench] workload {name}: generating seeded inputs")
    inp = group_workload_inputs(w)
    groups = w.groups
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.empty(1, device=dev)
    torch.cuda.reset_peak_memory_stats(dev)
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))

    def run(gp, qq, kk, vv, dd, steps, warmup):
        o = torch.empty_like(qq)
        lse = torch.empty((qq.shape[1], gp.T), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)
        wsf = torch.empty(load_ws(gp, qq, kk, False), dtype=torch.uint8, device=dev)
        wsb = torch.empty(load_ws(gp, qq, kk, True), dtype=torch.uint8, device=dev)
        s = torch.cuda.current_stream()
        for _ in range(warmup):
            binding.fwd_groups(qq, kk, vv, gp, inp.scale, o, lse, wsf)
            binding.bwd_groups(qq, kk, vv, o, lse, dd, gp, inp.scale, dq, dk, dv, wsb)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1, e2 in ev:
            e0.record(s)
            binding.fwd_groups(qq, kk, vv, gp, inp.scale, o, lse, wsf)
            e1.record(s)
            binding.bwd_groups(qq, kk, vv, o, lse, dd, gp, inp.scale, dq, dk, dv, wsb)
            e2.record(s)
        torch.cuda.synchronize()
        f = [a.elapsed_time(b) for a, b, _ in ev]
        t = [a.elapsed_time(c) for a, _, c in ev]
        return {"ms_per_step": sum(t) / steps, "min_ms_per_step": min(t),
                "median_ms_per_step": sorted(t)[steps // 2], "fwd_ms": sum(f) / steps,
                "bwd_ms": (sum(t) - sum(f)) / steps}

    def load_ws(gp, qq, kk, bwd):
        Hq, d, Hkv = qq.shape[1], qq.shape[2], kk.shape[1]
        lib = binding.load()
        if bwd:
            return lib.dualkv_bwd_workspace_bytes_groups(*gp.args(), Hq, Hkv, d, 0)
        return lib.dualkv_fwd_workspace_bytes_groups(*gp.args(), Hq, Hkv, d)

    gp = binding.GroupPacking(groups)
    log(f"[bench] {w.B} groups, T={gp.T}: {args.warmup} warmup + {args.steps} timed steps")
    t = run(gp, q, k, v, do, args.steps, args.warmup)
    peak = torch.cuda.max_memory_allocated(dev)
    pairs = sum(metrics.pairs(P, L) for P, L in groups)
    useful = 14 * inp.d * inp.Hq * pairs
    executed = 18 * inp.d * inp.Hq * pairs
    ms = t["ms_per_step"]
    value = useful / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.2f} ms/step, {value:.1f} useful TFLOP/s (fwd {t['fwd_ms']:.2f} ms, bwd {t['bwd_ms']:.2f} ms)")
    rep = None
    if not args.no_replicated:
        # the same kernels on the unshared layout: every sequence carries its own prompt copy
        rlen = [P + r for P, L in groups for r in L]
        idx = torch.cat([torch.cat([torch.arange(s0, s0 + P), torch.arange(o0, o0 + r)])
                         for (P, L), s0 in zip(groups, _group_starts(groups))
                         for o0, r in zip(_resp_offsets(P, L, s0), L)]).to(dev)
        rq, rk, rv, rd = (x.index_select(0, idx) for x in (q, k, v, do))
        del q, k, v, do
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        rgp = binding.GroupPacking([(0, rlen)])
        log(f"[bench] replicated layout T={rgp.T}")
        rt = run(rgp, rq, rk, rv, rd, max(2, args.steps // 2), 1)
        rpeak = torch.cuda.max_memory_allocated(dev)
        rep = {"ms_per_step": rt["ms_per_step"], "speedup_packed_over_replicated": rt["ms_per_step"] / ms,
               "tokens": rgp.T, "peak_hbm_gb": rpeak / 1e9}
        log(f"[bench] replicated: {rt['ms_per_step']:.2f} ms/step -> packed speed-up {rt['ms_per_step'] / ms:.2f}x")
    line = {
        "metric": "fwd+bwd useful TFLOP/s and % bf16 MFMA peak, several prompt groups per call",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic: seeded i.i.d. normal bf16 q/k/v/dO",
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "config": {"workload": name, "groups": w.B, "P": w.P, "N": w.N, "R": w.R, "Hq": inp.Hq,
                   "Hkv": inp.Hkv, "head_dim": inp.d, "packed_tokens": gp.T, "pairs_per_head": pairs,
                   "useful_tflop_per_step": useful / 1e12, "parallelism": "single GPU"},
        "timing_ms": {kk: round(vv, 4) for kk, vv in t.items()},
        "roofline": {"bound": "mfma", "kernel": "fwd+bwd step (all kernels)",
                     "achieved": useful / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "traffic": None,
                     "traffic_source": "no counters for this workload",
                     "algorithmic_flop_per_step": useful, "executed_flop_per_step": executed,
                     "executed_tflops": executed / (ms * 1e-3) / 1e12},
        "peak_hbm_gb": peak / 1e9, "replicated": rep, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def _group_starts(groups):
    s, out = 0, []
    for P, L in groups:
        out.append(s)
        s += P + sum(L)
    return out


def _resp_offsets(P, L, start):
    o, out = start + P, []
    for r in L:
        out.append(o)
        o += r
    return out


SWEEP_P = (1024, 4096, 16384)
SWEEP_R = (256, 1024, 4096)
SWEEP_N = (1, 2, 4, 8, 16, 32)


def sweep_main(args) -> int:
    """N / P / R sweep (Qwen3-8B heads): packed fwd+bwd time against the same
    kernels on the replicated layout, the token compression
    rho = N(P+R)/(P+NR) and the pair ratio, one JSON line per point and a
    Markdown table on stderr. Where the packed layout stops paying off is
    the row where the speed-up approaches 1. Each packed point is also timed
    with its launches queued behind a spin kernel: the gap between the two
    times is the host's share (argument checks, work lists, launches)."""
    import torch

    from exact_shared_prefix_amd import binding, metrics
    from exact_shared_prefix_amd.inputs import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Hq, Hkv, d = 32, 8, 128
    rows = []
    steps, warmup = max(2, args.steps // 3), 1
    for P in (args.sweep_p or SWEEP_P):
        for R in SWEEP_R:
            for N in SWEEP_N:
                L = [R] * N
                inp = make_inputs(P, L, Hq, Hkv, d, seed=7)
                q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
                t = time_steps(q, k, v, do, binding.Packing(P, L), inp.scale, steps, warmup, False)
                tq = time_steps(q, k, v, do, binding.Packing(P, L), inp.scale, steps, 0, False, queued=True)
                rq, rk, rv, rd, rlen = replicated_inputs(q, k, v, do, P, L)
                del q, k, v, do
                rt = time_steps(rq, rk, rv, rd, binding.Packing(0, rlen), inp.scale, steps, warmup, False)
                del rq, rk, rv, rd
                torch.cuda.empty_cache()
                packed_tok, rep_tok = metrics.tokens(P, L)
                pairs = metrics.pairs(P, L)
                rec = {"P": P, "R": R, "N": N, "packed_ms": t["ms_per_step"],
                       "packed_gpu_ms": tq["ms_per_step"], "host_share": 1 - tq["ms_per_step"] / t["ms_per_step"],
                       "replicated_ms": rt["ms_per_step"],
                       "speedup": rt["ms_per_step"] / t["ms_per_step"], "rho_tokens": rep_tok / packed_tok,
                       "pair_ratio": metrics.replicated_pairs(P, L) / pairs,
                       "useful_tflops": 14 * d * Hq * pairs / (t["ms_per_step"] * 1e-3) / 1e12}
                rows.append(rec)
                print(json.dumps(rec), flush=True)
                log(f"[sweep] P={P} R={R} N={N}: packed {t['ms_per_step']:.2f} ms, replicated "
                    f"{rt['ms_per_step']:.2f} ms, speed-up {rec['speedup']:.2f}x (pairs ratio {rec['pair_ratio']:.2f})")
    log("| P | R | N | packed ms | packed ms, launches queued | replicated ms | speed-up | pair ratio | "
        "token ratio rho | useful TFLOP/s |")
    log("|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        log(f"| {r['P']} | {r['R']} | {r['N']} | {r['packed_ms']:.2f} | {r['packed_gpu_ms']:.2f} | "
            f"{r['replicated_ms']:.2f} | {r['speedup']:.2f} | {r['pair_ratio']:.2f} | {r['rho_tokens']:.2f} | "
            f"{r['useful_tflops']:.0f} |")
    return 0


def layer_main(args) -> int:
    """One packed decoder layer (Qwen3-8B shapes, random weights) at the
    headline packing: fwd+bwd time on the P + sum(R) packed tokens against the
    same layer on the N(P+R) replicated tokens; the ratio is the whole-layer
    speed-up, to compare with the token ratio rho = N(P+R)/(P+NR)."""
    import torch

    from exact_shared_prefix_amd import binding, metrics
    from exact_shared_prefix_amd.inputs import HEADLINE, WORKLOADS, response_lengths
    from exact_shared_prefix_amd.layer import LayerConfig, init_weights, layer_forward, packed_positions

    w = WORKLOADS[args.workload or HEADLINE]
    P, L = w.P, response_lengths(w)
    cfg = LayerConfig(Hq=w.Hq, Hkv=w.Hkv, d=w.d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    weights = {k: t.requires_grad_(True) for k, t in init_weights(cfg, 8, dev).items()}

    def run(pk, pos, steps, warmup):
        g = torch.Generator(device=dev).manual_seed(9)
        x = torch.randn(pk.T, cfg.hidden, device=dev, generator=g).to(torch.bfloat16).requires_grad_(True)
        dy = torch.randn(pk.T, cfg.hidden, device=dev, generator=g).to(torch.bfloat16)
        pos = pos.to(dev)
        for _ in range(warmup):
            layer_forward(x, weights, cfg, pk, pos).backward(dy)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            layer_forward(x, weights, cfg, pk, pos).backward(dy)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, torch.cuda.max_memory_allocated(dev)

    steps, warmup = max(2, args.steps // 3), 1
    pk = binding.Packing(P, L)
    log(f"[layer] {w.name}: packed layer, T={pk.T}")
    ms_p, mem_p = run(pk, packed_positions(P, L), steps, warmup)
    log(f"[layer] packed: {ms_p:.1f} ms per fwd+bwd")
    rlen = [P + r for r in L]
    rpk = binding.Packing(0, rlen)
    rpos = torch.cat([torch.arange(n) for n in rlen])
    log(f"[layer] replicated layer, T={rpk.T}")
    ms_r, mem_r = run(rpk, rpos, steps, warmup)
    packed_tok, rep_tok = metrics.tokens(P, L)
    rec = {"metric": "decoder layer fwd+bwd time, packed vs replicated tokens", "workload": w.name,
           "layer": {"hidden": cfg.hidden, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "head_dim": cfg.d,
                     "intermediate": cfg.inter},
           "packed_ms": ms_p, "replicated_ms": ms_r, "speedup": ms_r / ms_p,
           "rho_tokens": rep_tok / packed_tok, "packed_tokens": packed_tok, "replicated_tokens": rep_tok,
           "peak_hbm_gb": {"packed": mem_p / 1e9, "replicated": mem_r / 1e9}, "steps": steps,
           "note": "projections and MLP are library GEMMs (bf16); attention is this library's kernels"}
    log(f"[layer] replicated: {ms_r:.1f} ms -> whole-layer speed-up {ms_r / ms_p:.2f}x (token ratio {rec['rho_tokens']:.2f})")
    print(json.dumps(rec), flush=True)
    return 0


def tree_main(args) -> int:
    """Two-level shared prefix: a system prompt of S tokens shared by B prompt
    groups (P tokens each, N responses of R), fwd+bwd through the tree entry
    points (the system prompt stored once), against the same batch as B flat
    groups (each group carrying its own copy of the system prompt) and against
    the fully replicated layout (every sequence carries both prefixes)."""
    import torch

    from exact_shared_prefix_amd import binding
    from exact_shared_prefix_amd.inputs import make_inputs

    S, B, P, N, R = 4096, 4, 2048, 8, 1024
    Hq, Hkv, d = 32, 8, 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps, warmup = max(3, args.steps // 2), 2
    node_len, node_parent = [S], [-1]
    for _ in range(B):
        node_parent.append(0)
        node_len.append(P)
        g = len(node_len) - 1
        node_len += [R] * N
        node_parent += [g] * N

    def timed(T, fwd, bwd):
        inp = make_inputs(0, [T], Hq, Hkv, d, seed=10)
        q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
        torch.cuda.reset_peak_memory_stats(dev)
        s = torch.cuda.current_stream()
        for _ in range(warmup):
            o, lse = fwd(q, k, v)
            bwd(q, k, v, o, lse, do)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            o, lse = fwd(q, k, v)
            bwd(q, k, v, o, lse, do)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, torch.cuda.max_memory_allocated(dev)

    tp = binding.TreePacking(node_len, node_parent)
    log(f"[tree] system prompt {S} + {B} x (prompt {P} + {N} x {R}): T={tp.T}")
    ms_t, mem_t = timed(tp.T, lambda q, k, v: binding.fwd_tree(q, k, v, tp),
                        lambda q, k, v, o, lse, do: binding.bwd_tree(q, k, v, o, lse, do, tp))
    gp = binding.GroupPacking([(S + P, [R] * N)] * B)
    ms_g, mem_g = timed(gp.T, lambda q, k, v: binding.fwd_groups(q, k, v, gp),
                        lambda q, k, v, o, lse, do: binding.bwd_groups(q, k, v, o, lse, do, gp))
    rp = binding.Packing(0, [S + P + R] * (B * N))
    ms_r, mem_r = timed(rp.T, lambda q, k, v: binding.fwd(q, k, v, rp),
                        lambda q, k, v, o, lse, do: binding.bwd(q, k, v, o, lse, do, rp))
    from exact_shared_prefix_amd import metrics
    useful = 14 * d * Hq * metrics.tree_pairs(node_len, node_parent)
    rec = {"metric": "two-level shared prefix: fwd+bwd ms, tree vs flat groups vs replicated",
           "useful_tflops": useful / (ms_t * 1e-3) / 1e12,
           "frac_of_peak": useful / (ms_t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "config": {"system_prompt": S, "groups": B, "P": P, "N": N, "R": R, "Hq": Hq, "Hkv": Hkv,
                      "head_dim": d},
           "tree": {"tokens": tp.T, "ms": ms_t, "peak_hbm_gb": mem_t / 1e9},
           "flat_groups": {"tokens": gp.T, "ms": ms_g, "peak_hbm_gb": mem_g / 1e9},
           "replicated": {"tokens": rp.T, "ms": ms_r, "peak_hbm_gb": mem_r / 1e9},
           "speedup_tree_over_groups": ms_g / ms_t, "speedup_tree_over_replicated": ms_r / ms_t,
           "steps": steps}
    log(f"[tree] tree {ms_t:.2f} ms, flat groups {ms_g:.2f} ms, replicated {ms_r:.2f} ms")
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-replicated", action="store_true", help="skip the unshared-layout run")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-mfma-peak", action="store_true", help="skip the measured MFMA peak")
    ap.add_argument("--no-deterministic", action="store_true",
                    help="skip the deterministic-mode (two-pass prompt dK/dV reduction) timing")
    ap.add_argument("--layer", action="store_true",
                    help="one packed decoder layer (random weights) vs the replicated layout")
    ap.add_argument("--tree", action="store_true",
                    help="two-level shared prefix (system prompt + prompt groups) vs flat groups")
    ap.add_argument("--sweep", action="store_true",
                    help="N/P/R sweep of packed vs replicated time (one JSON line per point)")
    ap.add_argument("--sweep-p", type=int, nargs="*", default=None, metavar="P",
                    help="restrict the sweep to these prompt lengths")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return 0

    import torch

    from exact_shared_prefix_amd import binding, metrics
    from exact_shared_prefix_amd.inputs import GROUP_WORKLOADS, HEADLINE, WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.load()
    if args.sweep:
        return sweep_main(args)
    if args.layer:
        return layer_main(args)
    if args.tree:
        return tree_main(args)
    name = args.workload or HEADLINE
    if name in GROUP_WORKLOADS:
        return group_main(args, name)
    w = WORKLOADS[name]
    log(f"[bench] workload {name}: generating seeded inputs")
    inp = workload_inputs(w)
    P, L = inp.P, inp.lengths
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.empty(1, device=dev)  # initialise the caching allocator before resetting its stats
    torch.cuda.reset_peak_memory_stats(dev)
    q, k, v, do = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
    pk = binding.Packing(P, L)
    flops = metrics.useful_flops(P, L, inp.Hq, inp.d)
    pairs = metrics.pairs(P, L)

    log(f"[bench] packed T={inp.T}: {args.warmup} warmup + {args.steps} timed steps")
    packed = time_steps(q, k, v, do, pk, inp.scale, args.steps, args.warmup)
    torch.cuda.synchronize()
    peak_packed = torch.cuda.max_memory_allocated(dev)
    ms = packed["ms_per_step"]
    value = flops["total"] / (ms * 1e-3) / 1e12
    log(f"[bench] packed: {ms:.2f} ms/step, {value:.1f} useful TFLOP/s "
        f"(fwd {packed['fwd_ms']:.2f} ms, bwd {packed['bwd_ms']:.2f} ms: dK/dV {packed['bwd_dkv_ms']:.2f} ms, "
        f"dQ {packed['bwd_dq_ms']:.2f} ms)")

    kflops = metrics.kernel_flops(P, L, inp.Hq, inp.d)
    kuseful = metrics.kernel_useful_flops(P, L, inp.Hq, inp.d)
    kms = {"fwd_kernel": packed["fwd_ms"], "dkv_kernel": packed["bwd_dkv_ms"],
           "dq_kernel": packed["bwd_dq_ms"]}
    dom = max(kms, key=lambda n: kms[n])
    # the dominant kernel's work is all useful (the backward's S, dP, dV, dK)
    ach = kuseful[dom] / (kms[dom] * 1e-3) / 1e12
    traffic, traffic_src = stored_traffic(dom, name)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic,
                "traffic_source": traffic_src,
                "algorithmic_flop_per_launch": kuseful[dom],
                "executed_flop_per_launch": kflops[dom],
                "avg_launch_ms": kms[dom]}
    # per kernel: the useful part of its work and everything it executes
    # (they differ only for the dQ pass, which recomputes S and dP)
    other = {n: {"ms": kms[n], "useful_tflop": kuseful[n] / 1e12, "executed_tflop": kflops[n] / 1e12,
                 "useful_tflops": kuseful[n] / (kms[n] * 1e-3) / 1e12,
                 "executed_tflops": kflops[n] / (kms[n] * 1e-3) / 1e12}
             for n in kms}

    deterministic = None
    if not args.no_deterministic:
        # the same step with the prompt dK/dV summed by the ordered two-pass
        # reduction (per-item partials, then reduce_kernel) instead of atomics
        dsteps = max(2, args.steps // 3)
        log(f"[bench] deterministic mode: 1 warmup + {dsteps} timed steps")
        det = time_steps(q, k, v, do, pk, inp.scale, dsteps, 1, deterministic=True)
        nws = binding.bwd_workspace_bytes(pk, inp.Hq, inp.Hkv, inp.d, True)
        deterministic = {"ms_per_step": det["ms_per_step"],
                         "bwd_dkv_ms": det["bwd_dkv_ms"], "bwd_reduce_ms": det["bwd_finish_ms"],
                         "bwd_workspace_gb": nws / 1e9,
                         "slowdown_vs_atomic": det["ms_per_step"] / ms}
        log(f"[bench] deterministic: {det['ms_per_step']:.2f} ms/step (ordered reduction "
            f"{det['bwd_finish_ms']:.2f} ms, workspace {nws / 1e9:.2f} GB)")
        torch.cuda.empty_cache()

    replicated = None
    if not args.no_replicated:
        del q, k, v, do
        torch.cuda.empty_cache()
        qh, kh, vh, dh = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.do))
        rq, rk, rv, rd, rlen = replicated_inputs(qh, kh, vh, dh, P, L)
        del qh, kh, vh, dh
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        rsteps = max(2, args.steps // 2)
        log(f"[bench] replicated layout T={rq.shape[0]}: 1 warmup + {rsteps} timed steps")
        try:
            rep = time_steps(rq, rk, rv, rd, binding.Packing(0, rlen), inp.scale, rsteps, 1,
                             phase_events=False)
            rflops = metrics.useful_flops(0, rlen, inp.Hq, inp.d)["total"]
            replicated = {"ms_per_step": rep["ms_per_step"],
                          "tflops_on_own_pairs": rflops / (rep["ms_per_step"] * 1e-3) / 1e12,
                          "speedup_packed_over_replicated": rep["ms_per_step"] / ms,
                          "tokens": int(rq.shape[0]),
                          "peak_hbm_gb": torch.cuda.max_memory_allocated(dev) / 1e9}
            log(f"[bench] replicated: {rep['ms_per_step']:.2f} ms/step -> packed speed-up "
                f"{replicated['speedup_packed_over_replicated']:.2f}x")
        except torch.cuda.OutOfMemoryError:
            replicated = {"status": "out of memory"}
        del rq, rk, rv, rd

    cpu = None
    if not args.no_cpu:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(inp, args.cpu_seconds)
        log(f"[bench] CPU oracle: {cpu['value']:.4g} TFLOP/s on {cpu['cores']} threads")

    mfma_peak = None
    if not args.no_mfma_peak:
        from exact_shared_prefix_amd import microbench
        meas = microbench.mfma_tflops()
        mfma_peak = {"measured_tflops": meas, "unit": "TFLOP/s",
                     "kernel": "mfma_rate_kernel / mfma_rate8_kernel (register operands, every CU)",
                     "value_frac_of_measured": value / meas,
                     "dominant_kernel_frac_of_measured": ach / meas}
        log(f"[bench] measured bf16 MFMA peak {meas:.0f} TFLOP/s")

    packed_tok, rep_tok = metrics.tokens(P, L)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. normal bf16 q/k/v/dO",
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "config": {"workload": name, "P": P, "N": len(L),
                   "R": L[0] if len(set(L)) == 1 else "ragged", "lengths_sum": sum(L),
                   "Hq": inp.Hq, "Hkv": inp.Hkv, "head_dim": inp.d,
                   "packed_tokens": packed_tok, "replicated_tokens": rep_tok,
                   "pairs_per_head": pairs, "useful_tflop_per_step": flops["total"] / 1e12,
                   "parallelism": "single GPU"},
        "timing_ms": {kk: round(vv, 4) for kk, vv in packed.items()},
        "kernels": other,
        "roofline": roofline,
        "peak_hbm_gb": peak_packed / 1e9,
        "mfma_peak": mfma_peak,
        "deterministic": deterministic,
        "replicated": replicated,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
