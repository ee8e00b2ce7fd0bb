"""Throughput of the TokenGate gated-prefill hot path on one MI355X.

One step = one pass of the whole path over one prompt (batch 1):
    tg_gate_score -> tg_select_topk -> tg_compact -> tg_rope_qk -> tg_gated_attention
at the Qwen3-1.7B-shaped gate layer: d_model 2048, scorer 2048->256->1,
N = 16384 tokens (last 64 forced-keep), K = 2048 kept, 16 q / 8 kv heads,
head_dim 128, one upper layer of token-gated attention.  Inputs are seeded
synthetic tensors already resident in HBM; the residual is rotated over six
copies (384 MB > the 256 MB MALL) so the scorer reads it from HBM.

Prints one JSON line.  `value` = N / (ms_per_step) in tokens/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-prefill tokens/s at N=16k Qwen3-1.7B shape; attn MFMA % of bf16 peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
N_RESID_COPIES = 6


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="n16k",
                   choices=["n16k", "n32k-k1024", "n32k-k4096", "n32k-k8192", "n128k", "full16k", "tiny"])
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--no-attn-sweep", action="store_true", help="skip the attention-only K sweep")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the whole-prompt comparison (28 decoder layers, full against gated)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def workload(name):
    from learned_token_pruning_mlp_amd import synth
    base = synth.QWEN3_1P7B_N16K
    if name == "n16k":
        return base, "qwen3-1.7b gate layer, N=16384, F=64, K=2048, 1 upper layer"
    if name.startswith("n32k"):
        k = int(name.split("k")[-1])
        shp = synth.GateShape(**{**base.__dict__, "n": 32768, "k": k})
        return shp, f"qwen3-1.7b gate layer, N=32768, F=64, K={k}, 1 upper layer"
    if name == "n128k":
        return synth.QWEN3_1P7B_N128K, "qwen3-1.7b gate layer, N=131072, F=128, K=8192, 1 upper layer"
    if name == "full16k":
        shp = synth.GateShape(**{**base.__dict__, "k": base.n})
        return shp, "qwen3-1.7b gate layer, N=16384, K=N (no pruning), 1 upper layer"
    return synth.TINY, "tiny gate layer, N=512, d=256, K=128"


def attn_flops(shp):
    return 4.0 * shp.hq * shp.head_dim * shp.k * (shp.k + 1) / 2.0


def gate_bytes(shp):
    # residual read once, W1 once, b1/w2 tiny, raw + normalised scores written/read
    return shp.n * shp.d * 2 + shp.hd * shp.d * 2 + shp.n * 4 * 3


def compact_bytes(shp):
    # kept residual rows read + written, index, position and score per kept row
    return shp.k * (shp.d * 2 * 2 + 4 * 4)


def source_sha(name):
    path = os.path.join(ROOT, "learned_token_pruning_mlp_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel_file, workload_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(workload_name, {}).get(kernel_file)
        if not ent or ent.get("source_sha") != source_sha(kernel_file):
            return None
        return ent["hbm_bytes_per_launch"]
    except Exception:
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X "
              "(see the sharding notes in the design document); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from learned_token_pruning_mlp_amd import binding as tg
    from learned_token_pruning_mlp_amd import synth

    tg.load()
    dev = torch.device("cuda:0")
    shp, desc = workload(args.workload)
    seed = 2

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs, resident in HBM before timing
    inp = synth.gate_inputs(shp, seed)
    resid = [bf(inp.resid)]
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    for _ in range(N_RESID_COPIES - 1):
        resid.append(torch.randn(resid[0].shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16))
    w1, w2 = bf(inp.w1), bf(inp.w2)
    forced = torch.from_numpy(inp.forced).to(dev)
    pos = torch.from_numpy(inp.pos).to(dev)
    n, k = shp.n, shp.k
    a = synth.attn_inputs(k, shp.hq, shp.hkv, shp.head_dim, seed)
    q, kk, vv = bf(a.q), bf(a.k), bf(a.v)
    gains = torch.from_numpy(a.gains).to(dev)
    # outputs and workspace
    s_norm = torch.empty(n, dtype=torch.float32, device=dev)
    ws = tg.workspace(n, dev)
    kept = torch.empty(k, dtype=torch.int32, device=dev)
    resid_k = torch.empty((k, shp.d), dtype=torch.bfloat16, device=dev)
    pos_k = torch.empty(k, dtype=torch.int32, device=dev)
    score_k = torch.empty(k, dtype=torch.float32, device=dev)
    out = torch.empty((k, shp.hq, shp.head_dim), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    stages = ["gate_score", "select_topk", "compact", "rope", "gated_attention"]

    def mark(ev, j):
        if ev is not None and ev[j] is not None:
            ev[j].record(stream)

    def step(i, ev=None):
        r = resid[i % N_RESID_COPIES]
        mark(ev, 0)
        tg.tg_gate_score(r, w1, None, w2, 0.0, 1e-6, 1e-6, s_norm, None, ws)
        mark(ev, 1)
        tg.tg_select_topk(s_norm, forced, shp.n_forced, k, kept, None, ws)
        mark(ev, 2)
        tg.tg_compact(kept, n, r, resid_k, pos, pos_k, s_norm, score_k)
        mark(ev, 3)
        tg.tg_rope_qk(q, kk, pos_k, shp.rope_theta)
        mark(ev, 4)
        tg.tg_gated_attention(q, kk, vv, score_k, gains, shp.temp_coef, pos_k, out)
        mark(ev, 5)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- per-stage breakdown (outside the timed region): events between all launches
    n_diag = max(1, min(20, args.steps))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_diag)]
    for i in range(n_diag):
        step(i, evs[i])
    torch.cuda.synchronize()
    per_stage = {s: 0.0 for s in stages}
    for e in evs:
        for j, s in enumerate(stages):
            per_stage[s] += e[j].elapsed_time(e[j + 1])
    per_stage = {s: v / n_diag for s, v in per_stage.items()}  # ms per step
    dom = max(per_stage, key=per_stage.get)
    dom_j = stages.index(dom)

    # ---- timed region: exactly `steps` steps, synchronised on both sides.  Only
    # the dominant stage is bracketed by events (on the stream its kernel runs
    # on), and only on every `ev_stride`-th step: each event record adds a
    # barrier packet and a timestamp to the queue (about 2.5 us per step for
    # the pair), which is instrumentation, not work of the path.
    ev_stride = max(1, args.steps // 25)
    ev_steps = list(range(0, args.steps, ev_stride))
    dom_ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in ev_steps}

    def timed_step(i):
        marks = [None] * 6
        if i in dom_ev:
            marks[dom_j], marks[dom_j + 1] = dom_ev[i]
        step(i, marks)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        timed_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    dom_ms = sum(a.elapsed_time(b) for a, b in dom_ev.values()) / len(dom_ev)

    # ---- roofline of the dominant kernel, timed inside the timed region
    if dom == "gated_attention":
        achieved = attn_flops(shp) / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": "gated_attn", "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic_for("k_attn.hip", args.workload)}
    elif dom == "gate_score":
        achieved = gate_bytes(shp) / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": "gate_mlp+gate_seqnorm", "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": traffic_for("k_gate.hip", args.workload)}
    else:
        achieved = compact_bytes(shp) / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    roof["launch_us"] = dom_ms * 1e3
    roof["timed_launches"] = len(dom_ev)
    per_stage[dom] = dom_ms
    attn_tflops = attn_flops(shp) / (per_stage["gated_attention"] * 1e-3) / 1e12
    gate_gbs = gate_bytes(shp) / (per_stage["gate_score"] * 1e-3) / 1e9
    event_ms = sum(per_stage.values())

    if args.copy_probe_mib:
        # counter calibration: one elementwise kernel that reads and writes exactly
        # copy_probe_mib MiB (float32 multiply into a separate buffer)
        src = torch.ones((args.copy_probe_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    sweep = None if args.no_attn_sweep else attn_sweep(tg, torch, dev, shp)
    prefill = None if (args.no_prefill or args.workload != "n16k") else prefill_compare(tg, torch, dev, shp, seed)
    backward = None if (args.no_attn_sweep or args.workload != "n16k") else \
        {"attention": attn_backward(tg, torch, dev, shp), "scorer": gate_backward(tg, torch, dev, shp)}
    hybrid = None if (args.no_attn_sweep or args.workload != "n16k") else hybrid_mixer(tg, torch, dev, shp)

    result = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init scorer weights, N(0,1) residual and q/k/v)",
        "config": {"workload": desc, "n_tokens": n, "kept": k, "forced": shp.n_forced, "d_model": shp.d,
                   "scorer_hidden": shp.hd, "q_heads": shp.hq, "kv_heads": shp.hkv, "head_dim": shp.head_dim,
                   "batch": 1},
        "attn_mfma_pct": 100.0 * attn_tflops / PEAK_BF16_TFLOPS,
        "stage_us": {s: round(v * 1e3, 3) for s, v in per_stage.items()},
        "stage_event_sum_ms": event_ms,
        "attn_tflops": attn_tflops,
        "gate_hbm_gbs": gate_gbs,
        "roofline": roof,
        "attn_sweep": sweep,
        "prefill": prefill,
        "backward": backward,
        "hybrid_mixer": hybrid,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shp, seed, inp, a)
    print(json.dumps(result), flush=True)


def prefill_compare(tg, torch, dev, shp, seed, n_layers=28, gate_layer=1, reps=3):
    """One prompt through a Qwen3-1.7B-shaped decoder stack (synthetic weights), both ways:
    full prefill (every layer on all N tokens, plain causal attention) and gated
    prefill (layer 0 and the gate layer's attention block on N tokens; scorer,
    top-K, compaction of the residual and of the lower layers' K/V; the gate
    layer's MLP and the 26 layers above on the K kept tokens, token-gated
    attention).  Returns wall times per prompt (ms), timed with HIP events on
    the stream, after one untimed run of each."""
    from learned_token_pruning_mlp_amd import synth, upper

    s = upper.QWEN3_1P7B_LAYER
    assert s.d == shp.d and s.hq == shp.hq and s.hkv == shp.hkv and s.head_dim == shp.head_dim
    inp = synth.gate_inputs(shp, seed)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    gains = (torch.rand(n_layers, shp.hq, generator=g, device=dev) * 1.5 + 0.5).float()
    pf = upper.Prefill(s, shp.n, n_layers, gate_layer, bf(inp.w1), bf(inp.w2), gains, shp.temp_coef, dev, seed)
    h = bf(inp.resid)
    forced = torch.from_numpy(inp.forced).to(dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    full_ms = timed(lambda: pf.full(h))
    gated_ms = timed(lambda: pf.gated(h, forced, shp.n_forced, shp.k))
    # the same gated prefill captured once as a HIP graph and replayed
    graph, _ = pf.capture_gated(h, forced, shp.n_forced, shp.k)
    graph_ms = timed(graph.replay)
    del graph
    pf.blas.close()
    del pf
    torch.cuda.empty_cache()

    # algorithmic FLOPs: projections 2 * rows * in * out, causal attention 4 hq D R(R+1)/2
    D, qd, kvd = s.head_dim, s.hq * s.head_dim, s.hkv * s.head_dim

    def attn_part(r):
        return 2 * r * s.d * (qd + 2 * kvd) + 2 * r * qd * s.d + 4 * s.hq * D * r * (r + 1) / 2

    def mlp_part(r):
        return 2 * r * s.d * 2 * s.inter + 2 * r * s.inter * s.d

    n, k = shp.n, shp.k
    full_flop = n_layers * (attn_part(n) + mlp_part(n))
    gated_flop = (gate_layer * (attn_part(n) + mlp_part(n)) + attn_part(n) + 2 * n * shp.d * shp.hd
                  + mlp_part(k) + (n_layers - gate_layer - 1) * (attn_part(k) + mlp_part(k)))
    return {"layers": n_layers, "gate_layer": gate_layer, "n_tokens": n, "kept": k,
            "full_ms": round(full_ms, 3), "gated_ms": round(gated_ms, 3), "speedup": round(full_ms / gated_ms, 2),
            "gated_graph_ms": round(graph_ms, 3),
            "full_tflops": round(full_flop / (full_ms * 1e-3) / 1e12, 1),
            "gated_tflops": round(gated_flop / (gated_ms * 1e-3) / 1e12, 1),
            "weights": "synthetic, one set per layer", "reps": reps}


def attn_backward(tg, torch, dev, shp, ks=(2048, 8192), reps=5):
    """tg_gated_attention_bwd alone (it recomputes the forward inside) at the
    Qwen3-1.7B head shape; algorithmic work 2.5x the forward's (five products
    of 2 D FLOP per visible (query, key) pair and head)."""
    out = {}
    for k in ks:
        g = torch.Generator(device=dev)
        g.manual_seed(k)
        bf = lambda *s: torch.randn(*s, generator=g, device=dev).to(torch.bfloat16)  # noqa: E731
        q, kk, vv, do = bf(k, shp.hq, shp.head_dim), bf(k, shp.hkv, shp.head_dim), bf(k, shp.hkv, shp.head_dim), \
            bf(k, shp.hq, shp.head_dim)
        ks_ = torch.randn(k, generator=g, device=dev)
        gains = torch.rand(shp.hq, generator=g, device=dev) + 0.5
        pos = torch.arange(k, dtype=torch.int32, device=dev) * 4
        f32 = dict(dtype=torch.float32, device=dev)
        o = [torch.empty(k, shp.hq, shp.head_dim, **f32), torch.empty(k, shp.hkv, shp.head_dim, **f32),
             torch.empty(k, shp.hkv, shp.head_dim, **f32), torch.empty(k, **f32), torch.empty(shp.hq, **f32),
             torch.empty(1, **f32)]
        ws = torch.empty(tg.tg_attention_bwd_workspace_bytes(k, shp.hq, shp.hkv, shp.head_dim), dtype=torch.uint8,
                         device=dev)

        def run():
            tg.tg_gated_attention_bwd(q, kk, vv, ks_, gains, 0.1, pos, do, *o, ws=ws)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flop = 2.5 * 4 * shp.hq * shp.head_dim * k * (k + 1) / 2
        out[str(k)] = {"us": round(us, 1), "tflops": round(flop / us / 1e6, 1),
                       "frac": round(flop / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    return out


def gate_backward(tg, torch, dev, shape, reps=5):
    """tg_gate_score_bwd at the gate layer's shape: three GEMMs of 2 n d hd
    FLOP each (z again, dz W1, dz^T h); algorithmic bytes = the residual read
    once (bf16) + its gradient written (fp32)."""
    n, d, hd, k = shape.n, shape.d, shape.hd, shape.k
    g = torch.Generator(device=dev)
    g.manual_seed(n)
    resid = torch.randn(n, d, generator=g, device=dev).to(torch.bfloat16)
    w1 = (torch.randn(hd, d, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(hd, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    s_raw = torch.randn(n, generator=g, device=dev)
    kept = torch.randperm(n, generator=g, device=dev)[:k].sort().values.to(torch.int32)
    dsk = torch.randn(k, generator=g, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = [torch.empty(n, d, **f32), torch.empty(hd, d, **f32), torch.empty(hd, **f32), torch.empty(hd, **f32),
           torch.empty(1, **f32)]
    ws = torch.empty(tg.tg_gate_score_bwd_workspace_bytes(n, d, hd), dtype=torch.uint8, device=dev)
    blas = tg.BlasHandle()
    try:
        def run():
            tg.tg_gate_score_bwd(blas, resid, w1, None, w2, 1e-6, 1e-6, s_raw, dsk, kept, *out, ws=ws)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
    finally:
        blas.close()
    flop = 3 * 2.0 * n * d * hd
    byts = n * d * 2 + n * d * 4
    return {"n": n, "us": round(us, 1), "tflops": round(flop / us / 1e6, 1),
            "mfma_frac": round(flop / us / 1e6 / PEAK_BF16_TFLOPS, 4), "hbm_gbs": round(byts / us / 1e3, 1),
            "hbm_frac": round(byts / us / 1e3 / PEAK_HBM_GBS, 4)}


def hybrid_mixer(tg, torch, dev, shape, reps=5):
    """tg_gated_delta_rule with 16 heads of 128 x 128 state over the kept
    tokens (K) and over the whole prompt (N): what pruning saves in an upper
    recurrent layer of the hybrid backbone."""
    heads, dk = 16, 128
    res = {}
    for name, t in (("kept", shape.k), ("full", shape.n)):
        g = torch.Generator(device=dev)
        g.manual_seed(t)
        qk = torch.nn.functional.normalize(torch.randn(2, t, heads, dk, generator=g, device=dev), dim=-1)
        q, k = qk[0].to(torch.bfloat16), qk[1].to(torch.bfloat16)
        v = torch.randn(t, heads, dk, generator=g, device=dev).to(torch.bfloat16)
        alpha = 0.9 + 0.1 * torch.rand(t, heads, generator=g, device=dev)
        beta = torch.rand(t, heads, generator=g, device=dev)
        out = torch.empty(t, heads, dk, dtype=torch.float32, device=dev)
        tg.tg_gated_delta_rule(q, k, v, alpha, beta, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            tg.tg_gated_delta_rule(q, k, v, alpha, beta, out)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[name] = {"tokens": t, "us": round(us, 1), "ns_per_token": round(us * 1e3 / t, 1)}
    res["speedup"] = round(res["full"]["us"] / res["kept"]["us"], 2)
    return res


def attn_sweep(tg, torch, dev, shp, ks=(4096, 8192, 16384), reps=10):
    """Gated attention alone at longer kept lists (same heads and head_dim):
    TFLOP/s of algorithmic causal work and the fraction of the bf16 peak.
    Timing-only inputs: N(0,1) q/k/v and scores, positions 4t."""
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for k in ks:
        q = torch.randn((k, shp.hq, shp.head_dim), generator=g, device=dev).to(torch.bfloat16)
        kk = torch.randn((k, shp.hkv, shp.head_dim), generator=g, device=dev).to(torch.bfloat16)
        vv = torch.randn((k, shp.hkv, shp.head_dim), generator=g, device=dev).to(torch.bfloat16)
        ks_ = torch.randn(k, generator=g, device=dev)
        gains = torch.rand(shp.hq, generator=g, device=dev) * 1.5 + 0.5
        pos = torch.arange(k, dtype=torch.int32, device=dev) * 4
        out = torch.empty_like(q)
        stream = torch.cuda.current_stream()

        def run():
            tg.tg_gated_attention(q, kk, vv, ks_, gains, shp.temp_coef, pos, out)

        for _ in range(2):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flops = 4.0 * shp.hq * shp.head_dim * k * (k + 1) / 2.0
        tf = flops / (us * 1e-6) / 1e12
        res[str(k)] = {"us": round(us, 2), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del q, kk, vv, out
    return res


def cpu_baseline(shp, seed, inp, a):
    """The fp64 oracle, as it stands, over one full step of the same workload."""
    from oracle import oracle
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    s_norm, _ = oracle.gate_score(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, nthreads=threads)
    kept = oracle.select_topk(s_norm, inp.forced, shp.k)
    oracle.gather_rows(inp.resid, kept)
    qr = oracle.rope(a.q, kept, shp.rope_theta)
    kr = oracle.rope(a.k, kept, shp.rope_theta)
    oracle.gated_attention(qr, kr, a.v, s_norm[kept], a.gains, shp.temp_coef, kept, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": shp.n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one full step of the same workload (N={shp.n}, K={shp.k}), fp64, {dt:.2f} s"}


if __name__ == "__main__":
    main()
