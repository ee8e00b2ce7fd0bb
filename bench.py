"""Throughput of the TokenGate gated-prefill hot path on one MI355X.

One step = one pass of the whole path over one prompt (batch 1):
    tg_gate_score -> tg_select_topk -> tg_compact -> (tg_rope_qk -> tg_gated_attention) per upper layer
Default workload (n16k): the Qwen3-1.7B-shaped gate layer, d_model 2048,
scorer 2048->256->1, N = 16384 tokens (last 64 forced-keep), K = 2048 kept,
16 q / 8 kv heads, head_dim 128, one upper layer of token-gated attention.
--workload selects the other sizes: N = 32768 with K = 1024 / 4096 / 8192
(Student-t scores into select), N = 131072 with K = 8192 over 26 upper
layers (and the lower layers' K/V trimmed by the compaction), and K = N.
Inputs are seeded synthetic tensors already resident in HBM; the residual is
rotated over copies whose total exceeds the 256 MB MALL, so the scorer reads
it from HBM.

Prints one JSON line.  `value` = N / ms_per_step in tokens/s, where
ms_per_step is the wall time of exactly --steps steps over their count.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-prefill tokens/s at N=16k Qwen3-1.7B shape; attn MFMA % of bf16 peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="n16k", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--no-attn-sweep", action="store_true",
                   help="skip the attention-only K sweep, the backward passes and the recurrent mixer")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the whole-prompt comparison (28 decoder layers, full against gated)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


# name -> (shape factory, description, upper layers, Student-t scores for select/compact/attention)
def _shape(n, k, n_forced=64, layout="tail"):
    from learned_token_pruning_mlp_amd import synth
    base = synth.QWEN3_1P7B_N16K
    return synth.GateShape(**{**base.__dict__, "n": n, "k": k, "n_forced": n_forced, "forced_layout": layout})


WORKLOADS = {
    "tiny": (lambda: __import__("learned_token_pruning_mlp_amd.synth", fromlist=["TINY"]).TINY,
             "tiny gate layer, N=512, d=256, F=32, K=128, 1 upper layer", 1, False),
    "n16k": (lambda: _shape(16384, 2048),
             "qwen3-1.7b gate layer, N=16384, F=64, K=2048, 1 upper layer", 1, False),
    "n32k-k1024": (lambda: _shape(32768, 1024),
                   "qwen3-1.7b gate layer, N=32768, F=64, K=1024, 1 upper layer, Student-t(3) scores", 1, True),
    "n32k-k4096": (lambda: _shape(32768, 4096),
                   "qwen3-1.7b gate layer, N=32768, F=64, K=4096, 1 upper layer, Student-t(3) scores", 1, True),
    "n32k-k8192": (lambda: _shape(32768, 8192),
                   "qwen3-1.7b gate layer, N=32768, F=64, K=8192, 1 upper layer, Student-t(3) scores", 1, True),
    "n128k": (lambda: _shape(131072, 8192, 128, "scatter_tail"),
              "qwen3-1.7b gate layer, N=131072, F=128 scattered over the last 1024, K=8192, 26 upper layers of "
              "kept-row K/V, 2 lower layers' K/V trimmed", 26, False),
    "full16k": (lambda: _shape(16384, 16384),
                "qwen3-1.7b gate layer, N=16384, F=64, K=N (no pruning), 1 upper layer", 1, False),
}
N_LOWER_KV_LAYERS = 2   # layers below the gate whose full-length K/V the n128k step trims
EV_STRIDE = 6           # the dominant kernel is bracketed by events on every 6th timed step,
EV_OFFSET = 3           # starting with the 4th (the first step after the synchronisation is left out)


def attn_flops(shp):
    return 4.0 * shp.hq * shp.head_dim * shp.k * (shp.k + 1) / 2.0


def gate_bytes(shp):
    # residual read once, W1 once, raw scores written and read back, normalised scores written
    return shp.n * shp.d * 2 + shp.hd * shp.d * 2 + shp.n * 4 * 3


def compact_bytes(shp, extra_row_bytes=0):
    # kept residual rows read + written, index read, position and score read + written,
    # plus each extra stream's kept rows read + written
    return shp.k * (shp.d * 2 * 2 + 4 * 5 + 2 * extra_row_bytes)


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


class Path:
    """Inputs resident in HBM and one step of the whole path over them:
    tg_gate_score -> tg_select_topk -> tg_compact -> (tg_rope_qk ->
    tg_gated_attention) for each upper layer."""

    STAGES = ["gate_score", "select_topk", "compact", "rope", "gated_attention"]

    def __init__(self, tg, torch, dev, name, seed):
        from learned_token_pruning_mlp_amd import synth
        make, self.desc, self.layers, t_scores = WORKLOADS[name]
        self.shp = shp = make()
        self.name, self.tg, self.torch = name, tg, torch
        self.inp = inp = synth.gate_inputs(shp, seed)
        bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        # the residual rotates over copies whose total exceeds the 256 MB MALL,
        # so the scorer reads it from HBM on every step
        copies = max(2, min(6, -(-(384 << 20) // (shp.n * shp.d * 2))))
        self.resid = [bf(inp.resid)] + [torch.randn((shp.n, shp.d), generator=g, device=dev).to(torch.bfloat16)
                                        for _ in range(copies - 1)]
        self.w1, self.w2 = bf(inp.w1), bf(inp.w2)
        self.forced = torch.from_numpy(inp.forced).to(dev)
        self.pos = torch.from_numpy(inp.pos).to(dev)
        n, k = shp.n, shp.k
        f32 = dict(dtype=torch.float32, device=dev)
        self.s_norm = torch.empty(n, **f32)
        # Student-t(3) scores drawn directly for select, compaction and attention
        self.t_scores = torch.from_numpy(synth.student_t_scores(n, seed)).to(dev) if t_scores else None
        self.ws = tg.workspace(n, dev)
        self.kept = torch.empty(k, dtype=torch.int32, device=dev)
        self.resid_k = torch.empty((k, shp.d), dtype=torch.bfloat16, device=dev)
        self.pos_k = torch.empty(k, dtype=torch.int32, device=dev)
        self.score_k = torch.empty(k, **f32)
        self.a = a = synth.attn_inputs(k, shp.hq, shp.hkv, shp.head_dim, seed)
        self.gains = torch.from_numpy(a.gains).to(dev)
        L = self.layers
        if L == 1:
            self.q, self.kk, self.vv = [bf(a.q)], [bf(a.k)], [bf(a.v)]
        else:
            # per upper layer: its q and its kept-row K/V, stacked [L, K, Hkv, D]
            self.q = [torch.randn((k, shp.hq, shp.head_dim), generator=g, device=dev).to(torch.bfloat16)
                      for _ in range(L)]
            kv = [torch.randn((L, k, shp.hkv, shp.head_dim), generator=g, device=dev).to(torch.bfloat16)
                  for _ in range(2)]
            self.kk, self.vv = list(kv[0]), list(kv[1])
        self.extra = []
        if name == "n128k":
            # the lower layers' full-length K and V, trimmed to the kept rows
            for _ in range(2 * N_LOWER_KV_LAYERS):
                src = torch.randn((n, shp.hkv, shp.head_dim), generator=g, device=dev).to(torch.bfloat16)
                self.extra.append((src, torch.empty((k, shp.hkv, shp.head_dim), dtype=torch.bfloat16, device=dev)))
        self.out = torch.empty((k, shp.hq, shp.head_dim), dtype=torch.bfloat16, device=dev)
        self.stream = torch.cuda.current_stream()

    def extra_row_bytes(self):
        return sum(s[0].numel() * s.element_size() for s, _ in self.extra)

    def step(self, i, ev=None, attn_ev=None):
        """One pass of the path.  ev: optional list of 6 events (or None
        entries) recorded between the stages; the rope / attention marks go
        around the first upper layer's launches.  attn_ev: optional pair of
        events that the first upper layer's attention launch records at the
        kernel's own start and end (tg_gated_attention_timed)."""
        tg, shp = self.tg, self.shp

        def mark(j):
            if ev is not None and ev[j] is not None:
                ev[j].record(self.stream)
        r = self.resid[i % len(self.resid)]
        sc = self.s_norm if self.t_scores is None else self.t_scores
        # scorer and select in one call (the sequence norm inside the select
        # up to 16384 tokens), unless they select on drawn scores or a mark
        # between them is asked for (the per-stage pass)
        fused = self.t_scores is None and (ev is None or (ev[1] is None and ev[2] is None))
        mark(0)
        if fused:
            tg.tg_gate_score_select(r, self.w1, None, self.w2, 0.0, 1e-6, 1e-6, self.forced, shp.n_forced, shp.k,
                                    self.s_norm, None, self.kept, None, self.ws)
        else:
            tg.tg_gate_score(r, self.w1, None, self.w2, 0.0, 1e-6, 1e-6, self.s_norm, None, self.ws)
            mark(1)
            tg.tg_select_topk(sc, self.forced, shp.n_forced, shp.k, self.kept, None, self.ws)
        mark(2)
        tg.tg_compact(self.kept, shp.n, r, self.resid_k, self.pos, self.pos_k, sc, self.score_k, extra=self.extra)
        mark(3)
        for L in range(self.layers):
            tg.tg_rope_qk(self.q[L], self.kk[L], self.pos_k, shp.rope_theta)
            if L == 0:
                mark(4)
            if L == 0 and attn_ev is not None:
                tg.tg_gated_attention_timed(self.q[L], self.kk[L], self.vv[L], self.score_k, self.gains,
                                            shp.temp_coef, self.pos_k, self.out, attn_ev[0], attn_ev[1])
            else:
                tg.tg_gated_attention(self.q[L], self.kk[L], self.vv[L], self.score_k, self.gains, shp.temp_coef,
                                      self.pos_k, self.out)
            if L == 0:
                mark(5)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X "
              "(see the sharding notes in the design document); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from learned_token_pruning_mlp_amd import binding as tg

    tg.load()
    dev = torch.device("cuda:0")
    seed = 2
    path = Path(tg, torch, dev, args.workload, seed)
    shp, stream, stages = path.shp, path.stream, Path.STAGES
    n, k = shp.n, shp.k
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    for i in range(args.warmup):
        path.step(i)
    torch.cuda.synchronize()

    # ---- per-stage breakdown and per-step times, outside the timed region:
    # events between all launches of a step (stage times, first upper layer
    # for rope and attention), then steps bracketed one by one (median step)
    n_diag = max(5, min(20, args.steps))
    evs = [[Ev() for _ in range(6)] for _ in range(n_diag)]
    for i in range(n_diag):
        path.step(i, evs[i])
    torch.cuda.synchronize()
    per_stage = {s: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / n_diag for j, s in enumerate(stages)}
    dom = max(per_stage, key=per_stage.get)
    dom_j = stages.index(dom)
    bounds = [Ev() for _ in range(n_diag + 1)]
    bounds[0].record(stream)
    for i in range(n_diag):
        path.step(i)
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(n_diag))
    median_step_ms = step_ms[n_diag // 2] if n_diag % 2 else 0.5 * (step_ms[n_diag // 2 - 1] + step_ms[n_diag // 2])

    # ---- timed region: exactly `steps` steps, synchronised on both sides.
    # Only the dominant stage's first launch is timed, on every EV_STRIDE-th
    # step whatever the step count.  Attention records a pair of events at
    # its kernel's own start and end (tg_gated_attention_timed, on the stream
    # the kernel runs on); another dominant stage is bracketed by events
    # recorded around its call, which also take in the dispatch gap before
    # the kernel starts.  Each timed launch adds queue work (timestamps),
    # which is instrumentation, not work of the path.
    ev_steps = list(range(min(EV_OFFSET, args.steps - 1), args.steps, EV_STRIDE))
    dom_ev = {i: (Ev(), Ev()) for i in ev_steps}
    kernel_events = dom == "gated_attention"
    if kernel_events:
        for a, b in dom_ev.values():  # torch creates an event's handle at its first record
            a.record(stream)
            b.record(stream)

    def timed_step(i):
        if i not in dom_ev:
            path.step(i)
        elif kernel_events:
            path.step(i, attn_ev=dom_ev[i])
        else:
            marks = [None] * 6
            marks[dom_j], marks[dom_j + 1] = dom_ev[i]
            path.step(i, marks)

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
        achieved = compact_bytes(shp, path.extra_row_bytes()) / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    roof["launch_us"] = dom_ms * 1e3
    roof["timed_launches"] = len(dom_ev)
    roof["timing"] = ("events recorded at the kernel's start and end (extended launch)" if kernel_events
                      else "events recorded around the call (dispatch gap included)")
    attn_tflops = attn_flops(shp) / (per_stage["gated_attention"] * 1e-3) / 1e12
    gate_gbs = gate_bytes(shp) / (per_stage["gate_score"] * 1e-3) / 1e9
    compact_gbs = compact_bytes(shp, path.extra_row_bytes()) / (per_stage["compact"] * 1e-3) / 1e9

    if args.copy_probe_mib:
        # counter calibration: one elementwise kernel that reads and writes exactly
        # copy_probe_mib MiB (float32 multiply into a separate buffer)
        src = torch.ones((args.copy_probe_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    headline = args.workload == "n16k"
    sweep = None if (args.no_attn_sweep or not headline) else attn_sweep(tg, torch, dev, shp)
    prefill = None if (args.no_prefill or not headline) else prefill_compare(tg, torch, dev, shp, seed)
    backward = None if (args.no_attn_sweep or not headline) else \
        {"attention": attn_backward(tg, torch, dev, shp), "scorer": gate_backward(tg, torch, dev, shp)}
    hybrid = None if (args.no_attn_sweep or not headline) else hybrid_mixer(tg, torch, dev, shp)

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
        "config": {"workload": path.desc, "n_tokens": n, "kept": k, "forced": shp.n_forced, "d_model": shp.d,
                   "scorer_hidden": shp.hd, "q_heads": shp.hq, "kv_heads": shp.hkv, "head_dim": shp.head_dim,
                   "upper_layers": path.layers, "batch": 1},
        "median_step_ms": median_step_ms,
        "attn_mfma_pct": 100.0 * attn_tflops / PEAK_BF16_TFLOPS,
        "stage_us": {s: round(v * 1e3, 3) for s, v in per_stage.items()},
        # the per-stage pass calls the scorer and the select separately; the
        # timed and median steps call them as one tg_gate_score_select
        # (unless the select takes drawn scores)
        "stage_calls": "separate" if path.t_scores is not None else "separate in stage_us; fused when timed",
        "stage_event_sum_ms": sum(per_stage.values()),
        "attn_tflops": attn_tflops,
        "gate_hbm_gbs": gate_gbs,
        "compact_hbm_gbs": compact_gbs,
        "roofline": roof,
        "attn_sweep": sweep,
        "prefill": prefill,
        "backward": backward,
        "hybrid_mixer": hybrid,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(path, seed)
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


def hybrid_mixer(tg, torch, dev, shape, rounds=3):
    """The gated delta rule with 16 heads of 128 x 128 state over the kept
    tokens (K) and over the whole prompt (N): what pruning saves in an upper
    recurrent layer of the hybrid backbone.  Both forms: the chunked one on
    the matrix cores (tg_gated_delta_rule_chunked, the main figures) and the
    scan (tg_gated_delta_rule, under "scan").  Each figure is the median of
    three rounds of back-to-back calls (20 over the kept tokens, 5 over the
    prompt) after three warm-up calls."""
    heads, dk = 16, 128
    res, scan = {}, {}
    for name, t in (("kept", shape.k), ("full", shape.n)):
        g = torch.Generator(device=dev)
        g.manual_seed(t)
        qk = torch.nn.functional.normalize(torch.randn(2, t, heads, dk, generator=g, device=dev), dim=-1)
        q, k = qk[0].to(torch.bfloat16), qk[1].to(torch.bfloat16)
        v = torch.randn(t, heads, dk, generator=g, device=dev).to(torch.bfloat16)
        alpha = 0.9 + 0.1 * torch.rand(t, heads, generator=g, device=dev)
        beta = torch.rand(t, heads, generator=g, device=dev)
        out = torch.empty(t, heads, dk, dtype=torch.float32, device=dev)
        ws = tg.gdn_workspace(t, heads, dev)
        forms = (("chunked", lambda: tg.tg_gated_delta_rule_chunked(q, k, v, alpha, beta, out, ws)),
                 ("scan", lambda: tg.tg_gated_delta_rule(q, k, v, alpha, beta, out)))
        reps = 20 if name == "kept" else 5
        for form, fn in forms:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            per_round = []
            for _ in range(rounds):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                per_round.append(e0.elapsed_time(e1) * 1e3 / reps)
            us = sorted(per_round)[len(per_round) // 2]
            (res if form == "chunked" else scan)[name] = {"tokens": t, "us": round(us, 1),
                                                          "ns_per_token": round(us * 1e3 / t, 1)}
        del ws
    res["speedup"] = round(res["full"]["us"] / res["kept"]["us"], 2)
    res["scan"] = scan
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


def cpu_baseline(path, seed, sample_rows=384):
    """The fp64 oracle, as it stands, on the host cores over the same workload:
    scorer, sequence norm, select, compaction and RoPE in full; attention in
    full for kept lists up to 2048, else on a seeded uniform sample of query
    rows of one upper layer, scaled to all rows and layers (a query row's
    cost is linear in its index, so a uniform sample estimates the mean)."""
    from oracle import oracle
    shp, inp, a = path.shp, path.inp, path.a
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    s_norm, _ = oracle.gate_score(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, nthreads=threads)
    sc = s_norm if path.t_scores is None else path.t_scores.cpu().numpy()
    kept = oracle.select_topk(sc, inp.forced, shp.k)
    oracle.gather_rows(inp.resid, kept)
    t_path = time.perf_counter() - t0
    t1 = time.perf_counter()
    qr = oracle.rope(a.q, kept, shp.rope_theta)
    kr = oracle.rope(a.k, kept, shp.rope_theta)
    t_path += (time.perf_counter() - t1) * path.layers
    if shp.k <= 2048 and path.layers == 1:
        t1 = time.perf_counter()
        oracle.gated_attention(qr, kr, a.v, sc[kept], a.gains, shp.temp_coef, kept, nthreads=threads)
        t_attn = time.perf_counter() - t1
        sample = f"one full step of the same workload (N={shp.n}, K={shp.k}), fp64"
    else:
        rows = np.sort(np.random.default_rng(seed).choice(shp.k, size=sample_rows, replace=False))
        t1 = time.perf_counter()
        oracle.gated_attention(qr, kr, a.v, sc[kept], a.gains, shp.temp_coef, kept, rows=rows, nthreads=threads)
        t_attn = (time.perf_counter() - t1) * (shp.k / sample_rows) * path.layers
        sample = (f"scorer, select, compaction in full (N={shp.n}, K={shp.k}), RoPE of one layer x {path.layers}; "
                  f"attention on "
                  f"{sample_rows} uniformly drawn query rows of one upper layer, scaled to {shp.k} rows x "
                  f"{path.layers} layer(s); fp64")
    dt = t_path + t_attn
    return {"value": shp.n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample}, {dt:.2f} s per step ({t_path:.2f} s measured before attention)"}


if __name__ == "__main__":
    main()
