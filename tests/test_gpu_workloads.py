"""GPU parity at the full sizes of the path's workloads, in the launch
configuration the benchmark times (same entry points, same shapes).

Where the oracle cannot redo everything in seconds it recomputes sampled
outputs one by one (query rows of the attention, rows of the scorer) and the
rest is checked through properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from learned_token_pruning_mlp_amd import synth
from oracle import gap, oracle

pytestmark = pytest.mark.gpu


def sample_rows(k: int, seed: int, n_rand: int = 320, per_block: bool = True):
    """First 64, last 128 and n_rand seeded random query rows, plus (per_block)
    one seeded row inside every 32-row query block, so every block of every
    launch shape's (b, last - b) pairing is checked (sorted, distinct)."""
    g = np.random.default_rng(seed)
    rows = set(range(min(64, k))) | set(range(max(0, k - 128), k))
    rows |= set(g.choice(k, size=min(n_rand, k), replace=False).tolist())
    if per_block:
        starts = np.arange(0, k, 32)
        rows |= set(np.minimum(starts + g.integers(0, 32, size=starts.size), k - 1).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _gate(inp, n):
    s_norm = torch.empty(n, dtype=torch.float32, device=gu.dev())
    s_raw = torch.empty(n, dtype=torch.float32, device=gu.dev())
    ws = tg.workspace(n)
    tg.tg_gate_score(gu.bf16(inp.resid), gu.bf16(inp.w1), None, gu.bf16(inp.w2), inp.b2, 1e-6, 1e-6,
                     s_norm, s_raw, ws)
    return s_norm, s_raw, ws


def test_headline_path_n16k():
    """Qwen3-1.7B-shaped gate layer, N=16384 (64 forced), K=2048: the whole
    path, each stage against the oracle."""
    shp = synth.QWEN3_1P7B_N16K
    gu.say("headline path N=16384 K=2048: inputs + oracle")
    inp = synth.gate_inputs(shp, seed=2)
    ref_norm, ref_raw = gap.enforce_gate_gap(inp, 2, [shp.k])
    ref_kept = oracle.select_topk(ref_norm, inp.forced, shp.k)

    gu.say("headline: gate_score")
    s_norm, s_raw, ws = _gate(inp, shp.n)
    got_norm = gu.host(s_norm)
    assert np.max(np.abs(got_norm - ref_norm)) <= gu.SCORE_ABS
    assert np.max(np.abs(gu.host(s_raw) - ref_raw)) <= gu.SCORE_ABS

    gu.say("headline: select")
    kept = torch.empty(shp.k, dtype=torch.int32, device=gu.dev())
    st = torch.empty(1, dtype=torch.int32, device=gu.dev())
    tg.tg_select_topk(s_norm, gu.u8(inp.forced), shp.n_forced, shp.k, kept, st, ws)
    assert int(gu.host(st)[0]) == 0
    assert np.array_equal(gu.host(kept), ref_kept)

    gu.say("headline: compact")
    resid_k = torch.empty((shp.k, shp.d), dtype=torch.bfloat16, device=gu.dev())
    pos_k = torch.empty(shp.k, dtype=torch.int32, device=gu.dev())
    score_k = torch.empty(shp.k, dtype=torch.float32, device=gu.dev())
    tg.tg_compact(kept, shp.n, gu.bf16(inp.resid), resid_k, gu.i32(inp.pos), pos_k, s_norm, score_k)
    assert np.array_equal(gu.bits(resid_k), inp.resid[ref_kept])
    assert np.array_equal(gu.host(pos_k), ref_kept)
    assert np.array_equal(gu.host(score_k), got_norm[ref_kept])

    gu.say("headline: attention K=2048 (full oracle)")
    a = synth.attn_inputs(shp.k, shp.hq, shp.hkv, shp.head_dim, seed=2, pos=ref_kept,
                          key_score=got_norm[ref_kept])
    q, kk = gu.bf16(a.q), gu.bf16(a.k)
    tg.tg_rope_qk(q, kk, pos_k, shp.rope_theta)
    q_bits, k_bits = gu.bits(q), gu.bits(kk)
    out = torch.empty((shp.k, shp.hq, shp.head_dim), dtype=torch.float32, device=gu.dev())
    tg.tg_gated_attention(q, kk, gu.bf16(a.v), score_k, gu.f32(a.gains), shp.temp_coef, pos_k, out)
    ref = oracle.gated_attention(q_bits, k_bits, a.v, a.key_score, a.gains, shp.temp_coef, ref_kept)
    gu.check_attention(gu.host(out), ref, "headline attention")
    gu.say("headline: attention K=2048, bf16 output (the benchmark's configuration)")
    out16 = torch.empty((shp.k, shp.hq, shp.head_dim), dtype=torch.bfloat16, device=gu.dev())
    tg.tg_gated_attention(q, kk, gu.bf16(a.v), score_k, gu.f32(a.gains), shp.temp_coef, pos_k, out16)
    gu.check_attention_bf16(gu.bits(out16), ref, "headline attention, bf16 out")


def test_path_graph_replays_match_eager():
    """The whole headline step captured as one HIP graph (the launch sequence
    is fixed once K is known): every replay, with eager work and
    synchronisations between the replays, reproduces the eager outputs bit
    for bit."""
    shp = synth.QWEN3_1P7B_N16K
    gu.say("graph replays of the headline step")
    n, k = shp.n, shp.k
    inp = synth.gate_inputs(shp, seed=2)
    a = synth.attn_inputs(k, shp.hq, shp.hkv, shp.head_dim, seed=2)
    resid, w1, w2 = gu.bf16(inp.resid), gu.bf16(inp.w1), gu.bf16(inp.w2)
    forced, pos = gu.u8(inp.forced), gu.i32(inp.pos)
    q0, k0, v, gains = gu.bf16(a.q), gu.bf16(a.k), gu.bf16(a.v), gu.f32(a.gains)
    q, kk = q0.clone(), k0.clone()
    dev = gu.dev()
    s_norm = torch.empty(n, dtype=torch.float32, device=dev)
    ws = tg.workspace(n)
    kept = torch.empty(k, dtype=torch.int32, device=dev)
    resid_k = torch.empty((k, shp.d), dtype=torch.bfloat16, device=dev)
    pos_k = torch.empty(k, dtype=torch.int32, device=dev)
    score_k = torch.empty(k, dtype=torch.float32, device=dev)
    out = torch.empty((k, shp.hq, shp.head_dim), dtype=torch.float32, device=dev)

    def step():
        tg.tg_gate_score(resid, w1, None, w2, 0.0, 1e-6, 1e-6, s_norm, None, ws)
        tg.tg_select_topk(s_norm, forced, shp.n_forced, k, kept, None, ws)
        tg.tg_compact(kept, n, resid, resid_k, pos, pos_k, s_norm, score_k)
        tg.tg_rope_qk(q, kk, pos_k, shp.rope_theta)
        tg.tg_gated_attention(q, kk, v, score_k, gains, shp.temp_coef, pos_k, out)

    def snapshot():
        ts = (s_norm, kept, resid_k.view(torch.int16), pos_k, score_k, out, q.view(torch.int16), kk.view(torch.int16))
        return [gu.host(t).view(np.uint8).copy() for t in ts]

    step()
    want = snapshot()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        q.copy_(q0)  # RoPE works in place: every replay starts from the same q and k
        kk.copy_(k0)
        for t in (s_norm, score_k, out):
            t.fill_(float("nan"))
        kept.fill_(-1)
        pos_k.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for x, y in zip(got, want):
            assert np.array_equal(x, y), f"replay {r}"


@pytest.mark.parametrize("k", synth.N32K_BUDGETS)
def test_budget_sweep_n32k(k):
    """N=32768, Student-t (df=3) scores fed straight to select; budgets
    1024 / 4096 / 8192 from one set of scores."""
    n, f = 32768, 64
    gu.say(f"n32k sweep K={k}")
    forced = np.zeros(n, np.uint8)
    forced[-f:] = 1
    scores = synth.student_t_scores(n, seed=3)
    gap.enforce_score_gap(scores, forced, 3, synth.N32K_BUDGETS)
    ref_kept = oracle.select_topk(scores, forced, k)
    d_scores = gu.f32(scores)
    kept = torch.empty(k, dtype=torch.int32, device=gu.dev())
    tg.tg_select_topk(d_scores, gu.u8(forced), f, k, kept, None, tg.workspace(n))
    assert np.array_equal(gu.host(kept), ref_kept)
    score_k = torch.empty(k, dtype=torch.float32, device=gu.dev())
    pos_k = torch.empty(k, dtype=torch.int32, device=gu.dev())
    tg.tg_compact(kept, n, None, None, None, pos_k, d_scores, score_k)
    a = synth.attn_inputs(k, 16, 8, 128, seed=3 + k, pos=ref_kept, key_score=scores[ref_kept])
    out = torch.empty((k, 16, 128), dtype=torch.float32, device=gu.dev())
    tg.tg_gated_attention(gu.bf16(a.q), gu.bf16(a.k), gu.bf16(a.v), score_k, gu.f32(a.gains), 0.1, pos_k, out)
    # K = 1024 and 4096: every row; K = 8192: sampled rows, one in every
    # 32-row query block among them
    rows = sample_rows(k, k) if k > 4096 else None
    ref = oracle.gated_attention(a.q, a.k, a.v, a.key_score, a.gains, 0.1, ref_kept, rows=rows)
    got = gu.host(out)
    gu.check_attention(got if rows is None else got[rows], ref, f"n32k K={k}")


def test_gate_score_n32k():
    shp = synth.QWEN3_1P7B_N32K
    gu.say("gate_score N=32768")
    inp = synth.gate_inputs(shp, seed=3)
    ref_norm, _ = oracle.gate_score(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2)
    s_norm, _, _ = _gate(inp, shp.n)
    assert np.max(np.abs(gu.host(s_norm) - ref_norm)) <= gu.SCORE_ABS


def test_long_n128k_26_layers():
    """N=131072, K=8192, 128 forced tokens scattered over the last 1024;
    K/V kept for kept rows only across 26 stacked upper layers; the two
    lower layers' full-length KV trimmed through extra gather streams.
    Scores are checked against the oracle's for all 131072 tokens, with the
    boundary gap enforced in the oracle's scores, and the kept set against
    the oracle's own top-K."""
    shp = synth.QWEN3_1P7B_N128K
    n, k, layers = shp.n, shp.k, synth.N128K_UPPER_LAYERS
    gu.say("n128k: inputs + oracle scores of all rows (boundary gap enforced)")
    inp = synth.gate_inputs(shp, seed=4)
    ref_norm, ref_raw = gap.enforce_gate_gap(inp, 4, [k])
    gc = gu.boundary_gap(ref_norm, inp.forced, k)
    assert gc is not None and gc[0] > 1e-3
    gu.say("n128k: gate_score")
    s_norm, s_raw, ws = _gate(inp, n)
    got_norm, got_raw = gu.host(s_norm), gu.host(s_raw)
    assert np.max(np.abs(got_raw - ref_raw)) <= gu.SCORE_ABS
    assert np.max(np.abs(got_norm - ref_norm)) <= gu.SCORE_ABS

    gu.say("n128k: select")
    kept = torch.empty(k, dtype=torch.int32, device=gu.dev())
    st = torch.empty(1, dtype=torch.int32, device=gu.dev())
    tg.tg_select_topk(s_norm, gu.u8(inp.forced), shp.n_forced, k, kept, st, ws)
    kept_h = gu.host(kept)
    assert int(gu.host(st)[0]) == 0
    ref_kept = oracle.select_topk(ref_norm, inp.forced, k)
    assert np.array_equal(kept_h, ref_kept)

    gu.say("n128k: compact + lower-layer KV trim")
    g = np.random.default_rng(4)
    lower = [gu.bf16(g.integers(0, 65536, size=(n, 8, 128), dtype=np.uint16)) for _ in range(4)]
    lower_out = [torch.empty((k, 8, 128), dtype=torch.bfloat16, device=gu.dev()) for _ in range(4)]
    resid_k = torch.empty((k, shp.d), dtype=torch.bfloat16, device=gu.dev())
    pos_k = torch.empty(k, dtype=torch.int32, device=gu.dev())
    score_k = torch.empty(k, dtype=torch.float32, device=gu.dev())
    tg.tg_compact(kept, n, gu.bf16(inp.resid), resid_k, gu.i32(inp.pos), pos_k, s_norm, score_k,
                  extra=list(zip(lower, lower_out)))
    assert np.array_equal(gu.bits(resid_k), inp.resid[ref_kept])
    assert np.array_equal(gu.host(pos_k), inp.pos[ref_kept])
    assert np.array_equal(gu.host(score_k), got_norm[ref_kept])
    for src, dst in zip(lower, lower_out):
        assert np.array_equal(gu.bits(dst), gu.bits(src)[ref_kept])
    del lower, lower_out

    gu.say("n128k: 26 upper layers of gated attention")
    kv_k = torch.empty((layers, k, 8, 128), dtype=torch.bfloat16, device=gu.dev())
    kv_v = torch.empty((layers, k, 8, 128), dtype=torch.bfloat16, device=gu.dev())
    check = {0: None, layers - 1: None}
    outs = {}
    for L in range(layers):
        a = synth.attn_inputs(k, 16, 8, 128, seed=4, layer=L, pos=ref_kept, key_score=got_norm[ref_kept])
        kv_k[L].copy_(gu.bf16(a.k))
        kv_v[L].copy_(gu.bf16(a.v))
        out = torch.empty((k, 16, 128), dtype=torch.float32, device=gu.dev())
        tg.tg_gated_attention(gu.bf16(a.q), kv_k[L], kv_v[L], score_k, gu.f32(a.gains), 0.1, pos_k, out)
        if L in check:
            outs[L] = (a, gu.host(out))
    for L, (a, got) in outs.items():
        r = sample_rows(k, 40 + L)
        ref = oracle.gated_attention(a.q, a.k, a.v, a.key_score, a.gains, 0.1, ref_kept, rows=r)
        gu.check_attention(got[r], ref, f"n128k layer {L}")


def test_degenerate_full_budget_is_causal_attention():
    """K = N = 16384, gains 0, temperature 0: standard causal GQA attention."""
    n = 16384
    gu.say("degenerate K=N")
    a = synth.attn_inputs(n, 16, 8, 128, seed=5, pos=np.arange(n, dtype=np.int32))
    out = torch.empty((n, 16, 128), dtype=torch.float32, device=gu.dev())
    tg.tg_gated_attention(gu.bf16(a.q), gu.bf16(a.k), gu.bf16(a.v), gu.f32(a.key_score),
                          gu.f32(np.zeros(16, np.float32)), 0.0, gu.i32(a.pos), out)
    rows = sample_rows(n, 5, n_rand=192)
    ref = oracle.gated_attention(a.q, a.k, a.v, a.key_score, np.zeros(16), 0.0, a.pos, rows=rows)
    gu.check_attention(gu.host(out)[rows], ref, "K=N")


def test_degenerate_all_ties_pipeline():
    """W1 = 0: every score is 0, K = N/16 = 1024 with the last 64 forced;
    ties go to the lower index, and a constant bias cancels in attention."""
    shp = synth.GateShape(n=16384, d=2048, hd=256, n_forced=64, k=1024, hq=16, hkv=8, head_dim=128)
    gu.say("degenerate all ties")
    inp = synth.gate_inputs(shp, seed=5, w1_zero=True)
    s_norm, _, ws = _gate(inp, shp.n)
    assert np.all(gu.host(s_norm) == 0.0)
    kept = torch.empty(shp.k, dtype=torch.int32, device=gu.dev())
    tg.tg_select_topk(s_norm, gu.u8(inp.forced), 64, shp.k, kept, None, ws)
    want = np.concatenate([np.arange(shp.k - 64), np.arange(shp.n - 64, shp.n)])
    assert np.array_equal(gu.host(kept), want)
    a = synth.attn_inputs(shp.k, 16, 8, 128, seed=5, pos=want.astype(np.int32),
                          key_score=np.zeros(shp.k, np.float32))
    out = torch.empty((shp.k, 16, 128), dtype=torch.float32, device=gu.dev())
    tg.tg_gated_attention(gu.bf16(a.q), gu.bf16(a.k), gu.bf16(a.v), gu.f32(a.key_score), gu.f32(a.gains), 0.1,
                          gu.i32(a.pos), out)
    ref = oracle.gated_attention(a.q, a.k, a.v, a.key_score, np.zeros(16), 0.1, a.pos)
    gu.check_attention(gu.host(out), ref, "all ties")
