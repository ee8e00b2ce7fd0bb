"""GPU parity of each step of the path against the fp64 oracle, through the C ABI.

Sizes are ones the oracle finishes in seconds, chosen to span several tiles
and a ragged tail; the full-size workloads are in test_gpu_workloads.py.
Integer outputs (kept indices, gathered rows, positions) must match
bit-exactly; floating-point outputs within the stated tolerances.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from learned_token_pruning_mlp_amd import synth
from oracle import gap, oracle

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- gate score

def _gate_case(n, d, hd, seed, with_b1=False, b2=0.0, w1_zero=False):
    shp = synth.GateShape(n=n, d=d, hd=hd, n_forced=0, k=1, hq=1, hkv=1, head_dim=64)
    inp = synth.gate_inputs(shp, seed, with_b1=with_b1, w1_zero=w1_zero)
    inp.b2 = b2
    return inp


def _run_gate(inp, eps_row=1e-6, eps_seq=1e-6, raw=True):
    n, d = inp.resid.shape
    s_norm = torch.empty(n, dtype=torch.float32, device=gu.dev())
    s_raw = torch.empty(n, dtype=torch.float32, device=gu.dev()) if raw else None
    ws = tg.workspace(n)
    tg.tg_gate_score(gu.bf16(inp.resid), gu.bf16(inp.w1), None if inp.b1 is None else gu.bf16(inp.b1),
                     gu.bf16(inp.w2), inp.b2, eps_row, eps_seq, s_norm, s_raw, ws)
    return gu.host(s_norm), (gu.host(s_raw) if raw else None)


@pytest.mark.parametrize("n,d,hd,b1,b2", [(512, 256, 64, False, 0.0), (1000, 256, 64, True, 0.3),
                                          (777, 512, 128, True, -0.2), (333, 2048, 256, False, 0.0),
                                          (1, 128, 64, True, 0.0), (700, 192, 128, True, 0.1),
                                          (300, 320, 256, False, 0.0)])
def test_gate_score(n, d, hd, b1, b2):
    gu.say(f"gate_score n={n} d={d} hd={hd}")
    inp = _gate_case(n, d, hd, seed=11, with_b1=b1, b2=b2)
    ref_norm, ref_raw = oracle.gate_score(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2)
    got_norm, got_raw = _run_gate(inp)
    assert np.max(np.abs(got_raw - ref_raw)) <= gu.SCORE_ABS
    assert np.max(np.abs(got_norm - ref_norm)) <= gu.SCORE_ABS
    # without a raw buffer the normalised scores are the same
    again, _ = _run_gate(inp, raw=False)
    assert np.array_equal(again, got_norm)


@pytest.mark.parametrize("n,d,hd,b1,b2", [(32768, 256, 64, True, 0.1), (40001, 512, 128, False, 0.0),
                                          (32769, 2048, 256, True, -0.3)])
def test_gate_score_long_prompt_tiles(n, d, hd, b1, b2):
    """Prompts long enough for 128 residual rows per workgroup: every hidden
    width, ragged tails (a last workgroup with 1 or 65 rows)."""
    gu.say(f"gate_score long-prompt tiles n={n} d={d} hd={hd}")
    inp = _gate_case(n, d, hd, seed=13, with_b1=b1, b2=b2)
    ref_norm, ref_raw = oracle.gate_score(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2)
    got_norm, got_raw = _run_gate(inp)
    assert np.max(np.abs(got_raw - ref_raw)) <= gu.SCORE_ABS
    assert np.max(np.abs(got_norm - ref_norm)) <= gu.SCORE_ABS


def test_gate_score_zero_weights_all_equal():
    gu.say("gate_score W1=0")
    inp = _gate_case(1000, 256, 64, seed=12, w1_zero=True)
    got, raw = _run_gate(inp)
    assert np.all(raw == 0.0) and np.all(got == 0.0)


# ------------------------------------------------------------- select

def _run_select(score_f32, forced, k, n_forced=None):
    n = score_f32.size
    kept = torch.empty(k, dtype=torch.int32, device=gu.dev())
    st = torch.full((1,), -7, dtype=torch.int32, device=gu.dev())
    nf = int(forced.sum()) if (forced is not None and n_forced is None) else (n_forced or 0)
    tg.tg_select_topk(gu.f32(score_f32), None if forced is None else gu.u8(forced), nf, k, kept, st,
                      tg.workspace(n))
    return gu.host(kept), int(gu.host(st)[0])


@pytest.mark.parametrize("seed", range(6))
def test_select_small_with_ties(seed):
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(1, 3000))
    score = (g.integers(-4, 5, size=n) * 0.25).astype(np.float32)
    forced = (g.random(n) < 0.1).astype(np.uint8)
    f = int(forced.sum())
    k = int(g.integers(max(f, 1), n + 1))
    gu.say(f"select ties n={n} k={k} F={f}")
    got, st = _run_select(score, forced, k)
    assert st == 0
    assert np.array_equal(got, oracle.select_topk(score, forced, k))


@pytest.mark.parametrize("n,k,f", [(16384, 2048, 64), (32768, 4096, 64), (40000, 9000, 100),
                                   (131072, 8192, 128)])
def test_select_gaussian(n, k, f):
    gu.say(f"select n={n} k={k}")
    g = np.random.default_rng(n)
    score = g.standard_normal(n).astype(np.float32)
    forced = np.zeros(n, np.uint8)
    forced[g.choice(n, size=f, replace=False)] = 1
    got, st = _run_select(score, forced, k)
    assert st == 0
    assert np.array_equal(got, oracle.select_topk(score, forced, k))


@pytest.mark.parametrize("n", [16384, 40000])
def test_select_all_equal_closed_form(n):
    """All scores equal: the ties go to the lowest indices.  At 40000 tokens
    (keys re-read from memory) the first round's bucket is too large to
    gather, so the later rounds take the prefix-filtered sweep."""
    k, f = 1024, 64
    gu.say(f"select all-equal n={n}")
    forced = np.zeros(n, np.uint8)
    forced[-f:] = 1
    got, st = _run_select(np.zeros(n, np.float32), forced, k)
    assert st == 0
    assert np.array_equal(got, np.concatenate([np.arange(k - f), np.arange(n - f, n)]))


def test_select_extremes_and_specials():
    gu.say("select extremes")
    g = np.random.default_rng(5)
    n = 5000
    score = g.standard_normal(n).astype(np.float32)
    forced = np.zeros(n, np.uint8)
    forced[[0, 17, 4999]] = 1
    assert np.array_equal(_run_select(score, forced, n)[0], np.arange(n))
    assert np.array_equal(_run_select(score, forced, 3)[0], np.array([0, 17, 4999]))
    assert np.array_equal(_run_select(score, None, 1)[0], np.array([np.argmax(score)]))
    sp = np.array([np.nan, -0.0, 0.0, -np.inf, 1.0, np.nan, np.inf, -1.0], np.float32)
    for k in range(1, sp.size + 1):
        assert np.array_equal(_run_select(sp, None, k)[0], oracle.select_topk(sp, None, k)), k


def test_select_forced_count_status():
    gu.say("select status")
    n = 2000
    score = np.random.default_rng(6).standard_normal(n).astype(np.float32)
    forced = np.zeros(n, np.uint8)
    forced[-50:] = 1
    got, st = _run_select(score, forced, 100, n_forced=40)  # caller's F is wrong
    assert st == tg.TG_STATUS_FORCED_MISMATCH
    assert np.array_equal(got, oracle.select_topk(score, forced, 100))
    got, st = _run_select(score, forced, 45, n_forced=45)  # 50 forced > k = 45
    assert st == tg.TG_STATUS_FORCED_MISMATCH | tg.TG_STATUS_FORCED_OVER_K
    assert np.array_equal(got, np.arange(n - 50, n - 5))


@pytest.mark.parametrize("case", ["ragged_16385", "ragged_50001", "ragged_131071", "kpt16_262147",
                                  "kpt32_524288", "one_wg_beyond_524289", "int_ties_100000", "student_t_65536",
                                  "specials_40000", "k_equals_n_70000", "k_one_70000", "all_equal_131072",
                                  "few_ties_131072", "no_forced_50001", "whole_chunks_98304"])
def test_select_many_workgroups(case):
    """Prompts past 16384 tokens: the select that runs over chunks of the
    prompt in several workgroups (three launches), at ragged lengths and
    whole chunks, each chunk size, heavy ties (five values at 131072 tokens:
    the first round's bin holds more keys than the last launch keeps in
    LDS, so it reads them from memory), heavy tails, special values, no
    forced mask, the budget extremes and the all-equal closed form; one case
    past its largest size (the one-workgroup fallback)."""
    name, n = case.rsplit("_", 1)
    n = int(n)
    g = np.random.default_rng(n + len(name))
    forced = np.zeros(n, np.uint8)
    forced[g.choice(n, size=96, replace=False)] = 1
    k = max(96, n // 16)
    if name == "int_ties":
        score = g.integers(-6, 7, size=n).astype(np.float32) * 0.5
    elif name == "few_ties":
        score = g.integers(-2, 3, size=n).astype(np.float32)
    elif name == "student_t":
        score = synth.student_t_scores(n, seed=9)
    elif name == "specials":
        score = g.standard_normal(n).astype(np.float32)
        sp = g.choice(n, size=4000, replace=False)
        score[sp] = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0], np.float32)[np.arange(4000) % 5]
    elif name == "all_equal":
        score = np.zeros(n, np.float32)
    else:
        score = g.standard_normal(n).astype(np.float32)
    if name == "k_equals":
        k = n
    elif name == "k_one":
        forced[:] = 0
        k = 1
    if name == "no_forced":
        forced = None
    gu.say(f"select many workgroups: {case} k={k}")
    got, st = _run_select(score, forced, k)
    assert st == 0
    if name == "all_equal":
        fi = np.flatnonzero(forced)
        want = np.sort(np.concatenate([np.setdiff1d(np.arange(n), fi)[:k - fi.size], fi]))
        assert np.array_equal(got, want)
    assert np.array_equal(got, oracle.select_topk(score, forced, k))


def test_select_many_workgroups_status():
    gu.say("select status, many workgroups")
    n = 70000
    score = np.random.default_rng(16).standard_normal(n).astype(np.float32)
    forced = np.zeros(n, np.uint8)
    forced[-500:] = 1
    got, st = _run_select(score, forced, 3000, n_forced=400)  # caller's F is wrong
    assert st == tg.TG_STATUS_FORCED_MISMATCH
    assert np.array_equal(got, oracle.select_topk(score, forced, 3000))
    got, st = _run_select(score, forced, 450, n_forced=450)  # 500 forced > k = 450
    assert st == tg.TG_STATUS_FORCED_MISMATCH | tg.TG_STATUS_FORCED_OVER_K
    assert np.array_equal(got, np.arange(n - 500, n - 50))


# ------------------------------------------------------------- compaction

@pytest.mark.parametrize("n,k,d", [(512, 128, 256), (16384, 2048, 2048), (3001, 1999, 64)])
def test_compact(n, k, d):
    gu.say(f"compact n={n} k={k} d={d}")
    g = np.random.default_rng(k)
    resid = g.integers(0, 65536, size=(n, d), dtype=np.uint16)
    idx = np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)
    pos = (np.arange(n) * 3 + 7).astype(np.int32)
    score = g.standard_normal(n).astype(np.float32)
    kv_k = g.integers(0, 65536, size=(n, 8, 128), dtype=np.uint16)
    kv_v = g.integers(0, 65536, size=(n, 2, 64), dtype=np.uint16)
    d_resid, d_kk, d_vv = gu.bf16(resid), gu.bf16(kv_k), gu.bf16(kv_v)
    out = torch.empty((k, d), dtype=torch.bfloat16, device=gu.dev())
    ok_, ov_ = (torch.empty((k, 8, 128), dtype=torch.bfloat16, device=gu.dev()),
                torch.empty((k, 2, 64), dtype=torch.bfloat16, device=gu.dev()))
    pos_out = torch.empty(k, dtype=torch.int32, device=gu.dev())
    s_out = torch.empty(k, dtype=torch.float32, device=gu.dev())
    tg.tg_compact(gu.i32(idx), n, d_resid, out, gu.i32(pos), pos_out, gu.f32(score), s_out,
                  extra=[(d_kk, ok_), (d_vv, ov_)])
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits(out), oracle.gather_rows(resid, idx))
    assert np.array_equal(gu.bits(ok_), oracle.gather_rows(kv_k, idx))
    assert np.array_equal(gu.bits(ov_), oracle.gather_rows(kv_v, idx))
    assert np.array_equal(gu.host(pos_out), oracle.gather_rows(pos, idx))
    assert np.array_equal(gu.host(s_out).view(np.uint32), oracle.gather_rows(score, idx).view(np.uint32))
    # default positions are the kept indices themselves
    tg.tg_compact(gu.i32(idx), n, None, None, None, pos_out, None, None)
    assert np.array_equal(gu.host(pos_out), idx)


# ------------------------------------------------------------- RoPE

@pytest.mark.parametrize("rows,heads,D", [(300, 4, 64), (2048, 24, 128), (5, 1, 2), (3, 2, 48), (131, 8, 256)])
def test_rope(rows, heads, D):
    gu.say(f"rope rows={rows} heads={heads} D={D}")
    g = np.random.default_rng(rows)
    x = synth.normal_bf16(rows, 1, (rows, heads, D))
    pos = np.sort(g.choice(131072, size=rows, replace=False)).astype(np.int32)
    t = gu.bf16(x)
    tg.tg_rope(t, gu.i32(pos), 1.0e6)
    got = gu.bits(t)
    want = oracle.rope(x, pos, 1.0e6)
    # identical bf16 except where a last-bit difference of the fp64 angle
    # crosses a rounding boundary: at most one unit in the last place
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff != 0) < 1e-3


def test_rope_unaligned_buffer():
    """A tensor that starts 2 bytes past a 16-byte boundary takes the
    per-element path; results are the same as for an aligned copy."""
    gu.say("rope unaligned rows=77 heads=3 D=128")
    rows, heads, D = 77, 3, 128
    g = np.random.default_rng(5)
    x = synth.normal_bf16(9, 1, (rows, heads, D))
    pos = np.sort(g.choice(50000, size=rows, replace=False)).astype(np.int32)
    flat = torch.empty(rows * heads * D + 8, dtype=torch.bfloat16, device=gu.dev())
    t = flat[1:1 + rows * heads * D].view(rows, heads, D)
    t.copy_(gu.bf16(x))
    assert t.data_ptr() % 16 == 2
    tg.tg_rope(t, gu.i32(pos), 1.0e6)
    a = gu.bf16(x)
    tg.tg_rope(a, gu.i32(pos), 1.0e6)
    assert np.array_equal(gu.bits(t), gu.bits(a))
    diff = np.abs(gu.bits(t).astype(np.int32) - oracle.rope(x, pos, 1.0e6).astype(np.int32))
    assert diff.max() <= 1


@pytest.mark.parametrize("rows,hq,hk,D", [(2048, 16, 8, 128), (301, 4, 2, 64), (7, 3, 5, 48), (1, 1, 1, 128),
                                          (999, 6, 2, 256)])
def test_rope_qk(rows, hq, hk, D):
    """q and k rotated in one launch equal the per-tensor results bit for bit."""
    gu.say(f"rope_qk rows={rows} hq={hq} hk={hk} D={D}")
    g = np.random.default_rng(rows + hq)
    xq = synth.normal_bf16(rows + 1, 1, (rows, hq, D))
    xk = synth.normal_bf16(rows + 2, 1, (rows, hk, D))
    pos = np.sort(g.choice(131072, size=rows, replace=False)).astype(np.int32)
    tq, tk = gu.bf16(xq), gu.bf16(xk)
    tg.tg_rope_qk(tq, tk, gu.i32(pos), 1.0e6)
    rq, rk = gu.bf16(xq), gu.bf16(xk)
    tg.tg_rope(rq, gu.i32(pos), 1.0e6)
    tg.tg_rope(rk, gu.i32(pos), 1.0e6)
    assert np.array_equal(gu.bits(tq), gu.bits(rq))
    assert np.array_equal(gu.bits(tk), gu.bits(rk))
    for got, x in ((gu.bits(tq), xq), (gu.bits(tk), xk)):
        diff = np.abs(got.astype(np.int32) - oracle.rope(x, pos, 1.0e6).astype(np.int32))
        assert diff.max() <= 1
        assert np.mean(diff != 0) < 1e-3


def test_rope_qk_unaligned_k():
    """A key buffer 2 bytes past a 16-byte boundary sends both tensors down
    the per-element path; results equal the aligned ones."""
    gu.say("rope_qk unaligned k rows=64 hq=4 hk=2 D=128")
    rows, hq, hk, D = 64, 4, 2, 128
    xq = synth.normal_bf16(21, 1, (rows, hq, D))
    xk = synth.normal_bf16(22, 1, (rows, hk, D))
    pos = (np.arange(rows) * 37).astype(np.int32)
    flat = torch.empty(rows * hk * D + 8, dtype=torch.bfloat16, device=gu.dev())
    tk = flat[1:1 + rows * hk * D].view(rows, hk, D)
    tk.copy_(gu.bf16(xk))
    tq = gu.bf16(xq)
    tg.tg_rope_qk(tq, tk, gu.i32(pos), 1.0e6)
    aq, ak = gu.bf16(xq), gu.bf16(xk)
    tg.tg_rope_qk(aq, ak, gu.i32(pos), 1.0e6)
    assert np.array_equal(gu.bits(tq), gu.bits(aq))
    assert np.array_equal(gu.bits(tk), gu.bits(ak))


# ------------------------------------------------------------- attention

def _run_attn(a, out_dtype=torch.float32):
    nk, hq, D = a.q.shape
    out = torch.empty((nk, hq, D), dtype=out_dtype, device=gu.dev())
    tg.tg_gated_attention(gu.bf16(a.q), gu.bf16(a.k), gu.bf16(a.v), gu.f32(a.key_score), gu.f32(a.gains),
                          a.temp_coef, gu.i32(a.pos), out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("nk,hq,hkv,D", [(128, 4, 2, 64), (200, 4, 2, 64), (333, 8, 1, 128),
                                         (257, 6, 6, 128), (96, 16, 2, 64), (1, 4, 2, 128),
                                         (1000, 16, 8, 128)])
def test_attention(nk, hq, hkv, D):
    gu.say(f"attention nk={nk} hq={hq} hkv={hkv} D={D}")
    a = synth.attn_inputs(nk, hq, hkv, D, seed=nk + hq)
    ref = oracle.gated_attention(a.q, a.k, a.v, a.key_score, a.gains, a.temp_coef, a.pos)
    out32 = _run_attn(a, torch.float32)
    gu.check_attention(gu.host(out32), ref, "fp32 out")
    out16 = _run_attn(a, torch.bfloat16)
    # the bf16 output against the oracle: relative RMS, and one bf16 unit of
    # the oracle's rounding (or the fp32 bound) per element
    gu.check_attention_bf16(gu.bits(out16), ref, "bf16 out")
    # and it is the nearest-even rounding of the fp32 result
    assert np.array_equal(gu.bits(out16), oracle.to_bf16(gu.host(out32).astype(np.float64)))


def test_attention_large_temperature_and_bias():
    # heavy-tailed scores (biases up to ~40) and a temperature coefficient
    # large enough to make lambda negative for early rows
    gu.say("attention heavy-tailed scores, negative lambda")
    nk = 700
    ks = synth.student_t_scores(nk, 3)
    pos = np.sort(np.random.default_rng(77).choice(50 * nk, size=nk, replace=False)).astype(np.int32)
    a = synth.attn_inputs(nk, 4, 2, 128, seed=77, key_score=ks, temp_coef=0.6, pos=pos)
    lam = 1 + 0.6 * np.log((np.arange(nk) + 1) / (a.pos + 1.0))
    assert lam.min() < 0
    ref = oracle.gated_attention(a.q, a.k, a.v, a.key_score, a.gains, a.temp_coef, a.pos)
    gu.check_attention(gu.host(_run_attn(a)), ref, "heavy tails")


@pytest.mark.parametrize("nk", [1000, 2048])
def test_attention_timed_matches_plain(nk):
    """tg_gated_attention_timed: the same output bit for bit (fp32 and bf16),
    and its events hold a positive interval no longer than that of events
    recorded around the call on the same stream."""
    gu.say(f"attention timed variant nk={nk}")
    a = synth.attn_inputs(nk, 16, 8, 128, seed=nk)
    args = (gu.bf16(a.q), gu.bf16(a.k), gu.bf16(a.v), gu.f32(a.key_score), gu.f32(a.gains), a.temp_coef,
            gu.i32(a.pos))
    stream = torch.cuda.current_stream()
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for dt in (torch.float32, torch.bfloat16):
        plain = torch.empty((nk, 16, 128), dtype=dt, device=gu.dev())
        timed = torch.full((nk, 16, 128), float("nan"), dtype=dt, device=gu.dev())
        tg.tg_gated_attention(*args, plain)
        s0, s1, o0, o1 = Ev(), Ev(), Ev(), Ev()
        for e in (s0, s1):
            e.record(stream)  # creates the event's handle
        torch.cuda.synchronize()
        o0.record(stream)
        tg.tg_gated_attention_timed(*args, timed, s0, s1)
        o1.record(stream)
        torch.cuda.synchronize()
        assert torch.equal(plain.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           timed.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        inner, outer = s0.elapsed_time(s1), o0.elapsed_time(o1)
        gu.say(f"  {dt}: kernel events {inner * 1e3:.1f} us, events around the call {outer * 1e3:.1f} us")
        assert 0.0 < inner <= outer + 1e-3
    with pytest.raises(ValueError):
        tg.tg_gated_attention_timed(*args, plain, Ev(), Ev())  # events never recorded: no handle yet


def test_attention_deterministic():
    gu.say("attention determinism")
    a = synth.attn_inputs(1500, 16, 8, 128, seed=3)
    o1 = gu.host(_run_attn(a))
    o2 = gu.host(_run_attn(a))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
