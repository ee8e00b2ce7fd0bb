"""Pins of the oracle's token-gated attention, RoPE and bf16 rounding (CPU only).

Special cases reduce the gated attention to torch's scaled_dot_product_attention
in fp64 (a library routine, not the oracle's loops); a pure-Python brute force
covers a tiny general case; a hand-worked two-key instance pins the logit and
temperature form; invariants cover the rest.
"""
import math

import numpy as np
import pytest
import torch

import brute
from conftest import golden
from learned_token_pruning_mlp_amd import synth
from oracle import oracle


def _sdpa_causal(q, k, v, scale=None, mask=None):
    """q [K,hq,D], k/v [K,hkv,D] float64 -> [K,hq,D]; GQA by contiguous groups."""
    K, hq, D = q.shape
    G = hq // k.shape[1]
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    Kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    Vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    if mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True, scale=scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=torch.from_numpy(mask)[None],
                                                             scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _inputs(K, hq, hkv, D, seed):
    a = synth.attn_inputs(K, hq, hkv, D, seed)
    return (oracle.widen_bf16(a.q), oracle.widen_bf16(a.k), oracle.widen_bf16(a.v), a)


def test_full_budget_zero_gain_is_causal_gqa_sdpa():
    # K = N (no pruning: pos = arange, so lambda = 1 for any c) and gains 0
    q, k, v, a = _inputs(96, 4, 2, 64, 1)
    pos = np.arange(96, dtype=np.int32)
    got = oracle.gated_attention_f64(q, k, v, a.key_score, np.zeros(4), 0.7, pos)
    want = _sdpa_causal(q, k, v)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_zero_gain_zero_temperature_is_sdpa_on_subsequence():
    q, k, v, a = _inputs(80, 6, 3, 32, 2)
    got = oracle.gated_attention_f64(q, k, v, a.key_score, np.zeros(6), 0.0, a.pos)
    assert np.max(np.abs(got - _sdpa_causal(q, k, v))) <= 1e-12


def test_constant_temperature_is_scaled_sdpa_with_key_bias():
    # pos_t = 2(t+1) - 1 makes (t+1)/(pos_t+1) = 1/2 for every row, so
    # lambda is the constant 1 + c ln(1/2): scale lambda/sqrt(D), bias lambda*g_h*s_j
    K, hq, hkv, D, c = 64, 4, 1, 64, 0.3
    q, k, v, a = _inputs(K, hq, hkv, D, 3)
    pos = (2 * (np.arange(K) + 1) - 1).astype(np.int32)
    got = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, c, pos)
    lam = 1.0 + c * math.log(0.5)
    causal = np.where(np.tril(np.ones((K, K), bool)), 0.0, -np.inf)
    mask = np.stack([causal + lam * float(a.gains[h]) * a.key_score[None, :].astype(np.float64)
                     for h in range(hq)])
    want = _sdpa_causal(q, k, v, scale=lam / math.sqrt(D), mask=mask)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_matches_bruteforce_tiny():
    K, hq, hkv, D = 9, 4, 2, 8
    q, k, v, a = _inputs(K, hq, hkv, D, 4)
    c = 0.35
    want = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), a.key_score.tolist(),
                                    a.gains.tolist(), c, a.pos.tolist()))
    got = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, c, a.pos)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_two_key_worked_example():
    rows = golden("attention_two_key.txt")
    r2 = math.sqrt(2.0)
    q = np.array([[[1.0, 0.0]], [[1.0, 0.0]]])
    k = np.array([[[0.0, 0.0]], [[r2, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    got = oracle.gated_attention_f64(q, k, v, np.array([0.0, 0.5]), np.array([2.0]), 0.5,
                                     np.array([0, 3], np.int32))
    for t, o0, o1 in rows:
        assert abs(got[int(t), 0, 0] - o0) <= 1e-15
        assert abs(got[int(t), 0, 1] - o1) <= 1e-15


def test_invariants():
    K, hq, hkv, D = 70, 4, 2, 16
    q, k, v, a = _inputs(K, hq, hkv, D, 5)
    base = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, 0.2, a.pos)
    # row 0 sees only key 0
    G = hq // hkv
    for h in range(hq):
        assert np.array_equal(base[0, h], v[0, h // G])
    # adding a constant to every key score shifts each row's logits by a constant
    shifted = oracle.gated_attention_f64(q, k, v, a.key_score.astype(np.float64) + 3.5, a.gains, 0.2, a.pos)
    assert np.max(np.abs(shifted - base)) <= 1e-12
    # all scores equal: the bias has no effect
    eq = oracle.gated_attention_f64(q, k, v, np.full(K, 1.7), a.gains, 0.2, a.pos)
    nobias = oracle.gated_attention_f64(q, k, v, np.zeros(K), np.zeros(hq), 0.2, a.pos)
    assert np.max(np.abs(eq - nobias)) <= 1e-12
    # the output is a convex combination of the visible values
    for t in (1, 17, K - 1):
        for h in range(hq):
            vis = v[: t + 1, h // G]
            assert np.all(base[t, h] <= vis.max(axis=0) + 1e-12)
            assert np.all(base[t, h] >= vis.min(axis=0) - 1e-12)


def test_row_subset_matches_full():
    q, k, v, a = _inputs(50, 4, 2, 32, 6)
    full = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, 0.1, a.pos)
    rows = [0, 7, 49, 20]
    sub = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, 0.1, a.pos, rows=rows)
    assert np.array_equal(sub, full[rows])


def test_thread_count_does_not_change_results():
    q, k, v, a = _inputs(64, 4, 2, 32, 7)
    one = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, 0.1, a.pos, nthreads=1)
    many = oracle.gated_attention_f64(q, k, v, a.key_score, a.gains, 0.1, a.pos, nthreads=5)
    assert np.array_equal(one, many)


# ------------------------------------------------------------------ RoPE

def test_rope_worked_example():
    rows = golden("rope_d4.txt")
    x = np.array([r[:4] for r in rows])[:, None, :]
    want = np.array([r[4:] for r in rows])
    got = oracle.rope_f64_values(x, np.full(len(rows), 100, np.int32), 1.0e4)[:, 0, :]
    assert np.max(np.abs(got - want)) <= 1e-14


def test_rope_properties():
    g = np.random.default_rng(8)
    D, theta = 128, 1.0e6
    x = g.standard_normal((6, 3, D))
    pos = np.array([0, 1, 5, 1000, 65535, 131071], np.int32)
    y = oracle.rope_f64_values(x, pos, theta)
    assert np.array_equal(y[0], x[0])  # position 0: identity
    half = D // 2
    nx = x[..., :half] ** 2 + x[..., half:] ** 2
    ny = y[..., :half] ** 2 + y[..., half:] ** 2
    assert np.max(np.abs(nx - ny)) <= 1e-12  # each half-split pair keeps its length
    # q'_m . k'_n depends only on m - n
    qv = g.standard_normal((1, 1, D))
    kv = g.standard_normal((1, 1, D))

    def dot(m, n):
        a = oracle.rope_f64_values(qv, np.array([m], np.int32), theta)
        b = oracle.rope_f64_values(kv, np.array([n], np.int32), theta)
        return float(np.sum(a * b))
    assert abs(dot(10, 3) - dot(1007, 1000)) <= 1e-9
    assert abs(dot(3, 10) - dot(50, 57)) <= 1e-9


def test_bf16_rounding_matches_torch_on_float32_values():
    g = np.random.default_rng(9)
    x32 = np.concatenate([g.standard_normal(20000).astype(np.float32) * 10,
                          np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0, 1e-39, 3.3e38],
                                   np.float32)])
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)
    # ties to even directly from double (no double rounding through float32)
    v = 1.0 + 2 ** -8 + 2 ** -40  # just above the tie: rounds up
    assert oracle.to_bf16(np.array([v]))[0] == 0x3F81
