"""Pins of the oracle's scorer and sequence RMSNorm (CPU only).

Each check ties the oracle to something other than itself: a pure-Python
brute force, torch's own rms_norm/linear/gelu in fp64, textbook normal-CDF
values, hand-worked closed forms and exact invariances.
"""
import math

import numpy as np
import pytest
import torch

import brute
from conftest import golden
from learned_token_pruning_mlp_amd import synth
from oracle import oracle


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def test_scorer_matches_bruteforce():
    n, d, hd = 12, 16, 8
    h = _rand((n, d), 1)
    w1 = _rand((hd, d), 2, 0.3)
    b1 = _rand((hd,), 3, 0.5)
    w2 = _rand((hd,), 4, 0.7)
    ref = brute.scores(h.tolist(), w1.tolist(), b1.tolist(), w2.tolist(), 0.25, 1e-6)
    got = oracle.score_mlp_f64(h, w1, b1, w2, 0.25, 1e-6)
    assert np.max(np.abs(got - np.array(ref))) <= 1e-12


def test_scorer_matches_torch_fp64_library_composition():
    # tiny workload shape: 512 tokens, d=256, hidden 64
    shp = synth.TINY
    inp = synth.gate_inputs(shp, seed=1, with_b1=True)
    got = oracle.score_mlp(inp.resid, inp.w1, inp.b1, inp.w2, 0.125, 1e-6)
    h = torch.from_numpy(oracle.widen_bf16(inp.resid))
    w1 = torch.from_numpy(oracle.widen_bf16(inp.w1))
    b1 = torch.from_numpy(oracle.widen_bf16(inp.b1))
    w2 = torch.from_numpy(oracle.widen_bf16(inp.w2))
    x = torch.nn.functional.rms_norm(h, (shp.d,), eps=1e-6)
    a = torch.nn.functional.linear(x, w1, b1)
    u = torch.nn.functional.gelu(a, approximate="none")
    ref = torch.nn.functional.linear(u, w2[None, :]).squeeze(1) + 0.125
    assert np.max(np.abs(got - ref.numpy())) <= 1e-10


@pytest.mark.parametrize("row", golden("normal_cdf.txt"))
def test_gelu_textbook_values(row):
    # one input, one hidden unit, W1 = 0: a = b1, s = w2 * GELU(b1)
    x, phi = row
    for sign in (1.0, -1.0):
        a = sign * x
        want = a * phi if sign > 0 else a * (1.0 - phi)
        s = oracle.score_mlp_f64(np.ones((1, 1)), np.zeros((1, 1)), np.array([a]), np.ones(1), 0.0, 0.0)
        assert abs(s[0] - want) <= 1e-14


def test_gelu_identities():
    xs = np.linspace(-4, 4, 33)
    n = xs.size
    s_pos = oracle.score_mlp_f64(np.ones((n, 1)), np.zeros((1, 1)), None, np.ones(1), 0.0, 0.0)
    assert np.all(s_pos == 0.0)  # GELU(0) = 0, no bias
    for x in xs:
        p = oracle.score_mlp_f64(np.ones((1, 1)), np.zeros((1, 1)), np.array([x]), np.ones(1), 0.0, 0.0)[0]
        m = oracle.score_mlp_f64(np.ones((1, 1)), np.zeros((1, 1)), np.array([-x]), np.ones(1), 0.0, 0.0)[0]
        assert abs((p - m) - x) <= 1e-14  # GELU(x) - GELU(-x) = x


def test_row_rms_normalisation_value():
    # h = (2,2,2,2): mean square 4, r = 1/2; W1 row = x/4 each, dot = 2x, a = x.
    for x, phi in golden("normal_cdf.txt"):
        h = np.full((1, 4), 2.0)
        w1 = np.full((1, 4), x / 4.0)
        s = oracle.score_mlp_f64(h, w1, None, np.ones(1), 0.0, 0.0)[0]
        assert abs(s - x * phi) <= 1e-14


def test_w1_zero_closed_form():
    # W1 = 0: every token gets sum_j w2_j GELU(b1_j) + b2, whatever its residual
    pts = golden("normal_cdf.txt")
    b1 = np.array([p[0] for p in pts] + [-p[0] for p in pts] + [0.0])
    cdf = np.array([p[1] for p in pts] + [1.0 - p[1] for p in pts] + [0.5])
    w2 = _rand(b1.shape, 5)
    want = float(np.sum(w2 * b1 * cdf)) + 0.75
    h = _rand((9, 32), 6)
    s = oracle.score_mlp_f64(h, np.zeros((b1.size, 32)), b1, w2, 0.75, 1e-6)
    assert np.max(np.abs(s - want)) <= 1e-13


def test_row_scale_invariance():
    h = _rand((7, 64), 7)
    w1 = _rand((16, 64), 8, 0.2)
    w2 = _rand((16,), 9)
    s0 = oracle.score_mlp_f64(h, w1, None, w2, 0.0, 0.0)
    for alpha in (2.0, 0.5, 1024.0):  # powers of two scale exactly
        s1 = oracle.score_mlp_f64(alpha * h, w1, None, w2, 0.0, 0.0)
        assert np.array_equal(s0, s1)
    s3 = oracle.score_mlp_f64(3.0 * h, w1, None, w2, 0.0, 0.0)
    assert np.max(np.abs(s3 - s0)) <= 1e-12


def test_seq_rmsnorm_worked_example():
    rows = golden("seqnorm_worked.txt")
    s = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows])
    got, rho = oracle.seq_rmsnorm(s, 0.0)
    assert np.max(np.abs(got - want)) <= 1e-15
    assert abs(rho - 5.0 / math.sqrt(2.0)) <= 1e-15


def test_seq_rmsnorm_mean_square_closed_form():
    s = _rand((1000,), 10, 0.01)
    for eps in (0.0, 1e-6, 1e-3):
        got, _ = oracle.seq_rmsnorm(s, eps)
        m = np.mean(s * s)
        assert abs(np.mean(got * got) - m / (m + eps)) <= 1e-14
        assert np.all(np.sign(got) == np.sign(s))
        # ratios are kept, so the order is kept
        assert np.max(np.abs(got[1:] / got[:-1] - s[1:] / s[:-1])) <= 1e-9


def test_seq_rmsnorm_uses_every_token():
    # the forced-keep tail enters the mean: changing it changes rho
    s = _rand((100,), 11)
    a, _ = oracle.seq_rmsnorm(s, 1e-6)
    s2 = s.copy()
    s2[-10:] *= 3.0
    b, _ = oracle.seq_rmsnorm(s2, 1e-6)
    assert not np.allclose(a[:90], b[:90])
    assert np.allclose(a[:90] / b[:90], np.sqrt(np.mean(s2 ** 2) + 1e-6) / np.sqrt(np.mean(s ** 2) + 1e-6))
