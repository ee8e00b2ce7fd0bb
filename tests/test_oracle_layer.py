"""Pins of the upper-layer oracle (oracle/layer.py) against closed forms and invariants.

The layer internals (Qwen3 decoder layer) are not described by the pages, so
these checks pin each piece to what the mathematics fixes: RMSNorm's scale
invariance and unit mean square, SiLU's odd part and limits, linearity of the
projections, and the layer's residual structure (zero output projections give
the identity; zero values take the attention branch out).
"""
import numpy as np
import pytest

from oracle import layer, oracle


def test_rmsnorm_scale_invariance_and_unit_mean_square():
    g = np.random.default_rng(1)
    x = g.normal(size=(7, 64))
    w = np.ones(64)
    y = layer.rmsnorm(x, w, 0.0)
    # mean square of every output row is exactly 1 with eps = 0
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    # scaling a row by alpha > 0 leaves its output unchanged
    alpha = g.uniform(0.1, 10.0, size=(7, 1))
    np.testing.assert_allclose(layer.rmsnorm(alpha * x, w, 0.0), y, rtol=1e-13, atol=1e-15)
    # with eps the mean square is m / (m + eps), m the input's mean square
    eps = 0.3
    m = np.mean(x * x, axis=-1)
    ye = layer.rmsnorm(x, w, eps)
    np.testing.assert_allclose(np.mean(ye * ye, axis=-1), m / (m + eps), rtol=1e-13)


def test_rmsnorm_constant_row_and_weight():
    # a constant row c*1 maps to sign(c) * w * sqrt(c^2 / (c^2 + eps))
    w = np.linspace(-2.0, 3.0, 16)
    for c in (-3.0, 0.5, 7.0):
        y = layer.rmsnorm(np.full((1, 16), c), w, 1e-2)
        np.testing.assert_allclose(y[0], np.sign(c) * w * np.sqrt(c * c / (c * c + 1e-2)), rtol=1e-14)


def test_silu_and_swiglu_closed_forms():
    x = np.linspace(-30.0, 30.0, 601)
    s = layer.silu(x)
    assert layer.silu(np.array([0.0]))[0] == 0.0
    # silu(x) - silu(-x) = x  (x sigmoid(x) + x sigmoid(x) - x ... = x)
    np.testing.assert_allclose(s - layer.silu(-x), x, rtol=1e-13, atol=1e-13)
    # large |x|: silu(x) -> x for x -> +inf and -> 0 for x -> -inf
    assert abs(layer.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(layer.silu(np.array([-40.0]))[0]) < 1e-15
    # swiglu with u = 1 is silu(g); with u = 0 it is 0
    g = np.random.default_rng(2).normal(size=(5, 8))
    np.testing.assert_array_equal(layer.swiglu(np.concatenate([g, np.ones_like(g)], -1)), layer.silu(g))
    assert not layer.swiglu(np.concatenate([g, np.zeros_like(g)], -1)).any()


def test_linear_identity_and_linearity():
    g = np.random.default_rng(3)
    x = g.normal(size=(6, 10))
    np.testing.assert_array_equal(layer.linear(x, np.eye(10)), x)
    w = g.normal(size=(4, 10))
    r = g.normal(size=(6, 4))
    y1 = layer.linear(x, w)
    np.testing.assert_allclose(layer.linear(2.0 * x, w), 2.0 * y1, rtol=1e-14)
    np.testing.assert_allclose(layer.linear(x, w, r), y1 + r, rtol=1e-14)


def _weights(g, d, hq, hkv, D, inter, scale=0.05):
    n = lambda *s: g.normal(size=s) * scale  # noqa: E731
    return layer.LayerWeights(w_in=1.0 + 0.1 * g.normal(size=d), wq=n(hq * D, d), wk=n(hkv * D, d),
                              wv=n(hkv * D, d), w_qn=1.0 + 0.1 * g.normal(size=D), w_kn=1.0 + 0.1 * g.normal(size=D),
                              wo=n(d, hq * D), w_post=1.0 + 0.1 * g.normal(size=d), wgu=n(2 * inter, d),
                              wdown=n(d, inter))


@pytest.mark.parametrize("rows", [1, 9, 40])
def test_layer_residual_structure(rows):
    g = np.random.default_rng(4 + rows)
    d, hq, hkv, D, inter = 32, 4, 2, 16, 48
    W = _weights(g, d, hq, hkv, D, inter)
    h = g.normal(size=(rows, d))
    pos = np.sort(g.choice(4 * rows + 8, size=rows, replace=False)).astype(np.int32)
    ks = g.normal(size=rows)
    gains = g.uniform(0.5, 2.0, size=hq)
    # zero output projections: the layer is the identity on its input rows
    W0 = layer.LayerWeights(**{**W.__dict__, "wo": np.zeros_like(W.wo), "wdown": np.zeros_like(W.wdown)})
    np.testing.assert_array_equal(layer.decoder_layer(h, W0, pos, ks, gains, 0.1, hq, hkv, D), h)
    # zero value projection: the attention branch adds nothing, so the layer is
    # h + MLP(rmsnorm(h)) whatever the queries, keys, scores and gains are
    Wv = layer.LayerWeights(**{**W.__dict__, "wv": np.zeros_like(W.wv)})
    out = layer.decoder_layer(h, Wv, pos, ks, gains, 0.1, hq, hkv, D)
    mlp = layer.linear(layer.swiglu(layer.linear(layer.rmsnorm(h, W.w_post, 1e-6), W.wgu)), W.wdown)
    np.testing.assert_allclose(out, h + mlp, rtol=1e-12, atol=1e-12)
    other = layer.decoder_layer(h, Wv, pos, g.normal(size=rows), 3.0 * gains, -0.2, hq, hkv, D)
    np.testing.assert_array_equal(out, other)


def test_layer_storage_rounding_is_close_to_exact():
    # rounding the stored activations to bf16 moves the layer's output by about
    # the bf16 step of its largest terms, not more
    g = np.random.default_rng(9)
    rows, d, hq, hkv, D, inter = 24, 32, 4, 2, 16, 48
    W = _weights(g, d, hq, hkv, D, inter)
    h = oracle.widen_bf16(oracle.to_bf16(g.normal(size=(rows, d))))
    pos = np.arange(rows, dtype=np.int32) * 3
    ks = g.normal(size=rows)
    gains = g.uniform(0.5, 2.0, size=hq)
    exact = layer.decoder_layer(h, W, pos, ks, gains, 0.1, hq, hkv, D)
    stored = layer.decoder_layer(h, W, pos, ks, gains, 0.1, hq, hkv, D, round_to=layer.bf16_round)
    assert np.max(np.abs(stored - exact)) <= 4 * 2.0 ** -8 * np.max(np.abs(exact))
    assert np.any(stored != exact)
