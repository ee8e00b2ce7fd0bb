"""Pins of the attention-backward oracle (oracle/attn_bwd.py).

* Central finite differences of the C forward oracle (an independent
  implementation of the forward) against every analytic gradient, on tiny
  inputs with negative and positive temperatures.
* Shift invariance: adding a constant to every key score adds the same
  per-row constant to the logits, so the output does not change and the
  score gradient sums to zero.
* Each softmax row sums to 1, so the value gradients of a kv head sum to the
  output gradients of its q heads.
"""
import numpy as np
import pytest

from oracle import attn_bwd, oracle


def _case(seed, K=7, hq=4, hkv=2, D=4, c=0.3):
    g = np.random.default_rng(seed)
    q = g.normal(size=(K, hq, D))
    k = g.normal(size=(K, hkv, D))
    v = g.normal(size=(K, hkv, D))
    s = g.normal(size=K)
    gains = g.uniform(0.5, 2.0, size=hq)
    pos = np.sort(g.choice(4 * K, size=K, replace=False)).astype(np.int32)
    dout = g.normal(size=(K, hq, D))
    return q, k, v, s, gains, c, pos, dout


def _loss(q, k, v, s, gains, c, pos, dout):
    return float(np.sum(oracle.gated_attention_f64(q, k, v, s, gains, c, pos, nthreads=1) * dout))


@pytest.mark.parametrize("seed,c", [(1, 0.3), (2, -0.45), (3, 0.0)])
def test_gradients_match_finite_differences(seed, c):
    q, k, v, s, gains, c, pos, dout = _case(seed, c=c)
    out, dq, dk, dv, ds, dg, dc = attn_bwd.gated_attention_grads(q, k, v, s, gains, c, pos, dout)
    np.testing.assert_allclose(out, oracle.gated_attention_f64(q, k, v, s, gains, c, pos, nthreads=1),
                               rtol=1e-12, atol=1e-13)
    eps = 1e-6

    def fd(arr, name):
        grad = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + eps
            lp = _loss(**inputs)
            arr[idx] = a0 - eps
            lm = _loss(**inputs)
            arr[idx] = a0
            grad[idx] = (lp - lm) / (2 * eps)
        return grad

    inputs = dict(q=q, k=k, v=v, s=s, gains=gains, c=c, pos=pos, dout=dout)
    for arr, analytic in ((q, dq), (k, dk), (v, dv), (s, ds), (gains, dg)):
        np.testing.assert_allclose(analytic, fd(arr, ""), rtol=1e-6, atol=1e-8)
    lp = _loss(q, k, v, s, gains, c + eps, pos, dout)
    lm = _loss(q, k, v, s, gains, c - eps, pos, dout)
    assert abs(dc - (lp - lm) / (2 * eps)) <= 1e-6 * max(1.0, abs(dc))


@pytest.mark.parametrize("seed", [4, 5])
def test_score_gradient_sums_to_zero(seed):
    q, k, v, s, gains, c, pos, dout = _case(seed, K=40, hq=4, hkv=1, D=8)
    _, _, _, _, ds, _, _ = attn_bwd.gated_attention_grads(q, k, v, s, gains, c, pos, dout)
    assert abs(ds.sum()) <= 1e-12 * np.abs(ds).sum()
    assert np.abs(ds).sum() > 0.1


def test_value_gradients_sum_to_output_gradients():
    q, k, v, s, gains, c, pos, dout = _case(6, K=33, hq=6, hkv=2, D=8)
    _, _, _, dv, _, _, _ = attn_bwd.gated_attention_grads(q, k, v, s, gains, c, pos, dout)
    G = 3
    for hk in range(2):
        np.testing.assert_allclose(dv[:, hk, :].sum(axis=0), dout[:, hk * G:(hk + 1) * G, :].sum(axis=(0, 1)),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed,c", [(7, 0.3), (8, -0.6)])
def test_dq_rows_match_finite_differences(seed, c):
    """The row-subset query gradient against central finite differences of
    the C forward oracle, row by row (q_t moves only row t's output)."""
    q, k, v, s, gains, c, pos, dout = _case(seed, K=9, c=c)
    rows = np.array([0, 3, 8])
    dq = attn_bwd.gated_attention_dq_rows(q, k, v, s, gains, c, pos, dout, rows)
    eps = 1e-6
    for i, t in enumerate(rows):
        for idx in np.ndindex(q.shape[1:]):
            a0 = q[(t,) + idx]
            q[(t,) + idx] = a0 + eps
            lp = _loss(q, k, v, s, gains, c, pos, dout)
            q[(t,) + idx] = a0 - eps
            lm = _loss(q, k, v, s, gains, c, pos, dout)
            q[(t,) + idx] = a0
            assert abs(dq[(i,) + idx] - (lp - lm) / (2 * eps)) <= 1e-6 * max(1.0, abs(dq[(i,) + idx]))


def test_dq_rows_equal_dense_rows():
    q, k, v, s, gains, c, pos, dout = _case(9, K=50, hq=6, hkv=3, D=8, c=0.2)
    _, dq, _, _, _, _, _ = attn_bwd.gated_attention_grads(q, k, v, s, gains, c, pos, dout)
    rows = np.array([0, 1, 17, 31, 49])
    np.testing.assert_allclose(attn_bwd.gated_attention_dq_rows(q, k, v, s, gains, c, pos, dout, rows), dq[rows],
                               rtol=1e-11, atol=1e-13)
