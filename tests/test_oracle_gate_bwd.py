"""Pins of the scorer-backward oracle (oracle/gate_bwd.py).

* Central finite differences of the C forward oracle (scorer, then the
  sequence RMSNorm; an independent implementation of the forward) against
  every analytic gradient, with dshat nonzero only on a kept subset.
* Row-norm scale invariance: with eps_row = 0 a token's score depends on its
  residual only through h_i / |h_i|, so each row's gradient is orthogonal to
  the row: sum_k dh_ik h_ik = 0.
* Sequence-norm scale invariance: with eps_seq = 0, scaling w2 and b2
  together leaves shat unchanged, so sum_j dw2_j w2_j + db2 b2 = 0.
"""
import numpy as np
import pytest

from oracle import gate_bwd, oracle


def _case(seed, n=6, d=8, hd=5):
    g = np.random.default_rng(seed)
    h = g.normal(size=(n, d))
    w1 = g.normal(size=(hd, d)) * 0.5
    b1 = g.normal(size=hd) * 0.3
    w2 = g.normal(size=hd)
    b2 = 0.2
    kept = np.sort(g.choice(n, size=max(1, n // 2), replace=False))
    dshat = gate_bwd.scatter_kept(n, kept, g.normal(size=kept.size))
    return h, w1, b1, w2, b2, dshat


def _loss(h, w1, b1, w2, b2, eps_row, eps_seq, dshat):
    s = oracle.score_mlp_f64(h, w1, b1, w2, b2, eps_row, nthreads=1)
    shat, _ = oracle.seq_rmsnorm(s, eps_seq)
    return float(np.dot(shat, dshat))


@pytest.mark.parametrize("seed,eps_row,eps_seq", [(1, 1e-6, 1e-6), (2, 0.3, 0.5), (3, 0.0, 0.0)])
def test_gradients_match_finite_differences(seed, eps_row, eps_seq):
    h, w1, b1, w2, b2, dshat = _case(seed)
    dh, dw1, db1, dw2, db2 = gate_bwd.gate_score_grads(h, w1, b1, w2, b2, eps_row, eps_seq, dshat)
    eps = 1e-6
    args = dict(h=h, w1=w1, b1=b1, w2=w2)

    def fd(name):
        arr = args[name]
        grad = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + eps
            lp = _loss(h, w1, b1, w2, b2, eps_row, eps_seq, dshat)
            arr[idx] = a0 - eps
            lm = _loss(h, w1, b1, w2, b2, eps_row, eps_seq, dshat)
            arr[idx] = a0
            grad[idx] = (lp - lm) / (2 * eps)
        return grad

    for name, analytic in (("h", dh), ("w1", dw1), ("b1", db1), ("w2", dw2)):
        np.testing.assert_allclose(analytic, fd(name), rtol=1e-6, atol=1e-8, err_msg=name)
    lp = _loss(h, w1, b1, w2, b2 + eps, eps_row, eps_seq, dshat)
    lm = _loss(h, w1, b1, w2, b2 - eps, eps_row, eps_seq, dshat)
    assert abs(db2 - (lp - lm) / (2 * eps)) <= 1e-6 * max(1.0, abs(db2))


def test_residual_gradient_orthogonal_to_row_without_eps():
    h, w1, b1, w2, b2, dshat = _case(4, n=20, d=16, hd=8)
    dh, *_ = gate_bwd.gate_score_grads(h, w1, b1, w2, b2, 0.0, 1e-6, dshat)
    dots = np.sum(dh * h, axis=1)
    assert np.max(np.abs(dots)) <= 1e-12 * np.max(np.abs(dh)) * np.max(np.abs(h)) * h.shape[1]
    assert np.max(np.abs(dh)) > 1e-3


def test_output_layer_scale_invariance_without_eps():
    h, w1, b1, w2, b2, dshat = _case(5, n=30, d=12, hd=6)
    _, _, _, dw2, db2 = gate_bwd.gate_score_grads(h, w1, b1, w2, b2, 1e-6, 0.0, dshat)
    assert abs(np.dot(dw2, w2) + db2 * b2) <= 1e-12 * (np.abs(dw2).sum() + abs(db2))
    assert np.abs(dw2).sum() > 1e-3
