"""Pins of the gated-delta-rule oracle (oracle/gdn.py).

* The recurrence's final state equals the unrolled product-of-transitions
  form, computed separately.
* Delta-rule retrieval: with alpha = beta = 1 and orthonormal keys, after
  writing (k_i, v_i) the state maps every written k_i to its v_i exactly, so
  a query equal to k_i reads back v_i.
* Pure decay: with beta = 0 nothing is written; the state is the initial one
  times the product of the alphas.
* Linearity in v for a zero initial state (fixed keys and gates).
"""
import numpy as np

from oracle import gdn


def test_recurrence_matches_unrolled_transitions():
    g = np.random.default_rng(1)
    T, dk, dv = 7, 5, 4
    k = g.normal(size=(T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.normal(size=(T, 1, dv))
    q = g.normal(size=(T, 1, dk))
    alpha = g.uniform(0.5, 1.0, size=(T, 1))
    beta = g.uniform(0.0, 1.0, size=(T, 1))
    S0 = g.normal(size=(1, dv, dk))
    _, S = gdn.gated_delta_rule(q, k, v, alpha, beta, S0)
    want = gdn.transition_product_state(k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], S0[0])
    np.testing.assert_allclose(S[0], want, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_are_retrieved_exactly():
    g = np.random.default_rng(2)
    dk, dv, T = 8, 6, 5
    Qm, _ = np.linalg.qr(g.normal(size=(dk, dk)))
    k = Qm[:T][:, None, :]                      # T orthonormal keys
    v = g.normal(size=(T, 1, dv))
    q = k.copy()
    # an earlier value written under key 0 is overwritten by the delta rule
    k2 = np.concatenate([k[:1], k], axis=0)
    v2 = np.concatenate([g.normal(size=(1, 1, dv)), v], axis=0)
    q2 = np.concatenate([q[:1], q], axis=0)
    ones = np.ones((T + 1, 1))
    out, S = gdn.gated_delta_rule(q2, k2, v2, ones, ones)
    for i in range(T):
        np.testing.assert_allclose(S[0] @ k[i, 0], v[i, 0], rtol=1e-12, atol=1e-12)
    # the query at step t (= the key just written) reads back its value
    np.testing.assert_allclose(out[1:, 0], v[:, 0], rtol=1e-12, atol=1e-12)


def test_zero_beta_is_pure_decay():
    g = np.random.default_rng(3)
    T, hk, hv, dk, dv = 6, 2, 4, 5, 3
    q, k = g.normal(size=(T, hk, dk)), g.normal(size=(T, hk, dk))
    v = g.normal(size=(T, hv, dv))
    alpha = g.uniform(0.3, 1.0, size=(T, hv))
    S0 = g.normal(size=(hv, dv, dk))
    out, S = gdn.gated_delta_rule(q, k, v, alpha, np.zeros((T, hv)), S0)
    decay = np.cumprod(alpha, axis=0)
    for h in range(hv):
        np.testing.assert_allclose(S[h], S0[h] * decay[-1, h], rtol=1e-12)
        for t in range(T):
            np.testing.assert_allclose(out[t, h], decay[t, h] * (S0[h] @ q[t, h // 2]), rtol=1e-12, atol=1e-12)


def test_linear_in_values_from_zero_state():
    g = np.random.default_rng(4)
    T, dk, dv = 9, 6, 5
    q, k = g.normal(size=(T, 1, dk)), g.normal(size=(T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    alpha, beta = g.uniform(0.5, 1, size=(T, 1)), g.uniform(0, 1, size=(T, 1))
    va, vb = g.normal(size=(T, 1, dv)), g.normal(size=(T, 1, dv))
    oa, _ = gdn.gated_delta_rule(q, k, va, alpha, beta)
    ob, _ = gdn.gated_delta_rule(q, k, vb, alpha, beta)
    oc, _ = gdn.gated_delta_rule(q, k, 2.0 * va - 3.0 * vb, alpha, beta)
    np.testing.assert_allclose(oc, 2.0 * oa - 3.0 * ob, rtol=1e-10, atol=1e-10)
