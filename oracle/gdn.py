"""fp64 CPU oracle of the gated delta rule, the recurrent mixer of the hybrid
variant.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU leg,
never by the product path; it shares no code with the HIP library.

In the hybrid backbone most layers are Gated-DeltaNet mixers and the gate can
sit after one of them; above the gate the recurrent mixers see only the kept
tokens, while the lower layers' recurrent state has read every token
(fluxbbs.com TokenGate article, section on the hybrid architecture;
aiwillknow.com, section on the two kinds of state in hybrid models;
news.farwalk.ai, "Does it work on hybrid-attention models?").  The pages do
not restate the mixer; it is the gated delta rule of Yang, Kautz and
Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule" (2024):
per head, with a state S in R^{dv x dk},

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,

alpha_t in (0, 1] the decay gate, beta_t in [0, 1] the write strength.  The
sequence here is the kept tokens in order (the pruned ones never enter).
"""
from __future__ import annotations

import numpy as np


def gated_delta_rule(q, k, v, alpha, beta, state0=None):
    """Returns (out [T, hv, dv], state [hv, dv, dk]) in float64.
    q, k [T, hk, dk]; v [T, hv, dv]; alpha, beta [T, hv]; v head h uses q/k
    head h // (hv // hk); state0 [hv, dv, dk] or None (zeros)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hk
    S = np.zeros((hv, dv, dk)) if state0 is None else np.array(state0, dtype=np.float64)
    out = np.zeros((T, hv, dv))
    for t in range(T):
        for h in range(hv):
            kk = k[t, h // grp]
            S[h] = alpha[t, h] * (S[h] - beta[t, h] * np.outer(S[h] @ kk, kk)) + beta[t, h] * np.outer(v[t, h], kk)
            out[t, h] = S[h] @ q[t, h // grp]
    return out, S


def transition_product_state(k, v, alpha, beta, state0):
    """The same final state from the unrolled form (one head):
    S_T = S_0 P_1 ... P_T + sum_t beta_t v_t k_t^T P_{t+1} ... P_T,
    P_t = alpha_t (I - beta_t k_t k_t^T) -- for the tests' cross-check."""
    k, v = np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64)
    T, dk = k.shape
    P = [alpha[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    S = np.asarray(state0, dtype=np.float64).copy()
    for t in range(T):
        S = S @ P[t]
    for t in range(T):
        term = beta[t] * np.outer(v[t], k[t])
        for s in range(t + 1, T):
            term = term @ P[s]
        S = S + term
    return S
