"""fp64 CPU oracle of the backward of token-gated attention.

TEST INFRASTRUCTURE ONLY: imported by the tests and the CPU-baseline leg of
the benchmark, never by the product path; it shares no code with the HIP
library.

The forward is the token-gated attention of ``oracle.py`` (fluxbbs.com
TokenGate article, section on token-gated attention; slinene.github.io
digest, method key points; news.farwalk.ai, "What is token-gated
attention?"; aiwillknow.com, Figure 1(c)).  The gate is trained through it:
the key-importance bias and the gains exist so that the scores receive a
gradient from the upper layers' attention (fluxbbs.com article, same
section).  For q head h (kv head h // G), query row t and keys j <= t:

    U_tj = q_t . k_j / sqrt(D) + g_h s_j,  Z_tj = lambda_t U_tj,
    P_t  = softmax_j(Z_t),  O_t = sum_j P_tj v_j,
    lambda_t = 1 + c ln((t + 1) / (pos_t + 1)).

Given dO, reverse-mode differentiation of these definitions gives

    dP_tj = dO_t . v_j,   D_t = dO_t . O_t,   dZ_tj = P_tj (dP_tj - D_t),
    dU_tj = lambda_t dZ_tj,   dlambda_t = sum_j dZ_tj U_tj,
    dq_t = sum_j dU_tj k_j / sqrt(D),   dk_j = sum_{h in group, t} dU_tj q_t / sqrt(D),
    dv_j = sum_{h in group, t} P_tj dO_t,   ds_j = sum_h g_h sum_t dU_tj,
    dg_h = sum_{t, j} dU_tj s_j,   dc = sum_{h, t} dlambda_t ln((t + 1) / (pos_t + 1)).

Each is written out below on dense [K, K] matrices per head (plain numpy,
fp64); the tests pin them to central finite differences of the C forward
oracle and to two exact invariants.
"""
from __future__ import annotations

import numpy as np


def gated_attention_grads(q, k, v, key_score, gains, temp_coef: float, pos, dout):
    """Returns (out, dq, dk, dv, dscore, dgains, dtemp) in float64.
    q, dout [K, hq, D]; k, v [K, hkv, D]; key_score [K]; gains [hq]; pos [K]."""
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    s = np.asarray(key_score, dtype=np.float64)
    g = np.asarray(gains, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    K, hq, D = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    t = np.arange(K, dtype=np.float64)
    logratio = np.log((t + 1.0) / (pos + 1.0))
    lam = 1.0 + float(temp_coef) * logratio
    causal = np.tril(np.ones((K, K), dtype=bool))
    rs = 1.0 / np.sqrt(D)
    out = np.zeros_like(q)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    ds = np.zeros(K)
    dg = np.zeros(hq)
    dc = 0.0
    for h in range(hq):
        hk = h // G
        U = q[:, h, :] @ k[:, hk, :].T * rs + g[h] * s[None, :]
        Z = np.where(causal, lam[:, None] * U, -np.inf)
        Z = Z - Z.max(axis=1, keepdims=True)
        E = np.exp(Z)
        P = E / E.sum(axis=1, keepdims=True)
        O = P @ v[:, hk, :]
        out[:, h, :] = O
        dP = dout[:, h, :] @ v[:, hk, :].T
        Dt = np.sum(dout[:, h, :] * O, axis=1)
        dZ = P * (dP - Dt[:, None])
        dU = lam[:, None] * dZ
        dlam = np.sum(np.where(causal, dZ * U, 0.0), axis=1)
        dq[:, h, :] = dU @ k[:, hk, :] * rs
        dk[:, hk, :] += dU.T @ q[:, h, :] * rs
        dv[:, hk, :] += P.T @ dout[:, h, :]
        ds += g[h] * dU.sum(axis=0)
        dg[h] = np.sum(dU * s[None, :])
        dc += float(np.sum(dlam * logratio))
    return out, dq, dk, dv, ds, dg, dc


def gated_attention_dq_rows(q, k, v, key_score, gains, temp_coef: float, pos, dout, rows):
    """dq for the given query rows only, in float64: every quantity the query
    gradient of row t uses (P_t, dP_t, D_t, dU_t) belongs to row t, so it is
    formed from that row's keys j <= t alone, with the same definitions as
    ``gated_attention_grads``.  Returns dq[rows] as [len(rows), hq, D]."""
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    s = np.asarray(key_score, dtype=np.float64)
    g = np.asarray(gains, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    K, hq, D = q.shape
    G = hq // k.shape[1]
    rs = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, hq, D))
    for i, t in enumerate(rows):
        lam = 1.0 + float(temp_coef) * np.log((t + 1.0) / (pos[t] + 1.0))
        kt, vt, st = k[: t + 1], v[: t + 1], s[: t + 1]
        for h in range(hq):
            hk = h // G
            U = kt[:, hk, :] @ q[t, h, :] * rs + g[h] * st
            Z = lam * U
            E = np.exp(Z - Z.max())
            P = E / E.sum()
            O = P @ vt[:, hk, :]
            dP = vt[:, hk, :] @ dout[t, h, :]
            Dt = float(dout[t, h, :] @ O)
            dU = lam * P * (dP - Dt)
            dq[i, h, :] = dU @ kt[:, hk, :] * rs
    return dq
