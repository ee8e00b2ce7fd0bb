"""fp64 CPU oracle of the backward of the gate's scoring network.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path;
it shares no code with the HIP library.

The forward is the scorer of ``oracle.py`` / ``tg_oracle.c`` (fluxbbs.com
TokenGate article, section on where the gate sits; slinene.github.io digest,
method key points; aiwillknow.com, Figure 1(a)(b)): for each token i with
residual row h_i and d = len(h_i),

    r_i  = (mean_k h_ik^2 + eps_row)^(-1/2),   z_ij = h_i . W1_j,
    a_ij = r_i z_ij + b1_j,   u_ij = GELU(a_ij) = a_ij Phi(a_ij),
    s_i  = sum_j w2_j u_ij + b2,
    rho  = (mean_i s_i^2 + eps_seq)^(1/2),   shat_i = s_i / rho.

The gate learns through the attention bias on the kept tokens (same
sources, section on token-gated attention), so the incoming gradient is
dshat on the kept tokens and zero elsewhere.  Reverse-mode differentiation:

    ds_i   = dshat_i / rho - s_i (sum_m dshat_m s_m) / (n rho^3)
    dw2_j  = sum_i ds_i u_ij,   db2 = sum_i ds_i
    da_ij  = ds_i w2_j GELU'(a_ij),   GELU'(a) = Phi(a) + a phi(a)
    db1_j  = sum_i da_ij
    dz_ij  = r_i da_ij,   dW1_jk = sum_i dz_ij h_ik
    dh_ik  = sum_j dz_ij W1_jk - (sum_j da_ij z_ij) r_i^3 h_ik / d

written out below with plain numpy in fp64; the tests pin it to central
finite differences of the C forward oracle and to two exact invariants.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def scatter_kept(n: int, kept_idx, dshat_kept) -> np.ndarray:
    """Dense dshat [n]: the kept tokens' gradients at their original indices."""
    out = np.zeros(n, dtype=np.float64)
    out[np.asarray(kept_idx, dtype=np.int64)] = np.asarray(dshat_kept, dtype=np.float64)
    return out


def gate_score_grads(h, w1, b1, w2, b2: float, eps_row: float, eps_seq: float, dshat):
    """Returns (dh [n, d], dw1 [hd, d], db1 [hd], dw2 [hd], db2) in float64.
    h [n, d]; w1 [hd, d]; b1 [hd] or None; w2 [hd]; dshat [n] dense."""
    h = np.asarray(h, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    hd = w1.shape[0]
    b1 = np.zeros(hd) if b1 is None else np.asarray(b1, dtype=np.float64)
    dshat = np.asarray(dshat, dtype=np.float64)
    n, d = h.shape
    r = 1.0 / np.sqrt(np.mean(h * h, axis=1) + eps_row)
    z = h @ w1.T
    a = r[:, None] * z + b1[None, :]
    Phi = 0.5 * (1.0 + erf(a / np.sqrt(2.0)))
    phi = np.exp(-0.5 * a * a) / np.sqrt(2.0 * np.pi)
    u = a * Phi
    s = u @ w2 + float(b2)
    rho = np.sqrt(np.mean(s * s) + eps_seq)
    ds = dshat / rho - s * float(np.dot(dshat, s)) / (n * rho ** 3)
    dw2 = u.T @ ds
    db2 = float(ds.sum())
    da = ds[:, None] * w2[None, :] * (Phi + a * phi)
    db1 = da.sum(axis=0)
    dz = r[:, None] * da
    dw1 = dz.T @ h
    dr = np.sum(da * z, axis=1)
    dh = dz @ w1 - (dr * r ** 3 / d)[:, None] * h
    return dh, dw1, db1, dw2, db2
