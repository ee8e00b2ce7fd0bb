"""Boundary-gap conditioning of seeded inputs (test infrastructure only).

Parity of the kept set is only meaningful when the K-th and (K+1)-th best
prunable scores are further apart than the scorer's rounding error.  This
helper redraws, from derived substreams, the prunable rows (or raw scores)
whose oracle score lies near the cut until the gap exceeds ``gap`` for every
budget asked for.  It uses the oracle's scores only; the drawing itself lives
in the input generator.
"""
from __future__ import annotations

from typing import Iterable

import numpy as np

from learned_token_pruning_mlp_amd import synth
from . import oracle


def _cut(s_hat: np.ndarray, forced: np.ndarray, k: int):
    """(a, b): the worst kept and best dropped prunable score, or None."""
    prun = np.flatnonzero(forced == 0)
    r = k - int(forced.sum())
    if r <= 0 or r >= prun.size:
        return None
    order = prun[np.lexsort((prun, -s_hat[prun]))]
    return s_hat[order[r - 1]], s_hat[order[r]]


def enforce_gate_gap(inp: synth.GateInputs, seed: int, budgets: Iterable[int], *,
                     gap: float = 1e-3, band: float = 2e-3, eps_row: float = 1e-6,
                     eps_seq: float = 1e-6, max_iter: int = 64):
    """Redraw residual rows in place until every budget has a gap > ``gap``
    in the oracle's normalised scores.  Returns (s_hat, s_raw) of the final inputs."""
    budgets = list(budgets)
    s = oracle.score_mlp(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, eps_row)
    for it in range(max_iter):
        s_hat, _ = oracle.seq_rmsnorm(s, eps_seq)
        bad = []
        for k in budgets:
            c = _cut(s_hat, inp.forced, k)
            if c is not None and c[0] - c[1] <= gap:
                mid = 0.5 * (c[0] + c[1])
                near = np.flatnonzero((np.abs(s_hat - mid) < band) & (inp.forced == 0))
                bad.append(near)
        if not bad:
            return s_hat, s
        rows = np.unique(np.concatenate(bad))
        synth.redraw_rows(inp.resid, rows, seed, it)
        s[rows] = oracle.score_mlp(inp.resid[rows], inp.w1, inp.b1, inp.w2, inp.b2, eps_row)
    raise RuntimeError("boundary gap not reached")


def enforce_score_gap(scores: np.ndarray, forced: np.ndarray, seed: int, budgets: Iterable[int],
                      *, df: float = 3.0, gap: float = 1e-3, band: float = 2e-3,
                      max_iter: int = 64) -> np.ndarray:
    """Same for scores drawn directly (float32), redrawn as Student-t values."""
    budgets = list(budgets)
    for it in range(max_iter):
        s = scores.astype(np.float64)
        bad = []
        for k in budgets:
            c = _cut(s, forced, k)
            if c is not None and c[0] - c[1] <= gap:
                mid = 0.5 * (c[0] + c[1])
                bad.append(np.flatnonzero((np.abs(s - mid) < band) & (forced == 0)))
        if not bad:
            return scores
        synth.redraw_scores(scores, np.unique(np.concatenate(bad)), seed, it, df)
    raise RuntimeError("boundary gap not reached")
