"""fp64 CPU oracle of an upper decoder layer on the kept rows.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library.

Above the gate layer only the kept tokens pass through the backbone's
layers, with their original positions (fluxbbs.com TokenGate article,
section on where the gate sits; aiwillknow.com, Figure 1(a)(b)).  The pages
name the backbone (Qwen3) but do not describe its layer internals, so the
layer here is the Qwen3 decoder layer as that architecture is publicly
specified -- a reading, not a page's statement (parity unpinned against the
pages for the layer internals; the tests pin each piece to closed forms and
invariants, and the attention inside it is the pinned token-gated attention
of ``oracle.py``):

    x  = rmsnorm(h, w_in)
    q  = x Wq^T, k = x Wk^T, v = x Wv^T          (per-head layouts [rows, H, D])
    q  = rmsnorm_per_head(q, w_qn), k = rmsnorm_per_head(k, w_kn)
    q, k = RoPE at the original positions (theta)
    a  = token-gated attention(q, k, v, key_score, gains, c, pos)
    h2 = a Wo^T + h
    x2 = rmsnorm(h2, w_post)
    h3 = swiglu(x2 Wgu^T) Wdown^T + h2          (Wgu = [W_gate; W_up])

Every step is exact IEEE double.  ``round_to`` (optional) is applied to each
tensor the GPU path stores between its launches (bf16 storage of the
activations, the precision the pages run the model in), so a test can ask
for the same storage points; None keeps everything in fp64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from . import oracle


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean over the last axis of x^2 + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x), written as x / (1 + e^-x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu(gate_up: np.ndarray) -> np.ndarray:
    """silu(g) * u, with g and u the first and second halves of each row."""
    gu = np.asarray(gate_up, dtype=np.float64)
    inter = gu.shape[-1] // 2
    return silu(gu[..., :inter]) * gu[..., inter:]


def linear(x: np.ndarray, w: np.ndarray, residual: Optional[np.ndarray] = None) -> np.ndarray:
    """x W^T (+ residual), W in the [out, in] layout."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    return y if residual is None else y + np.asarray(residual, dtype=np.float64)


@dataclass
class LayerWeights:
    """Weights of one decoder layer as float64 arrays (values of bf16 weights)."""
    w_in: np.ndarray     # [d]
    wq: np.ndarray       # [hq*D, d]
    wk: np.ndarray       # [hkv*D, d]
    wv: np.ndarray       # [hkv*D, d]
    w_qn: np.ndarray     # [D]
    w_kn: np.ndarray     # [D]
    wo: np.ndarray       # [d, hq*D]
    w_post: np.ndarray   # [d]
    wgu: np.ndarray      # [2*inter, d]
    wdown: np.ndarray    # [d, inter]


def decoder_layer(h: np.ndarray, W: LayerWeights, pos: np.ndarray, key_score: np.ndarray, gains: np.ndarray,
                  temp_coef: float, hq: int, hkv: int, head_dim: int, theta: float = 1.0e6, eps: float = 1e-6,
                  round_to: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> np.ndarray:
    """One upper layer on the rows h [rows, d] (the kept tokens, in order)."""
    r = round_to if round_to is not None else (lambda a: np.asarray(a, dtype=np.float64))
    h = np.asarray(h, dtype=np.float64)
    rows = h.shape[0]
    D = head_dim
    x = r(rmsnorm(h, W.w_in, eps))
    q = r(linear(x, W.wq)).reshape(rows, hq, D)
    k = r(linear(x, W.wk)).reshape(rows, hkv, D)
    v = r(linear(x, W.wv)).reshape(rows, hkv, D)
    q = r(rmsnorm(q, W.w_qn, eps))
    k = r(rmsnorm(k, W.w_kn, eps))
    q = r(oracle.rope_f64_values(q, pos, theta))
    k = r(oracle.rope_f64_values(k, pos, theta))
    a = r(oracle.gated_attention_f64(q, k, v, key_score, gains, temp_coef, pos))
    h2 = r(linear(a.reshape(rows, hq * D), W.wo, h))
    x2 = r(rmsnorm(h2, W.w_post, eps))
    act = r(swiglu(r(linear(x2, W.wgu))))
    return r(linear(act, W.wdown, h2))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest-even) and widen back to float64."""
    return oracle.widen_bf16(oracle.to_bf16(a))
