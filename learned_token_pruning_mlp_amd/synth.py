"""Seeded synthetic inputs for the gated-prefill path.

This module only draws numbers: it holds none of the method's arithmetic
(no normalisation, no scoring, no selection, no attention).  Both the fp64
oracle tests and the HIP path read their inputs from here, so the two sides
see the same bytes.

Every tensor comes from its own PCG64 stream, keyed by (seed, tag), so a
tensor does not change when another one is added or drawn in another order.
Floating-point tensors are drawn in float32 and rounded to bfloat16 by
round-to-nearest-even; they are handed out as raw ``uint16`` bit patterns.

Shapes and distributions follow the workloads of the path (Qwen3-1.7B-shaped
gate layer: d_model 2048, 16 q heads / 8 kv heads, head_dim 128, scorer MLP
2048->256->1; sequence lengths 16k/32k/128k as in the long-context results of
the TokenGate pages).  The pages evaluate on task datasets (RepoBench-P,
2WikiMultihopQA, MultiNews, BioDEX, NIAH) that are not used here: seeded
synthetic tensors of the same shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Stream tags: one independent PCG64 stream per tensor.
TAG_RESID = 1
TAG_W1 = 2
TAG_W2 = 3
TAG_B1 = 4
TAG_GAINS = 5
TAG_Q = 6
TAG_K = 7
TAG_V = 8
TAG_FORCED = 9
TAG_SCORES = 10
TAG_ROWS = 11
TAG_REDRAW = 1000  # + iteration number


def stream(seed: int, tag: int) -> np.random.Generator:
    """Independent PCG64 generator for (seed, tag)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag)])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return the
    16-bit patterns.  Inputs are finite draws, so no NaN special case."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for building inputs)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tag: int, shape, std: float = 1.0) -> np.ndarray:
    g = stream(seed, tag)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return f32_to_bf16_bits(x)


@dataclasses.dataclass(frozen=True)
class GateShape:
    """Sizes of one gate layer and the upper-layer attention that follows it."""
    n: int            # tokens in the prompt
    d: int            # d_model
    hd: int           # scorer hidden width
    n_forced: int     # forced-keep (question) tokens
    k: int            # total kept budget, forced tokens included
    hq: int           # query heads
    hkv: int          # key/value heads
    head_dim: int
    rope_theta: float = 1.0e6
    temp_coef: float = 0.1
    forced_layout: str = "tail"    # "tail": last F tokens; "scatter_tail": F drawn from the last 1024


# The workloads of the path, named by what they are.
TINY = GateShape(n=512, d=256, hd=64, n_forced=32, k=128, hq=4, hkv=2, head_dim=64)
QWEN3_1P7B_N16K = GateShape(n=16384, d=2048, hd=256, n_forced=64, k=2048, hq=16, hkv=8, head_dim=128)
QWEN3_1P7B_N32K = GateShape(n=32768, d=2048, hd=256, n_forced=64, k=4096, hq=16, hkv=8, head_dim=128)
QWEN3_1P7B_N128K = GateShape(n=131072, d=2048, hd=256, n_forced=128, k=8192, hq=16, hkv=8, head_dim=128,
                             forced_layout="scatter_tail")
N32K_BUDGETS = (1024, 4096, 8192)
N128K_UPPER_LAYERS = 26


@dataclasses.dataclass
class GateInputs:
    resid: np.ndarray          # [n, d] uint16 (bf16 bits), post-attention residual at the gate layer
    w1: np.ndarray             # [hd, d] uint16, norm weight already folded in
    b1: Optional[np.ndarray]   # [hd] uint16 or None
    w2: np.ndarray             # [hd] uint16
    b2: float
    forced: np.ndarray         # [n] uint8, 1 = never pruned
    pos: np.ndarray            # [n] int32 original position ids


def forced_mask(shape: GateShape, seed: int) -> np.ndarray:
    m = np.zeros(shape.n, dtype=np.uint8)
    f = shape.n_forced
    if f == 0:
        return m
    if shape.forced_layout == "tail":
        m[shape.n - f:] = 1
    elif shape.forced_layout == "scatter_tail":
        window = min(1024, shape.n)
        g = stream(seed, TAG_FORCED)
        pick = g.choice(window, size=f, replace=False)
        m[shape.n - window + pick] = 1
    else:
        raise ValueError(shape.forced_layout)
    return m


def gate_inputs(shape: GateShape, seed: int, *, w1_zero: bool = False,
                w_std: float = 0.02, with_b1: bool = False) -> GateInputs:
    """Residual ~ N(0,1), scorer weights ~ N(0, w_std), biases zero unless asked."""
    resid = normal_bf16(seed, TAG_RESID, (shape.n, shape.d))
    if w1_zero:
        w1 = np.zeros((shape.hd, shape.d), dtype=np.uint16)
    else:
        w1 = normal_bf16(seed, TAG_W1, (shape.hd, shape.d), w_std)
    w2 = normal_bf16(seed, TAG_W2, (shape.hd,), w_std)
    b1 = normal_bf16(seed, TAG_B1, (shape.hd,), 0.5) if with_b1 else None
    return GateInputs(resid=resid, w1=w1, b1=b1, w2=w2, b2=0.0,
                      forced=forced_mask(shape, seed),
                      pos=np.arange(shape.n, dtype=np.int32))


def redraw_rows(resid: np.ndarray, rows: np.ndarray, seed: int, iteration: int) -> None:
    """Replace the given residual rows, in place, by fresh N(0,1) bf16 draws
    from a substream derived from (seed, iteration).  Deterministic."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return
    g = stream(seed, TAG_REDRAW + int(iteration))
    x = g.standard_normal(size=(rows.size, resid.shape[1]), dtype=np.float32)
    resid[rows] = f32_to_bf16_bits(x)


def redraw_scores(scores: np.ndarray, idx: np.ndarray, seed: int, iteration: int, df: float) -> None:
    """Replace the given raw scores, in place, by fresh Student-t draws."""
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return
    g = stream(seed, TAG_REDRAW + int(iteration))
    scores[idx] = g.standard_t(df, size=idx.size).astype(np.float32)


def student_t_scores(n: int, seed: int, df: float = 3.0) -> np.ndarray:
    """Heavy-tailed importance scores (float32), drawn directly."""
    return stream(seed, TAG_SCORES).standard_t(df, size=n).astype(np.float32)


def gains(hq: int, seed: int, lo: float = 0.5, hi: float = 2.0, tag_offset: int = 0) -> np.ndarray:
    return stream(seed, TAG_GAINS + 100 * tag_offset).uniform(lo, hi, size=hq).astype(np.float32)


@dataclasses.dataclass
class AttnInputs:
    q: np.ndarray          # [k, hq, D] uint16
    k: np.ndarray          # [k, hkv, D] uint16
    v: np.ndarray          # [k, hkv, D] uint16
    key_score: np.ndarray  # [k] float32 (normalised importance of each kept key)
    gains: np.ndarray      # [hq] float32
    temp_coef: float
    pos: np.ndarray        # [k] int32, strictly increasing original positions


def attn_inputs(k: int, hq: int, hkv: int, head_dim: int, seed: int, *,
                pos: Optional[np.ndarray] = None, key_score: Optional[np.ndarray] = None,
                temp_coef: float = 0.1, layer: int = 0) -> AttnInputs:
    """Q/K/V of the kept rows ~ N(0,1) bf16; gains ~ U(0.5, 2).

    ``pos`` defaults to a sorted draw of k distinct positions out of 4k (a
    pruned prompt); ``key_score`` defaults to N(0,1) float32."""
    base = 10 * layer
    q = normal_bf16(seed, TAG_Q + base * 1000, (k, hq, head_dim))
    kk = normal_bf16(seed, TAG_K + base * 1000, (k, hkv, head_dim))
    v = normal_bf16(seed, TAG_V + base * 1000, (k, hkv, head_dim))
    if pos is None:
        g = stream(seed, TAG_ROWS)
        pos = np.sort(g.choice(4 * k, size=k, replace=False)).astype(np.int32)
    if key_score is None:
        key_score = stream(seed, TAG_SCORES + 7).standard_normal(size=k).astype(np.float32)
    return AttnInputs(q=q, k=kk, v=v, key_score=np.ascontiguousarray(key_score, dtype=np.float32),
                      gains=gains(hq, seed, tag_offset=layer), temp_coef=float(temp_coef),
                      pos=np.ascontiguousarray(pos, dtype=np.int32))
