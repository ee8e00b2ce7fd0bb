"""Python face of the fp64 CPU oracle (``tg_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library.

Inputs arrive as the raw bytes the GPU also sees (bf16 bit patterns as
``uint16``, float32, int32) and are widened exactly to float64 here; every
step then runs in IEEE double in ``tg_oracle.c``.  Which page passage each
step follows is stated next to each function there and below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tg_oracle.c")
_LIB = os.path.join(_HERE, "libtgoracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", _SRC, "-o", _LIB, "-lm", "-lpthread"]


def build() -> str:
    """Compile the oracle with gcc (plain C, no GPU)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        L.tgo_score_mlp.argtypes = [P, P, P, P, D, I64, I64, I64, D, P, ctypes.c_int]
        L.tgo_score_mlp.restype = None
        L.tgo_seq_rmsnorm.argtypes = [P, I64, D, P]
        L.tgo_seq_rmsnorm.restype = D
        L.tgo_select_topk.argtypes = [P, P, I64, I64, P]
        L.tgo_select_topk.restype = ctypes.c_int
        L.tgo_gather_rows.argtypes = [P, I64, I64, P, I64, P, I64]
        L.tgo_gather_rows.restype = None
        L.tgo_rope.argtypes = [P, P, I64, I64, I64, D, P]
        L.tgo_rope.restype = None
        L.tgo_to_bf16.argtypes = [P, I64, P]
        L.tgo_to_bf16.restype = None
        L.tgo_gated_attention.argtypes = [P, P, P, P, P, D, P, I64, I64, I64, I64, P, I64, P,
                                          ctypes.c_int]
        L.tgo_gated_attention.restype = None
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


# --------------------------------------------------------------- the steps

def score_mlp(resid_bits, w1_bits, b1_bits, w2_bits, b2: float, eps_row: float = 1e-6,
              nthreads: Optional[int] = None) -> np.ndarray:
    """Raw gate scores s [n] (fp64): row RMSNorm, W1, GELU(erf), w2.
    The scoring network of [P1 gate] / [P2 method] / [P5 Fig 1(a)(b)]."""
    h = widen_bf16(resid_bits)
    w1 = widen_bf16(w1_bits)
    w2 = widen_bf16(w2_bits)
    b1 = None if b1_bits is None else widen_bf16(b1_bits)
    n, d = h.shape
    hd = w1.shape[0]
    assert w1.shape == (hd, d) and w2.shape == (hd,)
    s = np.empty(n, dtype=np.float64)
    lib().tgo_score_mlp(_ptr(h), _ptr(w1), _ptr(b1), _ptr(w2), float(b2), n, d, hd,
                        float(eps_row), _ptr(s), nthreads or default_threads())
    return s


def score_mlp_f64(h: np.ndarray, w1: np.ndarray, b1: Optional[np.ndarray], w2: np.ndarray,
                  b2: float, eps_row: float, nthreads: int = 1) -> np.ndarray:
    """Same as score_mlp on float64 arrays (for closed-form checks with any values)."""
    h, w1, w2 = _f64(h), _f64(w1), _f64(w2)
    b1 = None if b1 is None else _f64(b1)
    n, d = h.shape
    hd = w1.shape[0]
    s = np.empty(n, dtype=np.float64)
    lib().tgo_score_mlp(_ptr(h), _ptr(w1), _ptr(b1), _ptr(w2), float(b2), n, d, hd,
                        float(eps_row), _ptr(s), nthreads)
    return s


def seq_rmsnorm(s: np.ndarray, eps_seq: float = 1e-6):
    """Sequence-wise RMSNorm of the scores [P1 gate][P2 method]. Returns (s_hat, rho)."""
    s = _f64(s)
    out = np.empty_like(s)
    rho = lib().tgo_seq_rmsnorm(_ptr(s), s.size, float(eps_seq), _ptr(out))
    return out, rho


def gate_score(resid_bits, w1_bits, b1_bits, w2_bits, b2: float, eps_row: float = 1e-6,
               eps_seq: float = 1e-6, nthreads: Optional[int] = None):
    """Scorer then sequence RMSNorm. Returns (s_hat, s_raw) in fp64."""
    s = score_mlp(resid_bits, w1_bits, b1_bits, w2_bits, b2, eps_row, nthreads)
    s_hat, _ = seq_rmsnorm(s, eps_seq)
    return s_hat, s


def select_topk(score, forced: Optional[np.ndarray], k: int) -> np.ndarray:
    """Forced-keep top-K [P1 gate][P2 method][P3 how]: kept indices, ascending.
    ``score`` may be float32 (selection on the exact float32 values) or float64."""
    s = _f64(score)
    n = s.size
    f = None if forced is None else np.ascontiguousarray(forced, dtype=np.uint8)
    out = np.empty(k, dtype=np.int32)
    rc = lib().tgo_select_topk(_ptr(s), _ptr(f), n, int(k), _ptr(out))
    if rc != 0:
        raise ValueError(f"infeasible budget: n={n} k={k}")
    return out


def gather_rows(src: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Row gather dst[t] = src[idx[t]] (compaction of kept rows, [P1 gate][P3 how])."""
    src = np.ascontiguousarray(src)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    k = idx.size
    row_bytes = src.strides[0] if src.ndim > 1 else src.itemsize
    dst = np.empty((k,) + src.shape[1:], dtype=src.dtype)
    lib().tgo_gather_rows(_ptr(src), row_bytes, row_bytes, _ptr(idx), k, _ptr(dst), row_bytes)
    return dst


def rope_f64(x_bits: np.ndarray, pos: np.ndarray, theta: float = 1.0e6) -> np.ndarray:
    """RoPE at original positions, unrounded fp64 output. x: [rows, heads, D] bf16 bits."""
    x = widen_bf16(x_bits)
    rows, heads, D = x.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    out = np.empty_like(x)
    lib().tgo_rope(_ptr(x), _ptr(pos), rows, heads, D, float(theta), _ptr(out))
    return out


def rope_f64_values(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """RoPE on arbitrary float64 values (for the closed-form checks)."""
    x = _f64(x)
    rows, heads, D = x.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    out = np.empty_like(x)
    lib().tgo_rope(_ptr(x), _ptr(pos), rows, heads, D, float(theta), _ptr(out))
    return out


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 bit patterns, nearest-even, in one step."""
    x = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().tgo_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def rope(x_bits: np.ndarray, pos: np.ndarray, theta: float = 1.0e6) -> np.ndarray:
    """RoPE rounded to bf16 (bit patterns)."""
    return to_bf16(rope_f64(x_bits, pos, theta))


def gated_attention_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, key_score, gains,
                        temp_coef: float, pos, rows: Optional[Sequence[int]] = None,
                        nthreads: Optional[int] = None) -> np.ndarray:
    """Token-gated causal attention over the kept list [P1 tga][P2 method][P3 tga]
    [P5 Fig 1(c)], on float64 arrays q [K,hq,D], k/v [K,hkv,D].
    Returns [K or len(rows), hq, D] float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    K, hq, D = q.shape
    hkv = k.shape[1]
    assert k.shape == (K, hkv, D) and v.shape == (K, hkv, D) and hq % hkv == 0
    ks = _f64(key_score)
    g = _f64(gains)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert ks.shape == (K,) and g.shape == (hq,) and pos.shape == (K,)
    if rows is None:
        out = np.empty((K, hq, D), dtype=np.float64)
        lib().tgo_gated_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(g), float(temp_coef),
                                  _ptr(pos), K, hq, hkv, D, None, 0, _ptr(out),
                                  nthreads or default_threads())
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        assert r.size == 0 or (r.min() >= 0 and r.max() < K)
        out = np.empty((r.size, hq, D), dtype=np.float64)
        lib().tgo_gated_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(g), float(temp_coef),
                                  _ptr(pos), K, hq, hkv, D, _ptr(r), r.size, _ptr(out),
                                  nthreads or default_threads())
    return out


def gated_attention(q_bits, k_bits, v_bits, key_score, gains, temp_coef: float, pos,
                    rows=None, nthreads: Optional[int] = None) -> np.ndarray:
    """Token-gated attention on bf16 inputs (bit patterns), fp64 result."""
    return gated_attention_f64(widen_bf16(q_bits), widen_bf16(k_bits), widen_bf16(v_bits),
                               key_score, gains, temp_coef, pos, rows, nthreads)
