"""Thin Python binding of libtokengate.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU; it checks dtypes and shapes, turns the
tensors into device pointers and passes torch's current HIP stream.  Every
step of the path runs in the library's HIP kernels; there is no other code
path.  A missing or unloadable library raises immediately.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtokengate.so")

TG_OK = 0
TG_EINVAL = -1
TG_EUNSUPPORTED = -2
TG_EALIGN = -3
TG_EWORKSPACE = -4
TG_EDEVICE = -5
TG_STATUS_FORCED_MISMATCH = 1
TG_STATUS_FORCED_OVER_K = 2
TG_MAX_GATHER = 16

EXPORTS = ("tg_status_string", "tg_abi_version", "tg_workspace_bytes", "tg_gate_score", "tg_gate_score_noalloc",
           "tg_select_topk", "tg_gate_score_select", "tg_compact", "tg_rope", "tg_rope_qk", "tg_gated_attention",
           "tg_gated_attention_timed",
           "tg_rmsnorm", "tg_swiglu", "tg_blas_create", "tg_blas_destroy", "tg_linear",
           "tg_attention_bwd_workspace_bytes", "tg_gated_attention_bwd", "tg_gate_score_bwd_workspace_bytes",
           "tg_gate_score_bwd", "tg_gated_delta_rule", "tg_gated_delta_rule_workspace_bytes",
           "tg_gated_delta_rule_chunked")


class TgGather(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("row_bytes", ctypes.c_int64),
                ("src_stride", ctypes.c_int64), ("dst_stride", ctypes.c_int64)]


class TokenGateError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


_lib = None


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m learned_token_pruning_mlp_amd.build`")
    L = ctypes.CDLL(path)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.tg_status_string.argtypes = [ctypes.c_int]
    L.tg_status_string.restype = ctypes.c_char_p
    L.tg_abi_version.argtypes = []
    L.tg_abi_version.restype = ctypes.c_int
    L.tg_workspace_bytes.argtypes = [I64]
    L.tg_workspace_bytes.restype = ctypes.c_size_t
    L.tg_gate_score.argtypes = [P, P, P, P, F, I64, I32, I32, F, F, P, P, P, ctypes.c_size_t, P]
    L.tg_gate_score.restype = ctypes.c_int
    L.tg_gate_score_noalloc.argtypes = [P, P, P, P, F, I64, I32, I32, F, F, P, P, P]
    L.tg_gate_score_noalloc.restype = ctypes.c_int
    L.tg_select_topk.argtypes = [P, P, I64, I64, I64, P, P, P, ctypes.c_size_t, P]
    L.tg_select_topk.restype = ctypes.c_int
    L.tg_gate_score_select.argtypes = [P, P, P, P, F, I64, I32, I32, F, F, P, I64, I64, P, P, P, P, P,
                                       ctypes.c_size_t, P]
    L.tg_gate_score_select.restype = ctypes.c_int
    L.tg_compact.argtypes = [P, I64, I64, P, P, I32, P, P, P, P, P, I32, P]
    L.tg_compact.restype = ctypes.c_int
    L.tg_rope.argtypes = [P, P, I64, I32, I32, ctypes.c_double, P]
    L.tg_rope.restype = ctypes.c_int
    L.tg_rope_qk.argtypes = [P, P, P, I64, I32, I32, I32, ctypes.c_double, P]
    L.tg_rope_qk.restype = ctypes.c_int
    L.tg_gated_attention.argtypes = [P, P, P, P, P, F, P, I64, I32, I32, I32, P, I32, P]
    L.tg_gated_attention.restype = ctypes.c_int
    L.tg_gated_attention_timed.argtypes = [P, P, P, P, P, F, P, I64, I32, I32, I32, P, I32, P, P, P]
    L.tg_gated_attention_timed.restype = ctypes.c_int
    L.tg_rmsnorm.argtypes = [P, P, P, I64, I32, F, P]
    L.tg_rmsnorm.restype = ctypes.c_int
    L.tg_swiglu.argtypes = [P, P, I64, I32, P]
    L.tg_swiglu.restype = ctypes.c_int
    L.tg_blas_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.tg_blas_create.restype = ctypes.c_int
    L.tg_blas_destroy.argtypes = [P]
    L.tg_blas_destroy.restype = ctypes.c_int
    L.tg_linear.argtypes = [P, P, P, P, P, I64, I32, I32, P]
    L.tg_linear.restype = ctypes.c_int
    L.tg_attention_bwd_workspace_bytes.argtypes = [I64, I32, I32, I32]
    L.tg_attention_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.tg_gated_attention_bwd.argtypes = [P, P, P, P, P, F, P, I64, I32, I32, I32, P, P, P, P, P, P, P, P,
                                         ctypes.c_size_t, P]
    L.tg_gated_attention_bwd.restype = ctypes.c_int
    L.tg_gate_score_bwd_workspace_bytes.argtypes = [I64, I32, I32]
    L.tg_gate_score_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.tg_gate_score_bwd.argtypes = [P, P, P, P, P, I64, I32, I32, F, F, P, P, P, I64, P, P, P, P, P, P,
                                    ctypes.c_size_t, P]
    L.tg_gate_score_bwd.restype = ctypes.c_int
    L.tg_gated_delta_rule.argtypes = [P, P, P, P, P, P, I64, I32, I32, I32, I32, P, P, P]
    L.tg_gated_delta_rule.restype = ctypes.c_int
    L.tg_gated_delta_rule_workspace_bytes.argtypes = [I64, I32]
    L.tg_gated_delta_rule_workspace_bytes.restype = ctypes.c_size_t
    L.tg_gated_delta_rule_chunked.argtypes = [P, P, P, P, P, P, I64, I32, I32, I32, I32, P, P, P, ctypes.c_size_t, P]
    L.tg_gated_delta_rule_chunked.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().tg_status_string(int(status)).decode()


def tg_status_string(status: int) -> str:
    return status_string(status)


def tg_abi_version() -> int:
    return int(load().tg_abi_version())


def tg_workspace_bytes(n: int) -> int:
    return int(load().tg_workspace_bytes(int(n)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, dtype, shape=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check(fn: str, status: int):
    if status != TG_OK:
        raise TokenGateError(fn, status)


def workspace(n: int, device=None) -> torch.Tensor:
    """A workspace tensor of tg_workspace_bytes(n) bytes."""
    return torch.empty(max(1, tg_workspace_bytes(n)), dtype=torch.uint8, device=device or "cuda")


def tg_gate_score(resid: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                  b2: float, eps_row: float, eps_seq: float, score_norm: torch.Tensor,
                  score_raw: Optional[torch.Tensor], ws: torch.Tensor, stream=None) -> None:
    n, d = resid.shape
    hd = w1.shape[0]
    _need(resid, "resid", torch.bfloat16, (n, d))
    _need(w1, "w1", torch.bfloat16, (hd, d))
    _need(b1, "b1", torch.bfloat16, (hd,), optional=True)
    _need(w2, "w2", torch.bfloat16, (hd,))
    _need(score_norm, "score_norm", torch.float32, (n,))
    _need(score_raw, "score_raw", torch.float32, (n,), optional=True)
    _need(ws, "ws", torch.uint8)
    _check("tg_gate_score", load().tg_gate_score(
        _ptr(resid), _ptr(w1), _ptr(b1), _ptr(w2), float(b2), n, d, hd, float(eps_row), float(eps_seq),
        _ptr(score_norm), _ptr(score_raw), _ptr(ws), ws.numel(), _stream(stream)))


def tg_gate_score_noalloc(resid: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                          b2: float, eps_row: float, eps_seq: float, score_norm: torch.Tensor,
                          score_raw: Optional[torch.Tensor], stream=None) -> None:
    """tg_gate_score without a workspace (the library's fixed scratch; see the header)."""
    n, d = resid.shape
    hd = w1.shape[0]
    _need(resid, "resid", torch.bfloat16, (n, d))
    _need(w1, "w1", torch.bfloat16, (hd, d))
    _need(b1, "b1", torch.bfloat16, (hd,), optional=True)
    _need(w2, "w2", torch.bfloat16, (hd,))
    _need(score_norm, "score_norm", torch.float32, (n,))
    _need(score_raw, "score_raw", torch.float32, (n,), optional=True)
    _check("tg_gate_score_noalloc", load().tg_gate_score_noalloc(
        _ptr(resid), _ptr(w1), _ptr(b1), _ptr(w2), float(b2), n, d, hd, float(eps_row), float(eps_seq),
        _ptr(score_norm), _ptr(score_raw), _stream(stream)))


def kept_budget(n: int, n_forced: int, max_kept: int) -> int:
    """The total kept count K for a prompt of n tokens under a user budget of
    at most max_kept kept tokens (news.farwalk.ai, "How do you deploy
    TokenGate?": generation takes a maximum kept-prefill-token budget, and the
    question span is never pruned): K = min(max_kept, n).  A budget smaller
    than the n_forced question tokens cannot be met and raises ValueError,
    as does a budget below 1 or n_forced outside [0, n]."""
    n, n_forced, max_kept = int(n), int(n_forced), int(max_kept)
    if n < 1 or not 0 <= n_forced <= n:
        raise ValueError(f"prompt of {n} tokens with {n_forced} forced")
    if max_kept < 1:
        raise ValueError(f"kept budget {max_kept} < 1")
    k = min(max_kept, n)
    if k < n_forced:
        raise ValueError(f"kept budget {max_kept} is smaller than the {n_forced} tokens that are never pruned")
    return k


def tg_select_topk(score: torch.Tensor, forced: Optional[torch.Tensor], n_forced: int, k: int,
                   kept_idx: torch.Tensor, dev_status: Optional[torch.Tensor], ws: torch.Tensor,
                   stream=None) -> None:
    n = score.shape[0]
    _need(score, "score", torch.float32, (n,))
    _need(forced, "forced", torch.uint8, (n,), optional=True)
    _need(kept_idx, "kept_idx", torch.int32, (k,))
    _need(dev_status, "dev_status", torch.int32, (1,), optional=True)
    _need(ws, "ws", torch.uint8)
    _check("tg_select_topk", load().tg_select_topk(
        _ptr(score), _ptr(forced), n, int(n_forced), int(k), _ptr(kept_idx), _ptr(dev_status), _ptr(ws),
        ws.numel(), _stream(stream)))


def tg_gate_score_select(resid: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                         b2: float, eps_row: float, eps_seq: float, forced: Optional[torch.Tensor], n_forced: int,
                         k: int, score_norm: torch.Tensor, score_raw: Optional[torch.Tensor], kept_idx: torch.Tensor,
                         dev_status: Optional[torch.Tensor], ws: torch.Tensor, stream=None) -> None:
    """tg_gate_score then tg_select_topk on its normalised scores, in one call."""
    n, d = resid.shape
    hd = w1.shape[0]
    _need(resid, "resid", torch.bfloat16, (n, d))
    _need(w1, "w1", torch.bfloat16, (hd, d))
    _need(b1, "b1", torch.bfloat16, (hd,), optional=True)
    _need(w2, "w2", torch.bfloat16, (hd,))
    _need(forced, "forced", torch.uint8, (n,), optional=True)
    _need(score_norm, "score_norm", torch.float32, (n,))
    _need(score_raw, "score_raw", torch.float32, (n,), optional=True)
    _need(kept_idx, "kept_idx", torch.int32, (k,))
    _need(dev_status, "dev_status", torch.int32, (1,), optional=True)
    _need(ws, "ws", torch.uint8)
    _check("tg_gate_score_select", load().tg_gate_score_select(
        _ptr(resid), _ptr(w1), _ptr(b1), _ptr(w2), float(b2), n, d, hd, float(eps_row), float(eps_seq),
        _ptr(forced), int(n_forced), int(k), _ptr(score_norm), _ptr(score_raw), _ptr(kept_idx), _ptr(dev_status),
        _ptr(ws), ws.numel(), _stream(stream)))


def tg_compact(kept_idx: torch.Tensor, n: int, resid: Optional[torch.Tensor], resid_out: Optional[torch.Tensor],
               pos: Optional[torch.Tensor], pos_out: Optional[torch.Tensor], score: Optional[torch.Tensor],
               score_out: Optional[torch.Tensor],
               extra: Sequence[tuple] = (), stream=None) -> None:
    """extra: (src, dst) tensor pairs whose first dim is the token; rows are
    copied as raw bytes (src row stride = dst row stride = bytes per row)."""
    k = kept_idx.shape[0]
    _need(kept_idx, "kept_idx", torch.int32, (k,))
    d = 0
    if resid is not None:
        d = resid.shape[1]
        _need(resid, "resid", torch.bfloat16, (n, d))
        _need(resid_out, "resid_out", torch.bfloat16, (k, d))
    _need(pos, "pos", torch.int32, (n,), optional=True)
    _need(pos_out, "pos_out", torch.int32, (k,), optional=True)
    _need(score, "score", torch.float32, (n,), optional=True)
    _need(score_out, "score_out", torch.float32, (k,), optional=True)
    if len(extra) > TG_MAX_GATHER:
        raise ValueError("too many extra streams")
    arr = (TgGather * max(1, len(extra)))()
    for e, (src, dst) in enumerate(extra):
        if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
            raise ValueError("extra streams must be contiguous GPU tensors")
        if src.shape[0] != n or dst.shape[0] != k or src.dtype != dst.dtype or src.shape[1:] != dst.shape[1:]:
            raise ValueError("extra stream shapes do not match")
        rb = src[0].numel() * src.element_size()
        arr[e] = TgGather(src.data_ptr(), dst.data_ptr(), rb, rb, rb)
    _check("tg_compact", load().tg_compact(
        _ptr(kept_idx), k, int(n), _ptr(resid), _ptr(resid_out), d, _ptr(pos), _ptr(pos_out), _ptr(score),
        _ptr(score_out), arr if extra else None, len(extra), _stream(stream)))


def tg_rope(x: torch.Tensor, pos: torch.Tensor, theta: float, stream=None) -> None:
    rows, heads, hd = x.shape
    _need(x, "x", torch.bfloat16)
    _need(pos, "pos", torch.int32, (rows,))
    _check("tg_rope", load().tg_rope(_ptr(x), _ptr(pos), rows, heads, hd, float(theta), _stream(stream)))


def tg_rope_qk(q: torch.Tensor, k: torch.Tensor, pos: torch.Tensor, theta: float, stream=None) -> None:
    rows, hq, hd = q.shape
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (rows, k.shape[1], hd))
    _need(pos, "pos", torch.int32, (rows,))
    _check("tg_rope_qk", load().tg_rope_qk(_ptr(q), _ptr(k), _ptr(pos), rows, hq, k.shape[1], hd, float(theta),
                                           _stream(stream)))


def _attention_args(q, k, v, key_score, gains, temp_coef, pos, out, stream):
    nk, hq, D = q.shape
    hkv = k.shape[1]
    _need(q, "q", torch.bfloat16, (nk, hq, D))
    _need(k, "k", torch.bfloat16, (nk, hkv, D))
    _need(v, "v", torch.bfloat16, (nk, hkv, D))
    _need(key_score, "key_score", torch.float32, (nk,))
    _need(gains, "gains", torch.float32, (hq,))
    _need(pos, "pos", torch.int32, (nk,))
    if out.dtype == torch.bfloat16:
        od = 0
    elif out.dtype == torch.float32:
        od = 1
    else:
        raise ValueError("out must be bfloat16 or float32")
    _need(out, "out", out.dtype, (nk, hq, D))
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(gains), float(temp_coef), _ptr(pos), nk, hq, hkv, D,
            _ptr(out), od, _stream(stream))


def tg_gated_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: torch.Tensor,
                       gains: torch.Tensor, temp_coef: float, pos: torch.Tensor, out: torch.Tensor,
                       stream=None) -> None:
    _check("tg_gated_attention", load().tg_gated_attention(
        *_attention_args(q, k, v, key_score, gains, temp_coef, pos, out, stream)))


def tg_gated_attention_timed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: torch.Tensor,
                             gains: torch.Tensor, temp_coef: float, pos: torch.Tensor, out: torch.Tensor,
                             start, stop, stream=None) -> None:
    """tg_gated_attention whose launch also records two torch.cuda.Event
    objects (timing enabled) at the attention kernel's own start and end.
    torch creates an event's HIP handle at its first record, so each must
    have been recorded once before."""
    for e in (start, stop):
        if not e.cuda_event:
            raise ValueError("record each event once before passing it (its HIP handle is created then)")
    _check("tg_gated_attention_timed", load().tg_gated_attention_timed(
        *_attention_args(q, k, v, key_score, gains, temp_coef, pos, out, stream), start.cuda_event,
        stop.cuda_event))


def tg_rmsnorm(x: torch.Tensor, weight: torch.Tensor, y: torch.Tensor, eps: float, stream=None) -> None:
    """Row RMSNorm over the last dimension of x (any leading shape)."""
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    _need(x, "x", torch.bfloat16)
    _need(weight, "weight", torch.bfloat16, (dim,))
    _need(y, "y", torch.bfloat16, tuple(x.shape))
    _check("tg_rmsnorm", load().tg_rmsnorm(_ptr(x), _ptr(weight), _ptr(y), rows, dim, float(eps), _stream(stream)))


def tg_swiglu(gate_up: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    rows, two_inter = gate_up.shape
    inter = two_inter // 2
    _need(gate_up, "gate_up", torch.bfloat16, (rows, 2 * inter))
    _need(out, "out", torch.bfloat16, (rows, inter))
    _check("tg_swiglu", load().tg_swiglu(_ptr(gate_up), _ptr(out), rows, inter, _stream(stream)))


class BlasHandle:
    """Owner of a rocBLAS handle from tg_blas_create (destroyed with the object)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check("tg_blas_create", load().tg_blas_create(ctypes.byref(h)))
        self.value = h

    def close(self):
        if self.value is not None and self.value.value:
            _check("tg_blas_destroy", load().tg_blas_destroy(self.value))
        self.value = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tg_linear(handle: BlasHandle, x: torch.Tensor, w: torch.Tensor, residual: Optional[torch.Tensor],
              y: torch.Tensor, stream=None) -> None:
    """y = x . w^T (+ residual); x [rows, in], w [out, in], y and residual [rows, out]."""
    rows, in_dim = x.shape
    out_dim = w.shape[0]
    _need(x, "x", torch.bfloat16, (rows, in_dim))
    _need(w, "w", torch.bfloat16, (out_dim, in_dim))
    _need(residual, "residual", torch.bfloat16, (rows, out_dim), optional=True)
    _need(y, "y", torch.bfloat16, (rows, out_dim))
    _check("tg_linear", load().tg_linear(handle.value, _ptr(x), _ptr(w), _ptr(residual), _ptr(y), rows, in_dim,
                                         out_dim, _stream(stream)))


def tg_attention_bwd_workspace_bytes(n_kept: int, hq: int, hkv: int, head_dim: int) -> int:
    return int(load().tg_attention_bwd_workspace_bytes(int(n_kept), int(hq), int(hkv), int(head_dim)))


def tg_gated_attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_score: torch.Tensor,
                           gains: torch.Tensor, temp_coef: float, pos: torch.Tensor, dout: torch.Tensor,
                           dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, dscore: torch.Tensor,
                           dgains: torch.Tensor, dtemp: torch.Tensor, ws: Optional[torch.Tensor] = None,
                           stream=None) -> None:
    """Gradients of tg_gated_attention (fp32 outputs, overwritten)."""
    nk, hq, D = q.shape
    hkv = k.shape[1]
    _need(q, "q", torch.bfloat16, (nk, hq, D))
    _need(k, "k", torch.bfloat16, (nk, hkv, D))
    _need(v, "v", torch.bfloat16, (nk, hkv, D))
    _need(key_score, "key_score", torch.float32, (nk,))
    _need(gains, "gains", torch.float32, (hq,))
    _need(pos, "pos", torch.int32, (nk,))
    _need(dout, "dout", torch.bfloat16, (nk, hq, D))
    _need(dq, "dq", torch.float32, (nk, hq, D))
    _need(dk, "dk", torch.float32, (nk, hkv, D))
    _need(dv, "dv", torch.float32, (nk, hkv, D))
    _need(dscore, "dscore", torch.float32, (nk,))
    _need(dgains, "dgains", torch.float32, (hq,))
    _need(dtemp, "dtemp", torch.float32, (1,))
    if ws is None:
        ws = torch.empty(max(1, tg_attention_bwd_workspace_bytes(nk, hq, hkv, D)), dtype=torch.uint8,
                         device=q.device)
    _need(ws, "ws", torch.uint8)
    _check("tg_gated_attention_bwd", load().tg_gated_attention_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(key_score), _ptr(gains), float(temp_coef), _ptr(pos), nk, hq, hkv, D,
        _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dscore), _ptr(dgains), _ptr(dtemp), _ptr(ws), ws.numel(),
        _stream(stream)))



def tg_gate_score_bwd_workspace_bytes(n: int, d: int, hd: int) -> int:
    return int(load().tg_gate_score_bwd_workspace_bytes(int(n), int(d), int(hd)))


def tg_gate_score_bwd(handle: BlasHandle, resid: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor],
                      w2: torch.Tensor, eps_row: float, eps_seq: float, score_raw: torch.Tensor,
                      dscore_kept: torch.Tensor, kept_idx: torch.Tensor, dresid: torch.Tensor, dw1: torch.Tensor,
                      db1: torch.Tensor, dw2: torch.Tensor, db2: torch.Tensor, ws: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Gradients of tg_gate_score's normalised scores (fp32 outputs, overwritten)."""
    n, d = resid.shape
    hd = w1.shape[0]
    k = kept_idx.shape[0]
    _need(resid, "resid", torch.bfloat16, (n, d))
    _need(w1, "w1", torch.bfloat16, (hd, d))
    _need(b1, "b1", torch.bfloat16, (hd,), optional=True)
    _need(w2, "w2", torch.bfloat16, (hd,))
    _need(score_raw, "score_raw", torch.float32, (n,))
    _need(dscore_kept, "dscore_kept", torch.float32, (k,))
    _need(kept_idx, "kept_idx", torch.int32, (k,))
    _need(dresid, "dresid", torch.float32, (n, d))
    _need(dw1, "dw1", torch.float32, (hd, d))
    _need(db1, "db1", torch.float32, (hd,))
    _need(dw2, "dw2", torch.float32, (hd,))
    _need(db2, "db2", torch.float32, (1,))
    if ws is None:
        ws = torch.empty(max(1, tg_gate_score_bwd_workspace_bytes(n, d, hd)), dtype=torch.uint8, device=resid.device)
    _need(ws, "ws", torch.uint8)
    _check("tg_gate_score_bwd", load().tg_gate_score_bwd(
        handle.value, _ptr(resid), _ptr(w1), _ptr(b1), _ptr(w2), n, d, hd, float(eps_row), float(eps_seq),
        _ptr(score_raw), _ptr(dscore_kept), _ptr(kept_idx), k, _ptr(dresid), _ptr(dw1), _ptr(db1), _ptr(dw2),
        _ptr(db2), _ptr(ws), ws.numel(), _stream(stream)))


def _gdn_args(q, k, v, alpha, beta, out, state_in, state_out):
    n, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    _need(q, "q", torch.bfloat16, (n, hk, dk))
    _need(k, "k", torch.bfloat16, (n, hk, dk))
    _need(v, "v", torch.bfloat16, (n, hv, dv))
    _need(alpha, "alpha", torch.float32, (n, hv))
    _need(beta, "beta", torch.float32, (n, hv))
    _need(out, "out", torch.float32, (n, hv, dv))
    _need(state_in, "state_in", torch.float32, (hv, dv, dk), optional=True)
    _need(state_out, "state_out", torch.float32, (hv, dv, dk), optional=True)
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in), n, hk, hv, dk, dv, _ptr(out),
            _ptr(state_out))


def tg_gated_delta_rule(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                        out: torch.Tensor, state_in: Optional[torch.Tensor] = None,
                        state_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """Gated delta rule over the token sequence (fp32 out and state), as a scan."""
    _check("tg_gated_delta_rule", load().tg_gated_delta_rule(
        *_gdn_args(q, k, v, alpha, beta, out, state_in, state_out), _stream(stream)))


def tg_gated_delta_rule_workspace_bytes(n: int, hv: int) -> int:
    return int(load().tg_gated_delta_rule_workspace_bytes(int(n), int(hv)))


def gdn_workspace(n: int, hv: int, device=None) -> torch.Tensor:
    """A workspace for tg_gated_delta_rule_chunked (uint8; no contents need clearing)."""
    return torch.empty(tg_gated_delta_rule_workspace_bytes(n, hv), dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def tg_gated_delta_rule_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                                beta: torch.Tensor, out: torch.Tensor, ws: torch.Tensor,
                                state_in: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
                                stream=None) -> None:
    """The gated delta rule in chunks on the matrix cores (same results to rounding)."""
    _need(ws, "ws", torch.uint8)
    _check("tg_gated_delta_rule_chunked", load().tg_gated_delta_rule_chunked(
        *_gdn_args(q, k, v, alpha, beta, out, state_in, state_out), _ptr(ws), ws.numel(), _stream(stream)))
