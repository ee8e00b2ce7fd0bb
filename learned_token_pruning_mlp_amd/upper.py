"""Decoder layers around the gate, composed from the library's entry points.

Above the gate layer only the kept tokens pass through the backbone's layers,
with their original positions, and no KV is written for the pruned ones
(fluxbbs.com TokenGate article, section on where the gate sits;
news.farwalk.ai, "How does TokenGate learned token pruning work?";
aiwillknow.com, Figure 1(a)(b)).  With a Qwen3-shaped backbone one layer is

    h2 = h + Wo . attention(rope(qk_norm(Wq, Wk . rmsnorm(h))), Wv . rmsnorm(h))
    h3 = h2 + Wdown . swiglu(Wgu . rmsnorm(h2))

Every step is a call of the C ABI (tg_rmsnorm, tg_linear, tg_rope_qk,
tg_gated_attention, tg_swiglu, and the gate path); this module only chains
them and owns the buffers.  ``Prefill`` runs a whole prompt both ways: every
layer on all N tokens with plain causal attention (full prefill), and the
gated form -- the layers below the gate on N tokens, the gate layer's
attention block on N, then scorer, top-K and compaction of its
post-attention residual (plus the lower layers' K and V, trimmed to the kept
rows), the gate layer's MLP and every upper layer on the K kept rows with
token-gated attention.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import binding as tg


@dataclass(frozen=True)
class LayerShape:
    d: int
    hq: int
    hkv: int
    head_dim: int
    inter: int
    theta: float = 1.0e6
    eps: float = 1e-6


# Qwen3-1.7B decoder layer
QWEN3_1P7B_LAYER = LayerShape(d=2048, hq=16, hkv=8, head_dim=128, inter=6144)


@dataclass
class LayerWeights:
    w_in: torch.Tensor    # [d]
    wq: torch.Tensor      # [hq*D, d]
    wk: torch.Tensor      # [hkv*D, d]
    wv: torch.Tensor      # [hkv*D, d]
    w_qn: torch.Tensor    # [D]
    w_kn: torch.Tensor    # [D]
    wo: torch.Tensor      # [d, hq*D]
    w_post: torch.Tensor  # [d]
    wgu: torch.Tensor     # [2*inter, d]
    wdown: torch.Tensor   # [d, inter]


def random_weights(s: LayerShape, gen: torch.Generator, device, scale: float = 0.02) -> LayerWeights:
    """Synthetic weights of one layer: projections ~ N(0, scale^2), norm weights ~ 1 + N(0, 0.1^2), bf16."""
    def n(*shape, sd=scale, mean=0.0):
        return (torch.randn(*shape, generator=gen, device=device) * sd + mean).to(torch.bfloat16)
    D = s.head_dim
    return LayerWeights(w_in=n(s.d, sd=0.1, mean=1.0), wq=n(s.hq * D, s.d), wk=n(s.hkv * D, s.d),
                        wv=n(s.hkv * D, s.d), w_qn=n(D, sd=0.1, mean=1.0), w_kn=n(D, sd=0.1, mean=1.0),
                        wo=n(s.d, s.hq * D), w_post=n(s.d, sd=0.1, mean=1.0), wgu=n(2 * s.inter, s.d),
                        wdown=n(s.d, s.inter))


class Buffers:
    """Activations of one layer for up to `rows` rows (reused layer after layer)."""

    def __init__(self, s: LayerShape, rows: int, device):
        bf = dict(dtype=torch.bfloat16, device=device)
        D = s.head_dim
        self.rows = rows
        self.x = torch.empty(rows, s.d, **bf)
        self.q = torch.empty(rows, s.hq, D, **bf)
        self.k = torch.empty(rows, s.hkv, D, **bf)
        self.v = torch.empty(rows, s.hkv, D, **bf)
        self.a = torch.empty(rows, s.hq, D, **bf)
        self.h2 = torch.empty(rows, s.d, **bf)
        self.gu = torch.empty(rows, 2 * s.inter, **bf)
        self.act = torch.empty(rows, s.inter, **bf)

    def view(self, rows: int) -> "Buffers":
        """The first `rows` rows of every buffer (contiguous views)."""
        b = Buffers.__new__(Buffers)
        b.rows = rows
        for name in ("x", "q", "k", "v", "a", "h2", "gu", "act"):
            setattr(b, name, getattr(self, name)[:rows])
        return b


def attention_block(blas: tg.BlasHandle, s: LayerShape, W: LayerWeights, h: torch.Tensor, pos: torch.Tensor,
                    key_score: torch.Tensor, gains: torch.Tensor, temp_coef: float, buf: Buffers,
                    h2: torch.Tensor, k_out: Optional[torch.Tensor] = None,
                    v_out: Optional[torch.Tensor] = None) -> None:
    """h2 = h + Wo . attention(...): rows of h are the tokens in order, at original positions pos.
    With gains = 0 and temp_coef = 0 the attention is plain causal attention."""
    rows = h.shape[0]
    D = s.head_dim
    k = k_out if k_out is not None else buf.k
    v = v_out if v_out is not None else buf.v
    tg.tg_rmsnorm(h, W.w_in, buf.x, s.eps)
    tg.tg_linear(blas, buf.x, W.wq, None, buf.q.view(rows, s.hq * D))
    tg.tg_linear(blas, buf.x, W.wk, None, k.view(rows, s.hkv * D))
    tg.tg_linear(blas, buf.x, W.wv, None, v.view(rows, s.hkv * D))
    tg.tg_rmsnorm(buf.q, W.w_qn, buf.q, s.eps)
    tg.tg_rmsnorm(k, W.w_kn, k, s.eps)
    tg.tg_rope_qk(buf.q, k, pos, s.theta)
    tg.tg_gated_attention(buf.q, k, v, key_score, gains, temp_coef, pos, buf.a)
    tg.tg_linear(blas, buf.a.view(rows, s.hq * D), W.wo, h, h2)


def mlp_block(blas: tg.BlasHandle, s: LayerShape, W: LayerWeights, h2: torch.Tensor, buf: Buffers,
              out: torch.Tensor) -> None:
    """out = h2 + Wdown . swiglu(Wgu . rmsnorm(h2))."""
    tg.tg_rmsnorm(h2, W.w_post, buf.x, s.eps)
    tg.tg_linear(blas, buf.x, W.wgu, None, buf.gu)
    tg.tg_swiglu(buf.gu, buf.act)
    tg.tg_linear(blas, buf.act, W.wdown, h2, out)


def decoder_layer(blas: tg.BlasHandle, s: LayerShape, W: LayerWeights, h: torch.Tensor, pos: torch.Tensor,
                  key_score: torch.Tensor, gains: torch.Tensor, temp_coef: float, buf: Buffers,
                  out: torch.Tensor) -> None:
    """One whole layer on the rows h [rows, d]; out may not alias h."""
    attention_block(blas, s, W, h, pos, key_score, gains, temp_coef, buf, buf.h2)
    mlp_block(blas, s, W, buf.h2, buf, out)


class Prefill:
    """A prompt of n tokens through n_layers layers, full or gated at layer `gate_layer`.

    Weights are synthetic (one set per layer); the scorer's w1 [hd, d] and
    w2 [hd] are given.  Upper layer l uses gains[l] [hq] and temp_coef.
    """

    def __init__(self, s: LayerShape, n: int, n_layers: int, gate_layer: int, w1: torch.Tensor, w2: torch.Tensor,
                 gains: torch.Tensor, temp_coef: float, device, seed: int = 0):
        assert 0 <= gate_layer < n_layers
        self.s, self.n, self.L, self.gl = s, n, n_layers, gate_layer
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        self.W: List[LayerWeights] = [random_weights(s, g, device) for _ in range(n_layers)]
        self.w1, self.w2 = w1, w2
        self.gains = gains
        self.temp_coef = temp_coef
        self.blas = tg.BlasHandle()
        self.buf = Buffers(s, n, device)
        f32 = dict(dtype=torch.float32, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        self.zeros_n = torch.zeros(n, **f32)
        self.zero_gains = torch.zeros(s.hq, **f32)
        self.arange = torch.arange(n, dtype=torch.int32, device=device)
        self.ha = torch.empty(n, s.d, **bf)
        self.hb = torch.empty(n, s.d, **bf)
        # K and V of the layers below the gate (and of the gate layer), N rows each
        self.k_low = [torch.empty(n, s.hkv, s.head_dim, **bf) for _ in range(gate_layer + 1)]
        self.v_low = [torch.empty(n, s.hkv, s.head_dim, **bf) for _ in range(gate_layer + 1)]
        self.h2_gate = torch.empty(n, s.d, **bf)  # the gate layer's post-attention residual
        self.s_norm = torch.empty(n, **f32)
        self.ws = tg.workspace(n, device)

    def full(self, h: torch.Tensor) -> torch.Tensor:
        """Every layer on all n tokens, plain causal attention; returns the last hidden rows."""
        src, dst = h, self.ha
        for l in range(self.L):
            decoder_layer(self.blas, self.s, self.W[l], src, self.arange, self.zeros_n, self.zero_gains, 0.0,
                          self.buf, dst)
            src, dst = dst, (self.hb if dst is self.ha else self.ha)
        return src

    def gated(self, h: torch.Tensor, forced: torch.Tensor, n_forced: int, max_kept: int):
        """Layers below the gate on n tokens, the gate on the gate layer's post-attention
        residual, then K = min(max_kept, n) tokens above (tg.kept_budget).  Returns
        (hidden [K, d], kept_idx, pos_k, trimmed K/V)."""
        s, n, dev = self.s, self.n, h.device
        k = tg.kept_budget(n, n_forced, max_kept)
        src, dst = h, self.ha
        for l in range(self.gl):
            attention_block(self.blas, s, self.W[l], src, self.arange, self.zeros_n, self.zero_gains, 0.0,
                            self.buf, self.buf.h2, self.k_low[l], self.v_low[l])
            mlp_block(self.blas, s, self.W[l], self.buf.h2, self.buf, dst)
            src, dst = dst, (self.hb if dst is self.ha else self.ha)
        # gate layer: its attention block on all n tokens, then the gate
        gl = self.gl
        attention_block(self.blas, s, self.W[gl], src, self.arange, self.zeros_n, self.zero_gains, 0.0,
                        self.buf, self.h2_gate, self.k_low[gl], self.v_low[gl])
        kept = torch.empty(k, dtype=torch.int32, device=dev)
        tg.tg_gate_score_select(self.h2_gate, self.w1, None, self.w2, 0.0, s.eps, s.eps, forced, n_forced, k,
                                self.s_norm, None, kept, None, self.ws)
        bf = dict(dtype=torch.bfloat16, device=dev)
        h2k = torch.empty(k, s.d, **bf)
        pos_k = torch.empty(k, dtype=torch.int32, device=dev)
        score_k = torch.empty(k, dtype=torch.float32, device=dev)
        kv_k = [(torch.empty(k, s.hkv, s.head_dim, **bf), torch.empty(k, s.hkv, s.head_dim, **bf))
                for _ in range(gl + 1)]
        extra = []
        for (kl, vl), kt, vt in zip(kv_k, self.k_low, self.v_low):
            extra += [(kt, kl), (vt, vl)]
        tg.tg_compact(kept, n, self.h2_gate, h2k, self.arange, pos_k, self.s_norm, score_k, extra)
        # the gate layer's MLP and every layer above it on the kept rows
        bk = self.buf.view(k)
        ha, hb = self.ha[:k], self.hb[:k]
        mlp_block(self.blas, s, self.W[gl], h2k, bk, ha)
        src, dst = ha, hb
        for l in range(gl + 1, self.L):
            decoder_layer(self.blas, s, self.W[l], src, pos_k, score_k, self.gains[l], self.temp_coef, bk, dst)
            src, dst = dst, (hb if dst is ha else ha)
        return src, kept, pos_k, kv_k

    def capture_gated(self, h: torch.Tensor, forced: torch.Tensor, n_forced: int, k: int):
        """The gated prefill captured as one HIP graph (the budget k fixes every
        shape, so one graph serves every prompt of n tokens).  One eager run
        first lets rocBLAS set itself up outside the capture.  Returns the
        graph and the tensors its replays write (hidden [k, d], kept_idx,
        pos_k, trimmed K/V); replay with ``graph.replay()`` after writing the
        next prompt into ``h``."""
        self.gated(h, forced, n_forced, k)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            outs = self.gated(h, forced, n_forced, k)
        torch.cuda.current_stream().wait_stream(side)
        return graph, outs

