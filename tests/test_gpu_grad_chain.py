"""The gate's training gradient end to end on the GPU, through the C ABI:
tg_gate_score -> tg_select_topk -> (kept scores as key bias) ->
tg_gated_attention_bwd -> its key-score gradient, in kept order ->
tg_gate_score_bwd -> dW1, db1, dw2, db2 and the residual gradient.

The oracle chains the two fp64 gradient oracles on the same kept set (the
one the GPU selected; the selection itself is tested bit-exact elsewhere)
and the oracle's own normalised scores.  The score gradient enters the
scorer backward with its own tolerance (5e-3 of its norm), which carries
linearly into the scorer's gradients: dw2, db1, db2 are held to 1e-2 of
their norm, dW1 and the residual gradient (bf16 dz in their GEMMs as well)
to 2e-2.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from learned_token_pruning_mlp_amd import synth
from oracle import attn_bwd, gate_bwd, oracle

pytestmark = pytest.mark.gpu


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def test_gate_gradient_through_attention_on_gpu():
    shape = synth.GateShape(n=2048, d=256, hd=64, n_forced=16, k=256, hq=4, hkv=2, head_dim=64)
    inp = synth.gate_inputs(shape, 21, with_b1=True, w_std=0.05)
    g = np.random.default_rng(22)
    K, hq, hkv, D = shape.k, shape.hq, shape.hkv, shape.head_dim
    q, k, v, dout = (oracle.to_bf16(g.normal(size=s)) for s in ((K, hq, D), (K, hkv, D), (K, hkv, D), (K, hq, D)))
    gains = g.uniform(0.5, 2.0, size=hq).astype(np.float32)
    c = 0.1
    dev = gu.dev()
    f32 = dict(dtype=torch.float32, device=dev)
    gu.say("gradient chain n=2048 K=256")
    # forward on the GPU: scores and the kept set
    resid = gu.bf16(inp.resid)
    w1, b1, w2 = gu.bf16(inp.w1), gu.bf16(inp.b1), gu.bf16(inp.w2)
    snorm, sraw = torch.empty(shape.n, **f32), torch.empty(shape.n, **f32)
    ws = tg.workspace(shape.n)
    tg.tg_gate_score(resid, w1, b1, w2, inp.b2, 1e-6, 1e-6, snorm, sraw, ws)
    kept = torch.empty(K, dtype=torch.int32, device=dev)
    tg.tg_select_topk(snorm, gu.u8(inp.forced), int(inp.forced.sum()), K, kept, None, ws)
    key_score = snorm[kept.long()].contiguous()
    # attention backward on the kept tokens, then the scorer backward
    outs = [torch.empty(K, hq, D, **f32), torch.empty(K, hkv, D, **f32), torch.empty(K, hkv, D, **f32),
            torch.empty(K, **f32), torch.empty(hq, **f32), torch.empty(1, **f32)]
    tg.tg_gated_attention_bwd(gu.bf16(q), gu.bf16(k), gu.bf16(v), key_score, gu.f32(gains), c, kept, gu.bf16(dout),
                              *outs)
    ds_kept = outs[3]
    blas = tg.BlasHandle()
    try:
        grads = [torch.empty(shape.n, shape.d, **f32), torch.empty(shape.hd, shape.d, **f32),
                 torch.empty(shape.hd, **f32), torch.empty(shape.hd, **f32), torch.empty(1, **f32)]
        tg.tg_gate_score_bwd(blas, resid, w1, b1, w2, 1e-6, 1e-6, sraw, ds_kept, kept, *grads)
        torch.cuda.synchronize()
    finally:
        blas.close()
    got = [x.cpu().numpy().astype(np.float64) for x in grads]
    kept_h = kept.cpu().numpy()

    # the same chain in fp64 on the same kept set
    w = oracle.widen_bf16
    s = oracle.score_mlp(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, 1e-6)
    shat, _ = oracle.seq_rmsnorm(s, 1e-6)
    _, _, _, _, ds_o, _, _ = attn_bwd.gated_attention_grads(w(q), w(k), w(v), shat[kept_h], gains, c, kept_h,
                                                            w(dout))
    want = gate_bwd.gate_score_grads(w(inp.resid), w(inp.w1), w(inp.b1), w(inp.w2), inp.b2, 1e-6, 1e-6,
                                     gate_bwd.scatter_kept(shape.n, kept_h, ds_o))
    names = ("dresid", "dw1", "db1", "dw2", "db2")
    errs = {nm: _rel(np.atleast_1d(a), np.atleast_1d(b)) for nm, a, b in zip(names, got, want)}
    gu.say("  " + " ".join(f"{nm} {e:.2e}" for nm, e in errs.items()))
    assert errs["dresid"] <= 2e-2 and errs["dw1"] <= 2e-2
    assert errs["db1"] <= 1e-2 and errs["dw2"] <= 1e-2 and errs["db2"] <= 1e-2
