"""GPU parity of the token-gated attention backward against the fp64 gradient oracle.

The oracle (oracle/attn_bwd.py) is pinned to finite differences of the C
forward oracle.  Tolerances follow the arithmetic: dq, dk and dv come out of
matrix-core products whose operands P and dU are rounded to bf16 (relative
step 2^-8), so they are held to a relative RMS of 1e-2 of their own norm.
The score and gain gradients are fp32 sums of the unrounded dU, but dU
carries D_t = dO.O, and O comes from the forward whose P.V product takes P in
bf16 (O within ~2^-9); they are held to 5e-3 of their norm.  The temperature
gradient sums dlambda_t ln(ratio) terms that cancel, most where lambda is
large (sharp rows): 1.5e-2 of its magnitude.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from oracle import attn_bwd, oracle

pytestmark = pytest.mark.gpu

TOL_QKV = 1e-2
TOL_SG = 5e-3
TOL_C = 1.5e-2


def _case(seed, nk, hq, hkv, D, c, pos_spread=4):
    g = np.random.default_rng(seed)
    q = oracle.to_bf16(g.normal(size=(nk, hq, D)))
    k = oracle.to_bf16(g.normal(size=(nk, hkv, D)))
    v = oracle.to_bf16(g.normal(size=(nk, hkv, D)))
    dout = oracle.to_bf16(g.normal(size=(nk, hq, D)))
    ks = g.normal(size=nk).astype(np.float32)
    gains = g.uniform(0.5, 2.0, size=hq).astype(np.float32)
    pos = np.sort(g.choice(pos_spread * nk, size=nk, replace=False)).astype(np.int32)
    return q, k, v, dout, ks, gains, pos, c


def _run(q, k, v, dout, ks, gains, pos, c):
    nk, hq, D = q.shape
    hkv = k.shape[1]
    f32 = dict(dtype=torch.float32, device=gu.dev())
    outs = dict(dq=torch.empty(nk, hq, D, **f32), dk=torch.empty(nk, hkv, D, **f32),
                dv=torch.empty(nk, hkv, D, **f32), ds=torch.empty(nk, **f32), dg=torch.empty(hq, **f32),
                dc=torch.empty(1, **f32))
    tg.tg_gated_attention_bwd(gu.bf16(q), gu.bf16(k), gu.bf16(v), gu.f32(ks), gu.f32(gains), c, gu.i32(pos),
                              gu.bf16(dout), outs["dq"], outs["dk"], outs["dv"], outs["ds"], outs["dg"], outs["dc"])
    torch.cuda.synchronize()
    return {n: t.cpu().numpy().astype(np.float64) for n, t in outs.items()}


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


# (97, ..., -0.9) with positions spread 40x: temperatures up to ~4 (sharp rows);
# (150, ..., 0.5) spread 40x: lambda < 0 on the early rows
@pytest.mark.parametrize("nk,hq,hkv,D,c,seed,spread", [(200, 4, 2, 64, 0.1, 1, 4), (333, 8, 1, 128, 0.1, 2, 4),
                                                       (256, 16, 8, 128, 0.1, 3, 4), (31, 2, 2, 64, 0.0, 4, 4),
                                                       (97, 4, 2, 128, -0.9, 5, 40), (150, 4, 2, 64, 0.5, 8, 40)])
def test_attention_backward_matches_oracle(nk, hq, hkv, D, c, seed, spread):
    q, k, v, dout, ks, gains, pos, c = _case(seed, nk, hq, hkv, D, c, pos_spread=spread)
    t = np.arange(nk)
    gu.say(f"  lambda range {np.min(1 + c * np.log((t + 1) / (pos + 1))):.2f} .. "
           f"{np.max(1 + c * np.log((t + 1) / (pos + 1))):.2f}")
    gu.say(f"attention backward nk={nk} hq={hq} hkv={hkv} D={D} c={c}")
    got = _run(q, k, v, dout, ks, gains, pos, c)
    w = oracle.widen_bf16
    _, dq, dk, dv, ds, dg, dc = attn_bwd.gated_attention_grads(w(q), w(k), w(v), ks, gains, c, pos, w(dout))
    errs = dict(dq=_rel(got["dq"], dq), dk=_rel(got["dk"], dk), dv=_rel(got["dv"], dv), ds=_rel(got["ds"], ds),
                dg=_rel(got["dg"], dg), dc=abs(got["dc"][0] - dc) / max(abs(dc), 1e-30))
    gu.say("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n in ("dq", "dk", "dv"):
        assert errs[n] <= TOL_QKV, n
    for n in ("ds", "dg"):
        assert errs[n] <= TOL_SG, n
    assert abs(got["dc"][0] - dc) <= TOL_C * max(abs(dc), 1e-6), "dc"


@pytest.mark.parametrize("hq,hkv,D", [(2, 1, 64), (4, 2, 128)])
def test_attention_backward_single_token(hq, hkv, D):
    """One kept token: every softmax row is the constant 1, so O = v_0, the
    value gradient is the sum of the group's output gradients, and every other
    gradient is zero (dP - D_t cancels exactly).  Zero is checked in absolute
    terms: the fp32 cancellation leaves ~1e-7 of |dO| |v|."""
    q, k, v, dout, ks, gains, pos, c = _case(6, 1, hq, hkv, D, 0.1)
    gu.say(f"attention backward single token hq={hq} hkv={hkv} D={D}")
    got = _run(q, k, v, dout, ks, gains, pos, c)
    w = oracle.widen_bf16
    G = hq // hkv
    want_dv = w(dout).reshape(1, hkv, G, D).sum(axis=2)
    assert np.allclose(got["dv"], want_dv, rtol=1e-6, atol=1e-6)
    scale = float(np.linalg.norm(w(dout)) * np.linalg.norm(w(v)))
    for n in ("dq", "dk", "ds", "dg", "dc"):
        assert np.max(np.abs(got[n])) <= 1e-5 * scale, n


def test_attention_backward_is_deterministic():
    case = _case(7, 300, 4, 2, 128, 0.1)
    gu.say("attention backward determinism")
    a = _run(*case)
    b = _run(*case)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
