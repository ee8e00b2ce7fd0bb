"""The gate's end-to-end gradient through the two backward oracles.

Forward (all fp64, the C forward oracle): residual -> scorer -> sequence
RMSNorm -> forced-keep top-K -> kept scores as the attention's key bias ->
token-gated attention over the kept tokens -> L = sum(dO * O).  The kept set
is a step function of the scores; the perturbations below are far too small
to change it (checked), so L is differentiable in W1, b1, w2 and the
residual there.  The analytic gradient chains the attention backward (its
key-score gradient, in kept order) into the scorer backward (scattered to
the kept tokens' original indices); it must match central finite
differences of the composed forward.  This pins the interface between the
two: kept order in, original index out, and the coupling of every token
through the sequence norm.
"""
import numpy as np

from oracle import attn_bwd, gate_bwd, oracle


def _setup(seed=11, n=14, d=8, hd=5, kk=6, hq=2, hkv=1, D=4):
    g = np.random.default_rng(seed)
    h = g.normal(size=(n, d))
    w1 = g.normal(size=(hd, d)) * 0.5
    b1 = g.normal(size=hd) * 0.3
    w2 = g.normal(size=hd)
    forced = np.zeros(n, dtype=np.uint8)
    forced[-2:] = 1
    q = g.normal(size=(kk, hq, D))
    k = g.normal(size=(kk, hkv, D))
    v = g.normal(size=(kk, hkv, D))
    gains = g.uniform(0.5, 2.0, size=hq)
    dout = g.normal(size=(kk, hq, D))
    return dict(h=h, w1=w1, b1=b1, w2=w2, b2=0.1, forced=forced, kk=kk, q=q, k=k, v=v, gains=gains, c=0.2,
                dout=dout)


def _forward(p, kept=None):
    s = oracle.score_mlp_f64(p["h"], p["w1"], p["b1"], p["w2"], p["b2"], 1e-6, nthreads=1)
    shat, _ = oracle.seq_rmsnorm(s, 1e-6)
    sel = oracle.select_topk(shat, p["forced"], p["kk"])
    if kept is not None:
        assert np.array_equal(sel, kept), "the perturbation changed the kept set"
    out = oracle.gated_attention_f64(p["q"], p["k"], p["v"], shat[sel], p["gains"], p["c"], sel, nthreads=1)
    return float(np.sum(out * p["dout"])), sel, shat


def test_gate_gradient_through_attention_matches_finite_differences():
    p = _setup()
    _, kept, shat = _forward(p)
    _, _, _, _, ds_kept, _, _ = attn_bwd.gated_attention_grads(p["q"], p["k"], p["v"], shat[kept], p["gains"],
                                                               p["c"], kept, p["dout"])
    n = p["h"].shape[0]
    dh, dw1, db1, dw2, db2 = gate_bwd.gate_score_grads(p["h"], p["w1"], p["b1"], p["w2"], p["b2"], 1e-6, 1e-6,
                                                       gate_bwd.scatter_kept(n, kept, ds_kept))
    eps = 1e-6
    for name, analytic in (("w1", dw1), ("b1", db1), ("w2", dw2), ("h", dh)):
        arr = p[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + eps
            lp, _, _ = _forward(p, kept)
            arr[idx] = a0 - eps
            lm, _, _ = _forward(p, kept)
            arr[idx] = a0
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(analytic, fd, rtol=1e-5, atol=1e-8, err_msg=name)
    # pruned tokens still get a residual gradient, through rho
    pruned = np.setdiff1d(np.arange(n), kept)
    assert np.abs(dh[pruned]).max() > 1e-6
