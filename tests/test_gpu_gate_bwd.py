"""GPU parity of the scorer backward (tg_gate_score_bwd) against the fp64
gradient oracle (oracle/gate_bwd.py, pinned to finite differences of the C
forward oracle).

Tolerances follow the arithmetic.  dz = r da is rounded to bf16 (relative
step 2^-8) as the operand of the two gradient GEMMs, so dresid and dw1 are
held to 1e-2 of their own norm (relative RMS).  dw2, db1 and db2 are fp32
values summed in fp64 from an fp32 recomputation of z (exact bf16 products)
and an erf good to 1.5e-7; they are held to 1e-5 of their norm (measured
2e-7 to 4e-7 up to 16K tokens), which leaves room for the cancellation in sums
of terms of both signs.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from learned_token_pruning_mlp_amd import synth
from oracle import gate_bwd, oracle

pytestmark = pytest.mark.gpu

TOL_GEMM = 1e-2
TOL_SUM = 1e-5


@pytest.fixture(scope="module")
def blas():
    h = tg.BlasHandle()
    yield h
    h.close()


def _case(n, d, hd, k, seed, with_b1):
    shape = synth.GateShape(n=n, d=d, hd=hd, n_forced=0, k=max(k, 1), hq=4, hkv=2, head_dim=64)
    inp = synth.gate_inputs(shape, seed, with_b1=with_b1)
    g = np.random.default_rng(seed + 1000)
    kept = np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)
    dsk = g.normal(size=k).astype(np.float32)
    return inp, kept, dsk


def _run(blas, inp, s_raw, kept, dsk, eps_row, eps_seq):
    n, d = inp.resid.shape
    hd = inp.w1.shape[0]
    f32 = dict(dtype=torch.float32, device=gu.dev())
    out = dict(dresid=torch.empty(n, d, **f32), dw1=torch.empty(hd, d, **f32), db1=torch.empty(hd, **f32),
               dw2=torch.empty(hd, **f32), db2=torch.empty(1, **f32))
    tg.tg_gate_score_bwd(blas, gu.bf16(inp.resid), gu.bf16(inp.w1), None if inp.b1 is None else gu.bf16(inp.b1),
                         gu.bf16(inp.w2), eps_row, eps_seq, gu.f32(s_raw), gu.f32(dsk), gu.i32(kept),
                         out["dresid"], out["dw1"], out["db1"], out["dw2"], out["db2"])
    torch.cuda.synchronize()
    return {n_: t.cpu().numpy().astype(np.float64) for n_, t in out.items()}


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("n,d,hd,k,seed,with_b1,eps_row,eps_seq", [
    (512, 256, 64, 128, 1, True, 1e-6, 1e-6),
    (1000, 512, 128, 250, 2, False, 0.3, 0.5),
    (777, 4096, 64, 77, 3, True, 1e-6, 1e-6),
    (5001, 256, 128, 400, 7, True, 1e-6, 1e-6),  # dW1 as two token chunks plus a one-row remainder
    (16384, 2048, 256, 2048, 4, False, 1e-6, 1e-6),  # the Qwen3-1.7B gate layer at 16K tokens
])
def test_gate_score_backward_matches_oracle(blas, n, d, hd, k, seed, with_b1, eps_row, eps_seq):
    inp, kept, dsk = _case(n, d, hd, k, seed, with_b1)
    s = oracle.score_mlp(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, eps_row)
    w = oracle.widen_bf16
    dh, dw1, db1, dw2, db2 = gate_bwd.gate_score_grads(
        w(inp.resid), w(inp.w1), None if inp.b1 is None else w(inp.b1), w(inp.w2), inp.b2, eps_row, eps_seq,
        gate_bwd.scatter_kept(n, kept, dsk))
    gu.say(f"scorer backward n={n} d={d} hd={hd} k={k}")
    got = _run(blas, inp, s.astype(np.float32), kept, dsk, eps_row, eps_seq)
    errs = dict(dresid=_rel(got["dresid"], dh), dw1=_rel(got["dw1"], dw1), db1=_rel(got["db1"], db1),
                dw2=_rel(got["dw2"], dw2), db2=abs(got["db2"][0] - db2) / max(abs(db2), 1e-30))
    gu.say("  " + " ".join(f"{a} {e:.2e}" for a, e in errs.items()))
    assert errs["dresid"] <= TOL_GEMM and errs["dw1"] <= TOL_GEMM
    assert errs["db1"] <= TOL_SUM and errs["dw2"] <= TOL_SUM
    assert abs(got["db2"][0] - db2) <= TOL_SUM * max(abs(db2), 1e-3 * np.abs(dsk).sum() / np.sqrt(n))


def test_gate_score_backward_no_kept_tokens_gives_zeros(blas):
    """k = 0: dshat is zero everywhere, so every gradient is exactly zero."""
    inp, _, _ = _case(300, 128, 64, 0, 5, True)
    s = oracle.score_mlp(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, 1e-6)
    gu.say("scorer backward k=0")
    got = _run(blas, inp, s.astype(np.float32), np.zeros(0, np.int32), np.zeros(0, np.float32), 1e-6, 1e-6)
    for name, v in got.items():
        assert not np.any(v), name


def test_gate_score_backward_is_deterministic(blas):
    inp, kept, dsk = _case(2048, 1024, 256, 300, 6, True)
    s = oracle.score_mlp(inp.resid, inp.w1, inp.b1, inp.w2, inp.b2, 1e-6).astype(np.float32)
    gu.say("scorer backward determinism")
    a = _run(blas, inp, s, kept, dsk, 1e-6, 1e-6)
    b = _run(blas, inp, s, kept, dsk, 1e-6, 1e-6)
    for name in a:
        assert np.array_equal(a[name], b[name]), name
