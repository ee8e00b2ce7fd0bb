"""GPU parity of the gated delta rule against the fp64 oracle (oracle/gdn.py,
pinned to the unrolled transition product, exact retrieval and pure decay),
in both forms: the scan (tg_gated_delta_rule) and the chunked form on the
matrix cores (tg_gated_delta_rule_chunked, with its workspace).

Keys and queries are unit rows (rounded to bf16), alpha in [0.9, 1) and beta
in [0, 1), so every step is non-expansive.  fp32 rounding adds about 6e-8 of
the state per step; independent roundings add up like a random walk,
sqrt(T) * 6e-8 (3e-6 at T = 2048), so the output and the final state are held
to 1e-5 relative RMS (measured about 1.2e-7).
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from oracle import gdn, oracle

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _case(seed, T, hk, hv, dk, dv, with_state):
    g = np.random.default_rng(seed)

    def unit_rows(shape):
        x = g.normal(size=shape)
        return oracle.to_bf16(x / np.linalg.norm(x, axis=-1, keepdims=True))
    q, k = unit_rows((T, hk, dk)), unit_rows((T, hk, dk))
    v = oracle.to_bf16(g.normal(size=(T, hv, dv)))
    alpha = g.uniform(0.9, 1.0, size=(T, hv)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, size=(T, hv)).astype(np.float32)
    s0 = g.normal(size=(hv, dv, dk)).astype(np.float32) * 0.1 if with_state else None
    return q, k, v, alpha, beta, s0


FORMS = ["scan", "chunked"]


def _mixer(form, q, k, v, alpha, beta, out, state_in=None, state_out=None):
    """One call of the given form on device tensors."""
    if form == "scan":
        tg.tg_gated_delta_rule(q, k, v, alpha, beta, out, state_in, state_out)
    else:
        ws = tg.gdn_workspace(q.shape[0], v.shape[1], gu.dev())
        tg.tg_gated_delta_rule_chunked(q, k, v, alpha, beta, out, ws, state_in, state_out)


def _run(q, k, v, alpha, beta, s0, form="scan"):
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    out = torch.empty(T, hv, dv, dtype=torch.float32, device=gu.dev())
    so = torch.empty(hv, dv, dk, dtype=torch.float32, device=gu.dev())
    _mixer(form, gu.bf16(q), gu.bf16(k), gu.bf16(v), gu.f32(alpha), gu.f32(beta), out,
           None if s0 is None else gu.f32(s0), so)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), so.cpu().numpy().astype(np.float64)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("T,hk,hv,dk,dv,seed,with_state", [
    (200, 2, 4, 128, 128, 1, True), (333, 4, 4, 64, 128, 2, False), (97, 1, 2, 128, 64, 3, True),
    (65, 2, 2, 64, 64, 4, False), (1, 2, 4, 128, 128, 5, True), (32, 2, 2, 128, 128, 12, True),
    (2048, 16, 16, 128, 128, 6, False),  # 16 heads of 128 over the 2048 kept tokens of a 16K prompt
])
def test_gated_delta_rule_matches_oracle(T, hk, hv, dk, dv, seed, with_state, form):
    q, k, v, alpha, beta, s0 = _case(seed, T, hk, hv, dk, dv, with_state)
    w = oracle.widen_bf16
    want_o, want_s = gdn.gated_delta_rule(w(q), w(k), w(v), alpha, beta, s0)
    gu.say(f"gated delta rule ({form}) T={T} hk={hk} hv={hv} dk={dk} dv={dv}")
    got_o, got_s = _run(q, k, v, alpha, beta, s0, form)
    eo, es = _rel(got_o, want_o), _rel(got_s, want_s)
    gu.say(f"  out {eo:.2e} state {es:.2e}")
    assert eo <= TOL and es <= TOL


@pytest.mark.parametrize("form", FORMS)
def test_gated_delta_rule_empty_sequence_passes_state_through(form):
    _, _, _, _, _, s0 = _case(7, 1, 2, 4, 128, 64, True)
    hv, dv, dk = s0.shape
    so = torch.full((hv, dv, dk), 7.0, dtype=torch.float32, device=gu.dev())
    e = torch.empty(0, dtype=torch.bfloat16, device=gu.dev())
    gu.say(f"gated delta rule ({form}) T=0")
    _mixer(form, e.view(0, 2, dk), e.view(0, 2, dk), e.view(0, hv, dv),
           torch.empty(0, hv, dtype=torch.float32, device=gu.dev()),
           torch.empty(0, hv, dtype=torch.float32, device=gu.dev()),
           torch.empty(0, hv, dv, dtype=torch.float32, device=gu.dev()), gu.f32(s0), so)
    torch.cuda.synchronize()
    assert np.array_equal(so.cpu().numpy(), s0)


@pytest.mark.parametrize("form,m", [("scan", 123), ("chunked", 128)])
def test_gated_delta_rule_state_carries_over_a_split(form, m):
    """Running tokens [0, m) then [m, T) from the carried state equals one run
    bit for bit (the chunked form at a multiple of its 32-token chunks)."""
    q, k, v, alpha, beta, s0 = _case(8, 300, 2, 4, 128, 128, True)
    gu.say(f"gated delta rule ({form}) split at {m}")
    o_all, s_all = _run(q, k, v, alpha, beta, s0, form)
    o1, s1 = _run(q[:m], k[:m], v[:m], alpha[:m], beta[:m], s0, form)
    o2, s2 = _run(q[m:], k[m:], v[m:], alpha[m:], beta[m:], s1.astype(np.float32), form)
    assert np.array_equal(np.concatenate([o1, o2]), o_all)
    assert np.array_equal(s2, s_all)


def test_gated_delta_rule_chunked_split_off_the_chunk_grid():
    """A split of the chunked form inside a chunk regroups the tokens into
    other chunks: the same results to rounding (within 1e-6)."""
    q, k, v, alpha, beta, s0 = _case(13, 300, 2, 4, 128, 128, True)
    gu.say("gated delta rule (chunked) split at 123")
    o_all, s_all = _run(q, k, v, alpha, beta, s0, "chunked")
    m = 123
    o1, s1 = _run(q[:m], k[:m], v[:m], alpha[:m], beta[:m], s0, "chunked")
    o2, s2 = _run(q[m:], k[m:], v[m:], alpha[m:], beta[m:], s1.astype(np.float32), "chunked")
    assert _rel(np.concatenate([o1, o2]), o_all) <= 1e-6
    assert _rel(s2, s_all) <= 1e-6


def test_gated_delta_rule_chunked_deterministic():
    q, k, v, alpha, beta, s0 = _case(14, 777, 4, 8, 128, 128, True)
    gu.say("gated delta rule (chunked) determinism")
    a = _run(q, k, v, alpha, beta, s0, "chunked")
    b = _run(q, k, v, alpha, beta, s0, "chunked")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("T,hk,hv,dk,dv", [(16384, 16, 16, 128, 128), (8191, 2, 8, 64, 64)])
def test_gated_delta_rule_chunked_deterministic_at_length(T, hk, hv, dk, dv):
    """At the hybrid mixer's full shape (16384 kept tokens, 16 heads of 128,
    512 chunks, inputs far beyond the caches), and with 64-wide heads shared
    four ways over a ragged 8191 tokens, three chunked calls agree bit for
    bit, and with the scan to the relative RMS bound above."""
    gu.say(f"gated delta rule (chunked) determinism at T={T}, hk={hk}, hv={hv}, dk={dk}, dv={dv}")
    g = torch.Generator(device=gu.dev())
    g.manual_seed(T)

    def unit(*shape):
        x = torch.randn(*shape, generator=g, device=gu.dev())
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    q, k = unit(T, hk, dk), unit(T, hk, dk)
    v = torch.randn(T, hv, dv, generator=g, device=gu.dev()).to(torch.bfloat16)
    alpha = torch.rand(T, hv, generator=g, device=gu.dev()) * 0.1 + 0.9
    beta = torch.rand(T, hv, generator=g, device=gu.dev())
    outs = []
    for form in ("chunked", "chunked", "chunked", "scan"):
        out = torch.empty(T, hv, dv, dtype=torch.float32, device=gu.dev())
        so = torch.empty(hv, dv, dk, dtype=torch.float32, device=gu.dev())
        _mixer(form, q, k, v, alpha, beta, out, None, so)
        outs.append((out, so))
    torch.cuda.synchronize()
    for o, s in outs[1:3]:
        assert torch.equal(o, outs[0][0]) and torch.equal(s, outs[0][1])
    for i in range(2):
        ref = outs[3][i].double()
        rel = ((outs[0][i].double() - ref).norm() / ref.norm()).item()
        assert rel < TOL, rel


@pytest.mark.parametrize("form", FORMS)
def test_gated_delta_rule_state_in_place(form):
    """state_out may be the state_in buffer: the state is updated in place."""
    q, k, v, alpha, beta, s0 = _case(9, 150, 2, 4, 128, 128, True)
    gu.say(f"gated delta rule ({form}) in-place state")
    want_o, want_s = _run(q, k, v, alpha, beta, s0, form)
    st = gu.f32(s0)
    out = torch.empty(150, 4, 128, dtype=torch.float32, device=gu.dev())
    _mixer(form, gu.bf16(q), gu.bf16(k), gu.bf16(v), gu.f32(alpha), gu.f32(beta), out, st, st)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), want_o)
    assert np.array_equal(st.cpu().numpy().astype(np.float64), want_s)


@pytest.mark.parametrize("form", FORMS)
def test_gated_delta_rule_over_compacted_kept_tokens(form):
    """Above the gate the recurrent mixer sees only the kept tokens, in order:
    q, k, v and the gates gathered by tg_compact, then scanned, equal the
    oracle's scan over the kept subsequence (and, bit for bit, a scan over
    the same rows gathered on the host)."""
    n, K = 1024, 192
    q, k, v, alpha, beta, _ = _case(10, n, 2, 4, 128, 128, False)
    kept = np.sort(np.random.default_rng(11).choice(n, size=K, replace=False)).astype(np.int32)
    dev = gu.dev()
    src = [gu.bf16(q), gu.bf16(k), gu.bf16(v), gu.f32(alpha), gu.f32(beta)]
    dst = [torch.empty((K,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev) for t in src]
    gu.say(f"gated delta rule ({form}) over compacted kept tokens n=1024 K=192")
    tg.tg_compact(gu.i32(kept), n, None, None, None, None, None, None, extra=list(zip(src, dst)))
    out = torch.empty(K, 4, 128, dtype=torch.float32, device=dev)
    _mixer(form, *dst, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    w = oracle.widen_bf16
    want, _ = gdn.gated_delta_rule(w(q[kept]), w(k[kept]), w(v[kept]), alpha[kept], beta[kept])
    assert _rel(got, want) <= TOL
    host_o, _ = _run(q[kept], k[kept], v[kept], alpha[kept], beta[kept], None, form)
    assert np.array_equal(got, host_o)
