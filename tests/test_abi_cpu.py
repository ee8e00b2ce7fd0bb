"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before anything reaches the GPU.

No call here enqueues GPU work: each one either fails a host-side check or is
a documented no-op (empty input).  Fake pointers are never dereferenced,
because every check runs before any HIP call."""
import ctypes
import os
import re

import pytest

from learned_token_pruning_mlp_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")

A = 1 << 20  # a 16-byte-aligned fake address (never dereferenced)
M = A + 2    # a misaligned one
WS = 1 << 24  # generous workspace size claimed for the fake buffer


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_status_and_workspace(lib):
    assert binding.tg_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert binding.tg_status_string(code) != "unknown status"
    assert binding.tg_status_string(12345) == "unknown status"
    # a workspace sized for a prompt serves every shorter one, across the
    # sizes where the select changes form or chunk size
    ns = (0, 1, 512, 16384, 16385, 32768, 131072, 131073, 262144, 262145, 524288, 524289, 1 << 20)
    sizes = [binding.tg_workspace_bytes(n) for n in ns]
    assert all(s > 0 and s % 256 == 0 for s in sizes)
    assert sizes == sorted(sizes)


def _gate(lib, **kw):
    a = dict(resid=A, w1=A, b1=None, w2=A, b2=0.0, n=512, d=256, hd=64, eps_row=1e-6, eps_seq=1e-6,
             score_norm=A, score_raw=None, ws=A, ws_bytes=WS, stream=None)
    a.update(kw)
    return lib.tg_gate_score(a["resid"], a["w1"], a["b1"], a["w2"], a["b2"], a["n"], a["d"], a["hd"],
                             a["eps_row"], a["eps_seq"], a["score_norm"], a["score_raw"], a["ws"],
                             a["ws_bytes"], a["stream"])


def test_gate_score_checks(lib):
    E = binding
    assert _gate(lib, n=0) == E.TG_OK  # empty prompt: no-op
    assert _gate(lib, n=-1) == E.TG_EINVAL
    assert _gate(lib, d=200) == E.TG_EUNSUPPORTED
    assert _gate(lib, hd=96) == E.TG_EUNSUPPORTED
    assert _gate(lib, resid=None) == E.TG_EINVAL
    assert _gate(lib, score_norm=None) == E.TG_EINVAL
    assert _gate(lib, resid=M) == E.TG_EALIGN
    assert _gate(lib, w1=M) == E.TG_EALIGN
    assert _gate(lib, ws=None) == E.TG_EWORKSPACE
    assert _gate(lib, ws_bytes=binding.tg_workspace_bytes(512) - 1) == E.TG_EWORKSPACE
    assert _gate(lib, eps_row=-1.0) == E.TG_EINVAL
    assert _gate(lib, eps_seq=float("nan")) == E.TG_EINVAL


def _sel(lib, **kw):
    a = dict(score=A, forced=A, n=1000, nf=10, k=100, kept=A, st=None, ws=A, ws_bytes=WS, stream=None)
    a.update(kw)
    return lib.tg_select_topk(a["score"], a["forced"], a["n"], a["nf"], a["k"], a["kept"], a["st"], a["ws"],
                              a["ws_bytes"], a["stream"])


def test_select_checks(lib):
    E = binding
    assert _sel(lib, k=0) == E.TG_EINVAL
    assert _sel(lib, k=1001) == E.TG_EINVAL
    assert _sel(lib, n=0, k=0) == E.TG_EINVAL
    assert _sel(lib, nf=101) == E.TG_EINVAL  # more forced than the budget
    assert _sel(lib, nf=-1) == E.TG_EINVAL
    assert _sel(lib, forced=None) == E.TG_EINVAL  # forced count without a mask
    assert _sel(lib, score=None) == E.TG_EINVAL
    assert _sel(lib, kept=None) == E.TG_EINVAL
    assert _sel(lib, score=A + 4) == E.TG_EALIGN
    assert _sel(lib, forced=A + 2) == E.TG_EALIGN
    assert _sel(lib, ws=None) == E.TG_EWORKSPACE
    assert _sel(lib, ws_bytes=16) == E.TG_EWORKSPACE


def _gsel(lib, **kw):
    a = dict(resid=A, w1=A, b1=None, w2=A, b2=0.0, n=1000, d=256, hd=64, eps_row=1e-6, eps_seq=1e-6, forced=A,
             nf=10, k=100, score_norm=A, score_raw=None, kept=A, st=None, ws=A, ws_bytes=WS, stream=None)
    a.update(kw)
    return lib.tg_gate_score_select(a["resid"], a["w1"], a["b1"], a["w2"], a["b2"], a["n"], a["d"], a["hd"],
                                    a["eps_row"], a["eps_seq"], a["forced"], a["nf"], a["k"], a["score_norm"],
                                    a["score_raw"], a["kept"], a["st"], a["ws"], a["ws_bytes"], a["stream"])


def test_gate_score_select_checks(lib):
    """Both calls' checks: the scorer's shapes and the select's budget."""
    E = binding
    assert _gsel(lib, n=0, k=0) == E.TG_EINVAL  # the select needs a token
    assert _gsel(lib, k=0) == E.TG_EINVAL
    assert _gsel(lib, k=1001) == E.TG_EINVAL
    assert _gsel(lib, nf=101) == E.TG_EINVAL
    assert _gsel(lib, forced=None) == E.TG_EINVAL
    assert _gsel(lib, d=200) == E.TG_EUNSUPPORTED
    assert _gsel(lib, hd=96) == E.TG_EUNSUPPORTED
    assert _gsel(lib, eps_seq=-1.0) == E.TG_EINVAL
    assert _gsel(lib, resid=None) == E.TG_EINVAL
    assert _gsel(lib, kept=None) == E.TG_EINVAL
    assert _gsel(lib, score_norm=A + 4) == E.TG_EALIGN  # the select reads it in 16-byte pieces
    assert _gsel(lib, w1=M) == E.TG_EALIGN
    assert _gsel(lib, forced=A + 2) == E.TG_EALIGN
    assert _gsel(lib, ws=None) == E.TG_EWORKSPACE
    assert _gsel(lib, ws_bytes=binding.tg_workspace_bytes(1000) - 1) == E.TG_EWORKSPACE


def _cmp(lib, **kw):
    a = dict(idx=A, k=64, n=512, resid=A, resid_out=A, d=256, pos=None, pos_out=A, score=A, score_out=A,
             extra=None, n_extra=0, stream=None)
    a.update(kw)
    return lib.tg_compact(a["idx"], a["k"], a["n"], a["resid"], a["resid_out"], a["d"], a["pos"], a["pos_out"],
                          a["score"], a["score_out"], a["extra"], a["n_extra"], a["stream"])


def test_compact_checks(lib):
    E = binding
    assert _cmp(lib, k=0) == E.TG_OK  # nothing kept: no-op
    assert _cmp(lib, k=-1) == E.TG_EINVAL
    assert _cmp(lib, n=0) == E.TG_EINVAL
    assert _cmp(lib, idx=None) == E.TG_EINVAL
    assert _cmp(lib, resid_out=None) == E.TG_EINVAL
    assert _cmp(lib, d=100) == E.TG_EALIGN  # 200-byte rows
    assert _cmp(lib, resid=M) == E.TG_EALIGN
    assert _cmp(lib, score=None) == E.TG_EINVAL  # score_out without score
    assert _cmp(lib, n_extra=17) == E.TG_EINVAL
    assert _cmp(lib, n_extra=1, extra=None) == E.TG_EINVAL
    bad = (binding.TgGather * 1)(binding.TgGather(A, A, 24, 32, 32))
    assert _cmp(lib, n_extra=1, extra=bad) == E.TG_EALIGN
    bad = (binding.TgGather * 1)(binding.TgGather(A, A, 64, 32, 64))
    assert _cmp(lib, n_extra=1, extra=bad) == E.TG_EINVAL  # stride shorter than a row
    bad = (binding.TgGather * 1)(binding.TgGather(None, A, 64, 64, 64))
    assert _cmp(lib, n_extra=1, extra=bad) == E.TG_EINVAL
    bad = (binding.TgGather * 1)(binding.TgGather(A + 8, A, 64, 64, 64))
    assert _cmp(lib, n_extra=1, extra=bad) == E.TG_EALIGN


def test_rope_checks(lib):
    E = binding
    assert lib.tg_rope(A, A, 0, 8, 128, 1e6, None) == E.TG_OK
    assert lib.tg_rope(A, A, 10, 8, 127, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope(A, A, 10, 8, 512, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope(A, A, 10, 0, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope(A, A, 10, 8, 128, 0.0, None) == E.TG_EINVAL
    assert lib.tg_rope(None, A, 10, 8, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope(A + 1, A, 10, 8, 128, 1e6, None) == E.TG_EALIGN


def test_rope_qk_checks(lib):
    E = binding
    assert lib.tg_rope_qk(A, A, A, 0, 16, 8, 128, 1e6, None) == E.TG_OK
    assert lib.tg_rope_qk(A, A, A, 10, 16, 0, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A, A, 10, 0, 8, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A, A, 10, 16, 8, 127, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A, A, 10, 16, 8, 258, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A, A, -1, 16, 8, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A, A, 10, 16, 8, 128, -1.0, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, None, A, 10, 16, 8, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A, None, 10, 16, 8, 128, 1e6, None) == E.TG_EINVAL
    assert lib.tg_rope_qk(A, A + 1, A, 10, 16, 8, 128, 1e6, None) == E.TG_EALIGN
    assert lib.tg_rope_qk(A, A, A + 2, 10, 16, 8, 128, 1e6, None) == E.TG_EALIGN


def _att(lib, **kw):
    a = dict(q=A, k=A, v=A, ks=A, g=A, c=0.1, pos=A, nk=128, hq=4, hkv=2, D=64, out=A, od=0, stream=None)
    a.update(kw)
    return lib.tg_gated_attention(a["q"], a["k"], a["v"], a["ks"], a["g"], a["c"], a["pos"], a["nk"], a["hq"],
                                  a["hkv"], a["D"], a["out"], a["od"], a["stream"])


def test_attention_checks(lib):
    E = binding
    assert _att(lib, nk=0) == E.TG_OK  # nothing kept: no-op
    assert _att(lib, nk=-5) == E.TG_EINVAL
    assert _att(lib, hq=6, hkv=4) == E.TG_EINVAL
    assert _att(lib, hkv=0) == E.TG_EINVAL
    assert _att(lib, D=96) == E.TG_EUNSUPPORTED
    assert _att(lib, nk=1 << 20, hq=16, hkv=8, D=128) == E.TG_EUNSUPPORTED  # K, V of 2 GiB
    assert _att(lib, nk=(1 << 20) - 1, hq=16, hkv=8, D=128, q=None) == E.TG_EINVAL  # just under: size accepted
    assert _att(lib, od=2) == E.TG_EINVAL
    assert _att(lib, c=float("nan")) == E.TG_EINVAL
    assert _att(lib, q=None) == E.TG_EINVAL
    assert _att(lib, pos=None) == E.TG_EINVAL
    assert _att(lib, q=M) == E.TG_EALIGN
    assert _att(lib, out=A + 8) == E.TG_EALIGN


def test_layer_piece_checks(lib):
    E = binding
    # tg_rmsnorm(x, w, y, rows, dim, eps, stream)
    assert lib.tg_rmsnorm(A, A, A, 0, 128, 1e-6, None) == E.TG_OK  # no rows: no-op
    assert lib.tg_rmsnorm(A, A, A, -1, 128, 1e-6, None) == E.TG_EINVAL
    assert lib.tg_rmsnorm(A, A, A, 4, 12, 1e-6, None) == E.TG_EINVAL    # dim not a multiple of 8
    assert lib.tg_rmsnorm(A, A, A, 4, 8192, 1e-6, None) == E.TG_EINVAL  # dim above 4096
    assert lib.tg_rmsnorm(A, A, A, 4, 128, -1.0, None) == E.TG_EINVAL
    assert lib.tg_rmsnorm(None, A, A, 4, 128, 1e-6, None) == E.TG_EINVAL
    assert lib.tg_rmsnorm(M, A, A, 4, 128, 1e-6, None) == E.TG_EALIGN
    assert lib.tg_rmsnorm(A, A, M, 4, 128, 1e-6, None) == E.TG_EALIGN
    # tg_swiglu(gate_up, out, rows, inter, stream)
    assert lib.tg_swiglu(A, A, 0, 512, None) == E.TG_OK
    assert lib.tg_swiglu(A, A, 4, 12, None) == E.TG_EINVAL
    assert lib.tg_swiglu(None, A, 4, 512, None) == E.TG_EINVAL
    assert lib.tg_swiglu(A, M, 4, 512, None) == E.TG_EALIGN
    # tg_linear(handle, x, w, residual, y, rows, in_dim, out_dim, stream)
    assert lib.tg_linear(None, A, A, None, A, 4, 64, 64, None) == E.TG_EINVAL  # no handle
    assert lib.tg_linear(A, A, A, None, A, 0, 64, 64, None) == E.TG_EINVAL
    assert lib.tg_linear(A, A, A, None, A, 4, 0, 64, None) == E.TG_EINVAL
    assert lib.tg_linear(A, None, A, None, A, 4, 64, 64, None) == E.TG_EINVAL
    assert lib.tg_blas_create(None) == E.TG_EINVAL
    assert lib.tg_blas_destroy(None) == E.TG_EINVAL


def _bwd(lib, n=64, hq=4, hkv=2, D=64, c=0.1, ws=A, ws_bytes=WS, **over):
    p = dict(q=A, k=A, v=A, s=A, g=A, pos=A, dout=A, dq=A, dk=A, dv=A, ds=A, dg=A, dc=A)
    p.update(over)
    return lib.tg_gated_attention_bwd(p["q"], p["k"], p["v"], p["s"], p["g"], c, p["pos"], n, hq, hkv, D, p["dout"],
                                      p["dq"], p["dk"], p["dv"], p["ds"], p["dg"], p["dc"], ws, ws_bytes, None)


def test_attention_backward_checks(lib):
    E = binding
    need = lib.tg_attention_bwd_workspace_bytes(64, 4, 2, 64)
    assert 0 < need <= WS
    # the workspace grows with the kept rows and the heads
    assert lib.tg_attention_bwd_workspace_bytes(4096, 16, 8, 128) > lib.tg_attention_bwd_workspace_bytes(64, 16, 8, 128)
    assert lib.tg_attention_bwd_workspace_bytes(-1, 4, 2, 64) == 0
    assert _bwd(lib, n=0) == E.TG_OK  # nothing kept: no-op
    assert _bwd(lib, n=-1) == E.TG_EINVAL
    assert _bwd(lib, hq=3, hkv=2) == E.TG_EINVAL
    assert _bwd(lib, D=96) == E.TG_EUNSUPPORTED
    assert _bwd(lib, c=float("nan")) == E.TG_EINVAL
    assert _bwd(lib, q=None) == E.TG_EINVAL
    assert _bwd(lib, dc=None) == E.TG_EINVAL
    assert _bwd(lib, dout=M) == E.TG_EALIGN
    assert _bwd(lib, dk=M) == E.TG_EALIGN
    assert _bwd(lib, ws=None) == E.TG_EWORKSPACE
    assert _bwd(lib, ws_bytes=need - 1) == E.TG_EWORKSPACE
    assert _bwd(lib, ws=A + 16) == E.TG_EALIGN  # workspace must be 256-byte aligned
    # Q and dout are read through 32-bit buffer offsets: 2 GiB each at most
    # (64 q heads of 128 over 131072 rows is exactly 2 GiB; 8 kv heads keep K/V at 256 MiB)
    assert _bwd(lib, n=131072, hq=64, hkv=8, D=128) == E.TG_EUNSUPPORTED
    assert _bwd(lib, n=131071, hq=64, hkv=8, D=128, ws_bytes=0) == E.TG_EWORKSPACE  # sizes pass, then the workspace check


def _gbw(lib, blas=A, n=64, d=128, hd=64, k=8, er=1e-6, es=1e-6, ws=A, ws_bytes=WS, **over):
    p = dict(resid=A, w1=A, b1=None, w2=A, s=A, dsk=A, idx=A, dres=A, dw1=A, db1=A, dw2=A, db2=A)
    p.update(over)
    return lib.tg_gate_score_bwd(blas, p["resid"], p["w1"], p["b1"], p["w2"], n, d, hd, er, es, p["s"], p["dsk"],
                                 p["idx"], k, p["dres"], p["dw1"], p["db1"], p["dw2"], p["db2"], ws, ws_bytes, None)


def test_gate_score_backward_checks(lib):
    E = binding
    need = lib.tg_gate_score_bwd_workspace_bytes(64, 128, 64)
    assert 0 < need <= WS
    assert lib.tg_gate_score_bwd_workspace_bytes(16384, 2048, 256) > lib.tg_gate_score_bwd_workspace_bytes(64, 2048, 256)
    assert lib.tg_gate_score_bwd_workspace_bytes(-1, 128, 64) == 0
    assert _gbw(lib, n=0, k=0) == E.TG_OK  # no tokens: no-op
    assert _gbw(lib, blas=None) == E.TG_EINVAL  # no rocBLAS handle
    assert _gbw(lib, n=-1) == E.TG_EINVAL
    assert _gbw(lib, k=65) == E.TG_EINVAL  # more kept than tokens
    assert _gbw(lib, er=-1.0) == E.TG_EINVAL
    assert _gbw(lib, es=float("nan")) == E.TG_EINVAL
    assert _gbw(lib, hd=96) == E.TG_EUNSUPPORTED
    assert _gbw(lib, d=96) == E.TG_EUNSUPPORTED
    assert _gbw(lib, d=8192) == E.TG_EUNSUPPORTED
    assert _gbw(lib, resid=None) == E.TG_EINVAL
    assert _gbw(lib, db2=None) == E.TG_EINVAL
    assert _gbw(lib, idx=None) == E.TG_EINVAL  # k > 0 needs the kept indices
    assert _gbw(lib, resid=M) == E.TG_EALIGN
    assert _gbw(lib, dres=A + 4) == E.TG_EALIGN
    assert _gbw(lib, dw1=A + 8) == E.TG_EALIGN
    assert _gbw(lib, ws=None) == E.TG_EWORKSPACE
    assert _gbw(lib, ws_bytes=need - 1) == E.TG_EWORKSPACE
    assert _gbw(lib, ws=A + 16) == E.TG_EALIGN


def test_gated_delta_rule_checks(lib):
    E = binding

    def call(n=16, hk=2, hv=4, dk=128, dv=128, q=A, k=A, v=A, al=A, be=A, si=None, out=A, so=None):
        return lib.tg_gated_delta_rule(q, k, v, al, be, si, n, hk, hv, dk, dv, out, so, None)
    assert call(n=0) == E.TG_OK  # no tokens, no state out: no-op
    assert call(n=-1) == E.TG_EINVAL
    assert call(hk=3, hv=4) == E.TG_EINVAL
    assert call(hk=0) == E.TG_EINVAL
    assert call(dk=96) == E.TG_EUNSUPPORTED
    assert call(dv=256) == E.TG_EUNSUPPORTED
    assert call(q=None) == E.TG_EINVAL
    assert call(be=None) == E.TG_EINVAL
    assert call(out=None) == E.TG_EINVAL
    assert call(k=M) == E.TG_EALIGN
    assert call(si=A + 4) == E.TG_EALIGN
    assert call(so=A + 8) == E.TG_EALIGN


def test_gated_delta_rule_chunked_checks(lib):
    """The chunked form takes the scan's checks, then its workspace's."""
    E = binding
    wsb = lib.tg_gated_delta_rule_workspace_bytes
    assert wsb(-1, 4) == 0 and wsb(16, 0) == 0
    assert wsb(0, 4) == wsb(32, 4) == 4 * 16384  # one 16 KB record per (v head, chunk of 32)
    assert wsb(33, 4) == 2 * 4 * 16384
    sizes = [wsb(n, 16) for n in range(0, 5000, 37)]
    assert sizes == sorted(sizes)

    def call(n=16, hk=2, hv=4, dk=128, dv=128, q=A, k=A, v=A, al=A, be=A, si=None, out=A, so=None, ws=A,
             wsn=None):
        wsn = wsb(max(n, 0), hv) if wsn is None else wsn
        return lib.tg_gated_delta_rule_chunked(q, k, v, al, be, si, n, hk, hv, dk, dv, out, so, ws, wsn, None)
    assert call(n=0, ws=None, wsn=0) == E.TG_OK  # no tokens, no state out: no-op
    assert call(n=-1) == E.TG_EINVAL
    assert call(hk=3, hv=4) == E.TG_EINVAL
    assert call(dk=96) == E.TG_EUNSUPPORTED
    assert call(q=None) == E.TG_EINVAL
    assert call(k=M) == E.TG_EALIGN
    assert call(so=A + 8) == E.TG_EALIGN
    assert call(ws=None) == E.TG_EWORKSPACE
    assert call(wsn=wsb(16, 4) - 1) == E.TG_EWORKSPACE
    assert call(ws=M) == E.TG_EALIGN


def test_kept_budget_semantics():
    """The user budget is a maximum: K = min(max_kept, n); the never-pruned
    question tokens must fit in it."""
    assert binding.kept_budget(16384, 64, 2048) == 2048
    assert binding.kept_budget(1000, 64, 2048) == 1000  # short prompt: everything kept
    assert binding.kept_budget(1000, 64, 64) == 64       # exactly the forced tokens
    assert binding.kept_budget(1000, 0, 1) == 1
    for args in ((1000, 64, 63), (1000, 0, 0), (0, 0, 5), (1000, 1001, 2000), (1000, -1, 10)):
        with pytest.raises(ValueError):
            binding.kept_budget(*args)
