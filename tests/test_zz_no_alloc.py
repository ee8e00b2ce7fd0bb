"""tg_gate_score_noalloc (the scorer with its scratch in a fixed device array
inside the library) against tg_gate_score (the same kernels with a caller
workspace): two calls in a row on one device, the second on a smaller prompt,
each bit-identical to the workspace entry point on the same inputs.  The
limit is rejected on the host."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from learned_token_pruning_mlp_amd import binding as tg
from learned_token_pruning_mlp_amd import synth

pytestmark = pytest.mark.gpu


def _both(shp, seed, with_b1):
    inp = synth.gate_inputs(shp, seed, with_b1=with_b1)
    resid, w1, w2 = gu.bf16(inp.resid), gu.bf16(inp.w1), gu.bf16(inp.w2)
    b1 = None if inp.b1 is None else gu.bf16(inp.b1)
    f32 = dict(dtype=torch.float32, device=gu.dev())
    want_n, want_r = torch.empty(shp.n, **f32), torch.empty(shp.n, **f32)
    tg.tg_gate_score(resid, w1, b1, w2, 0.25, 1e-6, 1e-6, want_n, want_r, tg.workspace(shp.n))
    got_n, got_r = torch.full((shp.n,), float("nan"), **f32), torch.full((shp.n,), float("nan"), **f32)
    tg.tg_gate_score_noalloc(resid, w1, b1, w2, 0.25, 1e-6, 1e-6, got_n, got_r)
    return [gu.host(t).view(np.uint32) for t in (want_n, want_r, got_n, got_r)]


def test_noalloc_matches_workspace_entry_point_twice():
    big = synth.QWEN3_1P7B_N16K
    small = synth.GateShape(n=1000, d=512, hd=128, n_forced=8, k=64, hq=4, hkv=2, head_dim=64)
    for shp, seed, b1 in ((big, 31, False), (small, 32, True)):
        gu.say(f"gate_score_noalloc n={shp.n} d={shp.d} hd={shp.hd}")
        wn, wr, gn, gr = _both(shp, seed, b1)
        assert np.array_equal(gn, wn) and np.array_equal(gr, wr)


def test_noalloc_rejects_prompts_beyond_its_scratch():
    lib = tg.load()
    A = 1 << 20
    assert lib.tg_gate_score_noalloc(A, A, None, A, 0.0, (1 << 22) + 1, 2048, 256, 1e-6, 1e-6, A, None,
                                     None) == tg.TG_EUNSUPPORTED
