"""Helpers for the GPU parity tests: move seeded inputs to the device, read
results back, and the tolerance checks stated once."""
import sys

import numpy as np
import torch

ATTN_MAX_ABS = 1e-2     # fp32-output max |O_gpu - O_ref|
ATTN_REL_RMS = 5e-3     # ||O_gpu - O_ref|| / ||O_ref||
SCORE_ABS = 1e-4        # |s^_gpu - s^_ref|


def say(msg: str):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 GPU tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 GPU tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_attention(got: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(got.astype(np.float64) - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-30))
    assert max_abs <= ATTN_MAX_ABS, f"{what}: max abs {max_abs:.3e}"
    assert rel <= ATTN_REL_RMS, f"{what}: rel rms {rel:.3e}"
    return max_abs, rel


def boundary_gap(ref_norm: np.ndarray, forced: np.ndarray, k: int):
    """(gap, cut): the oracle-score distance between the worst kept and the
    best dropped prunable token at budget k, and their midpoint; None when
    every prunable token is kept or none is."""
    prun = np.flatnonzero(forced == 0)
    r = k - int(np.count_nonzero(forced))
    if r <= 0 or r >= prun.size:
        return None
    order = prun[np.lexsort((prun, -ref_norm[prun]))]
    a, b = ref_norm[order[r - 1]], ref_norm[order[r]]
    return float(a - b), 0.5 * float(a + b)


def assert_kept_matches_oracle(got_kept: np.ndarray, ref_norm: np.ndarray, forced: np.ndarray, k: int,
                               what: str, score_tol: float = SCORE_ABS):
    """The GPU's kept set against the oracle's top-K of the oracle's own
    normalised scores.  The GPU selects on its scores, which are within
    score_tol of the oracle's, so when the oracle's boundary gap exceeds
    2 * score_tol the sets must be identical (bit-exact); otherwise only the
    tokens within 2 * score_tol of the cut may differ, and the count, the
    order and the forced tokens are still checked.  Returns the gap."""
    from oracle import oracle as _o
    ref_kept = _o.select_topk(ref_norm, forced, k)
    got_kept = np.asarray(got_kept)
    assert got_kept.shape == (k,), f"{what}: kept count"
    assert np.all(np.diff(got_kept) > 0), f"{what}: not ascending"
    assert np.all(np.isin(np.flatnonzero(forced), got_kept)), f"{what}: a forced token was dropped"
    gc = boundary_gap(ref_norm, forced, k)
    if gc is None or gc[0] > 2 * score_tol:
        assert np.array_equal(got_kept, ref_kept), f"{what}: kept set differs from the oracle's"
        return None if gc is None else gc[0]
    band = np.abs(ref_norm - gc[1]) <= 2 * score_tol
    diff = np.setxor1d(got_kept, ref_kept)
    assert np.all(band[diff]), f"{what}: kept set differs outside the rounding band of the cut"
    say(f"  {what}: oracle boundary gap {gc[0]:.2e} <= {2 * score_tol:.0e}; "
        f"{diff.size // 2} swap(s) inside the band allowed")
    return gc[0]


def check_attention_bf16(got_bits: np.ndarray, ref: np.ndarray, what: str):
    """bf16 attention output against the fp64 oracle: relative RMS as for the
    fp32 output, and every element within one bf16 unit of the oracle's
    nearest-even rounding or within the fp32 max-abs bound (a bf16 half-unit
    at |O| in [4, 8) alone exceeds that bound)."""
    from oracle import oracle as _o
    got = bf16_to_f64(got_bits)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert rel <= ATTN_REL_RMS, f"{what}: rel rms {rel:.3e}"
    ref_b = bf16_to_f64(_o.to_bf16(ref))
    # one unit of the bf16 grid at the rounded oracle value (2^(e-7) for |x| in [2^e, 2^(e+1)))
    mag = np.maximum(np.abs(ref_b), np.finfo(np.float32).tiny)
    ulp = np.ldexp(1.0, np.floor(np.log2(mag)).astype(np.int64) - 7)
    err = np.abs(got - ref_b)
    ok = (err <= ulp) | (np.abs(got - ref) <= ATTN_MAX_ABS)
    assert ok.all(), f"{what}: {int((~ok).sum())} bf16 outputs off by more than one unit (max {err.max():.3e})"
    return rel
