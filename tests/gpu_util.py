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
