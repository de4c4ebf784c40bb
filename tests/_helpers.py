"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# tolerances (bf16 outputs; lse absolute)
O_ATOL, O_RTOL, LSE_ATOL = 1e-2, 1e-2, 1e-3


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits: np.ndarray) -> np.ndarray:
    # NaN bit patterns (poisoned rows outside the sequences) stay NaN
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_o_close(got, ref, what="o", atol=O_ATOL, rtol=O_RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    excess = np.abs(got - ref) - rtol * np.abs(ref)
    worst = float(excess.max()) if excess.size else 0.0
    idx = np.unravel_index(int(np.argmax(excess)), excess.shape) if excess.size else None
    assert worst <= atol, f"{what}: |err| - rtol|ref| = {worst:.3e} > {atol} at {idx} (got {got[idx]}, ref {ref[idx]})"
    return float(np.abs(got - ref).max()) if got.size else 0.0


def assert_lse_close(got, ref, what="lse", atol=LSE_ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both are -inf: masked out below
        d = np.where(both_inf, 0.0, np.abs(got - ref))
    worst = float(np.nanmax(d)) if d.size else 0.0
    assert not np.isnan(d).any() and worst <= atol, f"{what}: max |err| {worst:.3e} > {atol}"
    return worst


def log(msg: str) -> None:
    print(msg, flush=True)
