"""Shared test plumbing: moving seeded inputs to the GPU and back, error metrics.

Holds no method arithmetic: expected values always come from the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_cross_amd import inputs

DEV = "cuda"

# Tolerances: bf16 inputs -> max abs <= 2e-2 and relative Frobenius <= 1e-2,
# LSE <= 1e-3 absolute; fp32 inputs -> 1e-5 relative.
BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
LSE_ABS = 1e-3
F32_REL = 1e-5


def to_dev(x: np.ndarray, device=DEV) -> torch.Tensor:
    """Generated array (bf16 bits as uint16, or fp32/int) -> device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact fp64 numpy values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def vals64(x: np.ndarray) -> np.ndarray:
    """Generated array -> exact fp64 values."""
    return inputs.as_f32(x).astype(np.float64)


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def assert_close_bf16(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    assert np.isfinite(got).all(), what + ": non-finite values"
    mx = float(np.abs(got - ref).max()) if got.size else 0.0
    rf = rel_fro(got, ref)
    assert mx <= BF16_MAX_ABS and rf <= BF16_REL_FRO, "%s: max abs %.3e, rel fro %.3e" % (what, mx, rf)


def assert_close_f32(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    assert np.isfinite(got).all(), what + ": non-finite values"
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(got - ref).max()) / scale if got.size else 0.0
    rf = rel_fro(got, ref)
    assert err <= F32_REL and rf <= F32_REL, "%s: rel max %.3e, rel fro %.3e" % (what, err, rf)


def assert_lse(got: np.ndarray, ref: np.ndarray, what: str = "lse", tol: float = LSE_ABS) -> None:
    ninf_ref = np.isneginf(ref)
    assert (np.isneginf(got) == ninf_ref).all(), what + ": -inf pattern differs"
    fin = ~ninf_ref
    if fin.any():
        err = float(np.abs(got[fin] - ref[fin]).max())
        assert err <= tol, "%s: max abs %.3e" % (what, err)


def rank_of_max_load(load: np.ndarray) -> int:
    """The critical-path rank: largest load, lowest index on ties."""
    return int(np.argmax(load))
