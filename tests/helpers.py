"""Shared test helpers: the output tolerance and device/host conversions."""

from __future__ import annotations

import numpy as np
import torch

# Output tolerance for y against the float64 oracle, per call, over the whole
# output tensor: relative Frobenius error and max abs error over rms(y).
# Budget: bf16 rounding of y (~1.1e-3 relative rms, at most 2^-9 |y|) plus,
# on the prefill path, bf16 rounding of W_eff (~1.1e-3 relative rms).
REL_FRO_TOL = 5e-3
MAX_ABS_OVER_RMS_TOL = 2e-2


def bits16(t: torch.Tensor) -> np.ndarray:
    """Host uint16 bit patterns of a bf16 tensor."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def packed_u64(p: torch.Tensor) -> np.ndarray:
    return p.detach().cpu().contiguous().numpy().view(np.uint64)


def alpha_bits(a: torch.Tensor) -> np.ndarray:
    return a.detach().cpu().contiguous().numpy().view(np.uint32)


def y_error(y_dev: torch.Tensor, y_ref: np.ndarray):
    """(rel_fro, max_abs / rms) of a bf16 device output against float64."""
    y = y_dev.detach().float().cpu().numpy().astype(np.float64).reshape(y_ref.shape)
    fin = np.isfinite(y_ref)
    assert np.array_equal(np.isfinite(y), fin), "non-finite outputs differ from the oracle"
    if not fin.any():
        return 0.0, 0.0
    err = (y - y_ref)[fin]
    ref = y_ref[fin]
    nref = float(np.linalg.norm(ref))
    rms = float(np.sqrt(np.mean(ref * ref)))
    if nref == 0.0:
        return float(np.linalg.norm(err)), float(np.max(np.abs(err)))
    return float(np.linalg.norm(err)) / nref, float(np.max(np.abs(err))) / rms


def assert_y_close(y_dev, y_ref, what="", min_finite=0.5):
    """Within the tolerance, and the comparison is not vacuous: at least
    min_finite of the reference values are finite."""
    frac = float(np.mean(np.isfinite(y_ref)))
    assert frac >= min_finite, f"{what}: only {frac:.1%} of the reference outputs are finite"
    rel, mx = y_error(y_dev, y_ref)
    assert rel <= REL_FRO_TOL and mx <= MAX_ABS_OVER_RMS_TOL, (
        f"{what}: rel_fro={rel:.3e} (tol {REL_FRO_TOL}), max_abs/rms={mx:.3e} "
        f"(tol {MAX_ABS_OVER_RMS_TOL})")
    return rel, mx
