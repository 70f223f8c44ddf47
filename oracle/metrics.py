"""Error metrics used by the parity tests (test infrastructure only).

The gated figure is the per-row infinity-norm relative error
``max_{b,h,i} |o_hat_i - o_i|_inf / |o_i|_inf``. Outputs are weighted means of
the values, so single coordinates can sit arbitrarily close to zero and an
elementwise ratio would measure noise; a row's own largest coordinate is the
natural scale of its errors.
"""
from __future__ import annotations

import numpy as np


def rowwise_rel_err(got, ref):
    """Max over rows (all leading axes) of |got - ref|_inf / |ref|_inf.

    A row whose reference is exactly zero contributes 0 if ``got`` is zero
    there too and +inf otherwise.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    if got.size == 0:
        return 0.0
    diff = np.max(np.abs(got - ref), axis=-1)
    scale = np.max(np.abs(ref), axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0),
                       np.where(diff > 0, np.inf, 0.0))
    if np.any(np.isnan(got)):
        return float("inf")
    return float(np.max(rel))
