"""Acceptance checks of GPU outputs against the FP64 oracle.

Tolerance (fixed by the benchmark spec of the fused 4-bit GEMV study, and
consistent with the 0.25-0.35% relative RMSE the Lab 5 page reports in
"INT4 融合 GEMV" against a BF16-weight reference):
  * relative RMSE over one call's outputs  ||y - y_ref||_2 / ||y_ref||_2 <= 4e-3
  * per element (m, n)  |y - y_ref| <= 2e-2 * ||x_m||_2 * max_k |W[n, k]|
where y_ref is the unrounded FP64 oracle result.
"""
from __future__ import annotations

import numpy as np

REL_RMSE_MAX = 4e-3
ELEM_FACTOR = 2e-2


def check_outputs(y, y_ref, x_norm, w_absmax, what=""):
    """y, y_ref: [M, N] (or [N]); x_norm: [M] (or scalar); w_absmax: [N]."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    y_ref = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = y - y_ref
    rel = float(np.sqrt(np.sum(err ** 2) / max(np.sum(y_ref ** 2), 1e-300)))
    assert rel <= REL_RMSE_MAX, f"{what}: relative RMSE {rel:.3e} > {REL_RMSE_MAX}"
    bound = ELEM_FACTOR * np.asarray(x_norm, dtype=np.float64).reshape(-1, 1) * \
        np.asarray(w_absmax, dtype=np.float64).reshape(1, -1)
    worst = float(np.max(np.abs(err) / bound))
    assert worst <= 1.0, f"{what}: element error {worst:.3f} x the per-element bound"
    return rel, worst
