"""Helpers for the GPU parity tests (inputs from synth, expected values from
the oracle, never from the GPU path)."""
from __future__ import annotations

import numpy as np
import torch

# Per-row bound of the integer-dot paths: max|y - y_ref| / max|y_ref| per row.
ROW_TOL = 1e-4


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def poisoned(shape, dtype=torch.float32) -> torch.Tensor:
    """Output buffer filled with NaN (floats) or 0xA5 bytes, so an element the
    kernel never writes cannot pass as a result."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(0xA5)
    return t


def row_errors(y: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """max|y - y_ref| / max|y_ref| per row (0 where both rows are all zero,
    inf where the reference row is zero but y is not)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.max(np.abs(y - y_ref), axis=1)
    scale = np.max(np.abs(y_ref), axis=1)
    out = np.zeros(len(err))
    nz = scale > 0
    out[nz] = err[nz] / scale[nz]
    out[~nz] = np.where(err[~nz] == 0, 0.0, np.inf)
    return out


def assert_rows_close(y: np.ndarray, y_ref: np.ndarray, tol: float = ROW_TOL, what: str = "") -> float:
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: {np.sum(~np.isfinite(y))} outputs not written (NaN poison left)"
    # Outputs that a kernel adds into a Y zeroed beforehand are not covered
    # by the NaN poison: an element nobody wrote would stay 0.  A computed
    # fp32 result is exactly 0 only if the reference is (about) 0 too, so a
    # zero where the reference is far from 0 means "not written".
    big = np.abs(y_ref) > 1e-6 * np.max(np.abs(y_ref), axis=1, keepdims=True)
    unwritten = (np.asarray(y) == 0) & big
    assert not unwritten.any(), f"{what}: {int(unwritten.sum())} outputs are 0 where the reference is not"
    e = row_errors(y, y_ref)
    worst = int(np.argmax(e))
    assert e[worst] <= tol, f"{what}: row {worst} error {e[worst]:.3e} > {tol:g}"
    return float(e.max())
