"""Comparison rules between a device result and the fp64 oracle.

official:  max |gpu - ref| <= 1e-2 * (1 + |ref|)            (elementwise)
strict:    |gpu - ref| <= 1e-2 * (rms_row(ref) + |ref|)      (elementwise)
           |gpu - ref| <= 1e-2 * (rms_all(ref) + |ref|)      (elementwise)
           and ||gpu - ref||_2 / ||ref||_2 <= 2^-7
The official bound alone has an absolute floor of 1e-2, far above the
typical magnitude of these outputs (an all-zero answer would pass), so
every parity test applies both.  The strict bound is the official one with
the output rescaled to unit RMS, taken both ways and both required: each
row (a token's output, a routed pair's h or y) rescaled on its own, and the
whole tensor rescaled at once.  A 1-D array is one row.
"""
from __future__ import annotations

import numpy as np

NRMSE_MAX = 2.0 ** -7


def _f64(a) -> np.ndarray:
    try:
        import torch

        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def errors(gpu, ref) -> dict:
    g, r = _f64(gpu), _f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    rows = r.reshape(-1, r.shape[-1]) if r.ndim >= 1 and r.size else r.reshape(1, -1)
    rms_row = np.sqrt(np.mean(rows * rows, axis=1, keepdims=True)) if rows.size else rows
    er = err.reshape(rows.shape)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "official_ratio": float((err / (1.0 + np.abs(r))).max()) / 1e-2 if err.size else 0.0,
        "strict_ratio": max(float((er / (rms_row + np.abs(rows) + 1e-300)).max()),
                            float((err / (rms + np.abs(r) + 1e-300)).max())) / 1e-2 if err.size else 0.0,
        "nrmse": float(np.sqrt(np.mean(err * err)) / rms) if rms > 0 else float(err.max() if err.size else 0.0),
        "rms_ref": rms,
        "finite": bool(np.isfinite(g).all()),
    }


def passes(gpu, ref) -> bool:
    e = errors(gpu, ref)
    return e["finite"] and e["official_ratio"] <= 1.0 and e["strict_ratio"] <= 1.0 and e["nrmse"] <= NRMSE_MAX


def assert_parity(gpu, ref, name: str = "") -> dict:
    e = errors(gpu, ref)
    ok = e["finite"] and e["official_ratio"] <= 1.0 and e["strict_ratio"] <= 1.0 and e["nrmse"] <= NRMSE_MAX
    assert ok, f"{name}: parity failed {e}"
    return e


def assert_parity_relative(gpu, ref, name: str = "") -> dict:
    """The scale-invariant half of the rules (strict bound and NRMSE).  For
    inputs far from unit magnitude, where the official bound's absolute floor
    of 1e-2 no longer scales with the data."""
    e = errors(gpu, ref)
    ok = e["finite"] and e["strict_ratio"] <= 1.0 and e["nrmse"] <= NRMSE_MAX
    assert ok, f"{name}: parity failed {e}"
    return e
