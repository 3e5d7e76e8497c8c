"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (written here, used by every parity test):

* fp32 outputs: |gpu - ref| <= 1e-5 * (|ref| + rms(ref over the read)), the
  "1e-5 relative" bar measured so that near-zero outputs of a read do not blow
  the relative error up.
* bf16 outputs: |gpu - ref| <= 2e-2 + ulp_bf16(ref) / 2.  The GPU computes in
  fp32 and rounds once to bf16; the rounding alone costs up to half an ulp,
  which exceeds 2e-2 once |ref| >= 8 (ulp 2^-4), so the absolute 2e-2 bar is
  applied to the arithmetic and the half-ulp of the final rounding is added.
* fp32 log-sum-exp: |gpu - ref| <= 1e-5 * (1 + |ref|).

``ref`` is the fp64 oracle value before any rounding.
"""
from __future__ import annotations

import numpy as np


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_out(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "out") -> dict:
    """Assert gpu ~ ref under the dtype's bar.  gpu/ref: [n_q, T, d] float64.
    Returns statistics (max error, fraction exactly equal to RNE(ref) for bf16)."""
    import oracle
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    stats = {"max_abs_err": float(err.max()) if err.size else 0.0}
    if dtype == "f32":
        rms = np.sqrt((ref ** 2).reshape(ref.shape[0], -1).mean(axis=1))[:, None, None]
        tol = 1e-5 * (np.abs(ref) + rms)
    else:
        tol = 2e-2 + 0.5 * oracle.ulp_bf16(ref)
        stats["frac_equal_rne"] = float((gpu == oracle.round_to_bf16(ref)).mean()) if ref.size else 1.0
    bad = err > tol
    if bad.any():
        idx = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{what} ({dtype}): {int(bad.sum())} of {bad.size} outside tolerance; worst at {idx}: "
            f"gpu={gpu[idx]!r} ref={ref[idx]!r} tol={tol[idx]!r}")
    return stats


def check_lse(gpu: np.ndarray, ref: np.ndarray, what: str = "lse"):
    assert gpu.shape == ref.shape
    err = np.abs(gpu - ref)
    tol = 1e-5 * (1.0 + np.abs(ref))
    bad = err > tol
    if bad.any():
        idx = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} outside tolerance; worst at {idx}: "
                             f"gpu={gpu[idx]!r} ref={ref[idx]!r}")


def check_rel(gpu: np.ndarray, ref: np.ndarray, rel: float, what: str):
    """|gpu - ref| <= rel * (|ref| + rms(ref)) element-wise (fp32 results such
    as dw and fp32 dhist)."""
    err = np.abs(gpu - ref)
    rms = np.sqrt((ref ** 2).mean()) if ref.size else 0.0
    tol = rel * (np.abs(ref) + rms)
    bad = err > tol
    if bad.any():
        idx = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside {rel} relative; "
                             f"worst at {idx}: gpu={gpu[idx]!r} ref={ref[idx]!r}")
