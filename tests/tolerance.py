"""Parity bar shared by every comparison with the oracle.

Output: |got - ref| <= 1e-2 + 1e-2 * |ref| elementwise (bf16/fp16 inputs).
LSE:    |got - ref| <= 1e-2 log2 units; -inf must match -inf exactly; any NaN or
        +inf in the result fails.
"""
from __future__ import annotations

import numpy as np

OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-2


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def out_errors(got, ref):
    """Return (max excess over the bound, max abs error); excess <= 0 means pass."""
    got, ref = _np(got), _np(ref)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} != {ref.shape}")
    if not np.all(np.isfinite(got)):
        return np.inf, np.inf
    err = np.abs(got - ref)
    excess = err - (OUT_ATOL + OUT_RTOL * np.abs(ref))
    return (float(excess.max()) if err.size else -1.0), (float(err.max()) if err.size else 0.0)


def lse_errors(got, ref):
    """Return the max LSE error in log2 units (inf on any NaN or -inf mismatch)."""
    got, ref = _np(got), _np(ref)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} != {ref.shape}")
    if np.isnan(got).any() or np.isposinf(got).any():
        return np.inf
    ninf_ref, ninf_got = np.isneginf(ref), np.isneginf(got)
    if (ninf_ref != ninf_got).any():
        return np.inf
    fin = ~ninf_ref
    return float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0


def assert_out_close(got, ref, what="out"):
    excess, err = out_errors(got, ref)
    assert excess <= 0.0, f"{what}: max abs error {err:.4g} exceeds 1e-2 + 1e-2*|ref|"


def assert_lse_close(got, ref, what="lse"):
    err = lse_errors(got, ref)
    assert err <= LSE_ATOL, f"{what}: max LSE error {err:.4g} log2 units > {LSE_ATOL}"
