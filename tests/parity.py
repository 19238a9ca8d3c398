"""Shared comparison rules for the parity tests.

Parity bar for floating-point outputs of the W4A16 matmul: every output must satisfy
    |y_gpu - y_oracle| <= 4e-3 * sum_k |a_k * w_kn| + 1e-6
where y_oracle is the oracle's fp64 result and the sum is its fp64 |a*w| bound. 4e-3 is about
twice the bf16 unit roundoff, so the same bar covers bf16 outputs.
"""
import numpy as np

REL = 4e-3
ABS = 1e-6


def tolerance(bound: np.ndarray) -> np.ndarray:
    return REL * bound + ABS


def check_close(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str = "") -> float:
    """Assert the parity bar; return the largest used fraction of the allowed error."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite outputs"
    err = np.abs(y_gpu - y_ref)
    tol = tolerance(bound)
    frac = err / tol
    worst = np.unravel_index(int(np.argmax(frac)), frac.shape)
    assert np.all(err <= tol), (
        f"{what}: {int(np.sum(err > tol))} outputs outside the bar; worst at {worst}: "
        f"gpu={y_gpu[worst]!r} ref={y_ref[worst]!r} err={err[worst]:.3e} tol={tol[worst]:.3e}")
    return float(frac.max())
