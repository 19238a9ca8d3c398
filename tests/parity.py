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


# Gated feed-forward input h = silu(g) * u. With g and u each within the bar above (dg, du),
# and |silu'| <= 1.1 everywhere (pinned in the oracle tests):
#   |h_gpu - h| <= 1.1 dg (|u| + du) + (|silu(g)| + 1.1 dg) du
# plus the fp32 evaluation of silu and the product, a few units of 2^-24 relative, allowed
# here as 1e-6 of the magnitude.
SILU_SLOPE = 1.1
EVAL_REL = 1e-6


def gate_up_tolerance(y_gate, bound_gate, y_up, bound_up):
    import oracle
    dg = tolerance(bound_gate)
    du = tolerance(bound_up)
    sg = np.abs(oracle.silu_mul(y_gate, np.ones_like(y_gate)))   # |silu(g)|
    mag = (sg + SILU_SLOPE * dg) * (np.abs(y_up) + du)
    return SILU_SLOPE * dg * (np.abs(y_up) + du) + (sg + SILU_SLOPE * dg) * du + EVAL_REL * mag + ABS


def check_gate_up(h_gpu, h_ref, y_gate, bound_gate, y_up, bound_up, what: str = "") -> float:
    """Assert the gated-product bar; return the largest used fraction of the allowed error."""
    h_gpu = np.asarray(h_gpu, dtype=np.float64)
    assert h_gpu.shape == h_ref.shape, (h_gpu.shape, h_ref.shape)
    assert np.all(np.isfinite(h_gpu)), f"{what}: non-finite outputs"
    err = np.abs(h_gpu - h_ref)
    tol = gate_up_tolerance(y_gate, bound_gate, y_up, bound_up)
    frac = err / tol
    worst = np.unravel_index(int(np.argmax(frac)), frac.shape)
    assert np.all(err <= tol), (
        f"{what}: {int(np.sum(err > tol))} outputs outside the bar; worst at {worst}: "
        f"gpu={h_gpu[worst]!r} ref={h_ref[worst]!r} err={err[worst]:.3e} tol={tol[worst]:.3e}")
    return float(frac.max())
