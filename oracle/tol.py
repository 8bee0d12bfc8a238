"""Tolerances the GPU results are held to (test infrastructure).

Floating outputs: |gpu - oracle| <= 1e-3 * B + 1e-6 per element, where B = sum_k |a_k w_k|
over the dequantised operands of that output. Where the GPU writes bf16, half a bf16
ulp of the value is added: that is the output format's own rounding, which the 1e-3 * B
term does not cover when |y| comes close to B.
"""

from __future__ import annotations

import numpy as np

REL = 1e-3
ABS = 1e-6


def gemm_bound(bound: np.ndarray) -> np.ndarray:
    return REL * np.asarray(bound, np.float64) + ABS


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (normal range): 2^(floor(log2|x|) - 8)."""
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(np.where(x == 0, 1.0, x))
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 1 - 8))


def check_close(gpu, ref, tol, what=""):
    """Assert |gpu - ref| <= tol elementwise; report the worst violation."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)),
                             err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
            f"gpu={gpu[i]!r} ref={ref[i]!r} err={err[i]:.3e} tol={np.broadcast_to(tol, err.shape)[i]:.3e}")
