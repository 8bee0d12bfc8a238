"""Small numeric helpers of the oracle (test infrastructure): bf16 rounding, cosine."""

from __future__ import annotations

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value, ties to even, returned as float64.

    bf16 keeps 8 significant bits; for |x| in [2^e, 2^(e+1)) the spacing is 2^(e-7).
    Works from the float64 value directly (one rounding). Finite, normal-range inputs.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    step = np.ldexp(1.0, e - 1 - 7)
    r = np.rint(x / step) * step
    return np.where(x == 0, x, r)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 value that is exactly a bf16 -> its uint16 bit pattern."""
    f = np.asarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64).reshape(-1)
    b = np.asarray(b, np.float64).reshape(-1)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
