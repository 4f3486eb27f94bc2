"""Walsh-Hadamard transform along the value axis of a key row.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

[DAMP] "Key Points" and "Quantization & calibration details": before INT8 storage
each key channel (row) is rotated by a Hadamard transform along the value dimension
to flatten its within-row range. The pages give no normalisation, ordering or random
signs; this oracle reads the plainest form: the Sylvester matrix in natural order,
scaled by 1/sqrt(n), so that H is symmetric and orthonormal (H = H^T = H^-1).

Two independent forms are provided and tested against each other: the explicit
matrix (Kronecker powers of [[1, 1], [1, -1]]) and the in-place butterfly.
"""
from __future__ import annotations

import numpy as np


def sylvester(n: int) -> np.ndarray:
    """Orthonormal Sylvester-Hadamard matrix of order n (a power of two)."""
    assert n >= 1 and n & (n - 1) == 0
    h = np.array([[1.0]])
    base = np.array([[1.0, 1.0], [1.0, -1.0]])
    while h.shape[0] < n:
        h = np.kron(h, base)
    return h / np.sqrt(n)


def fwht(x: np.ndarray) -> np.ndarray:
    """Butterfly form of the same transform, applied along the last axis."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    assert n & (n - 1) == 0
    span = 1
    while span < n:
        for start in range(0, n, 2 * span):
            a = y[..., start:start + span].copy()
            b = y[..., start + span:start + 2 * span].copy()
            y[..., start:start + span] = a + b
            y[..., start + span:start + 2 * span] = a - b
        span *= 2
    return y / np.sqrt(n)


def rotate_rows(X: np.ndarray) -> np.ndarray:
    """Row transform y_i = H x_i for every row x_i of X (last axis = value axis)."""
    H = sylvester(X.shape[-1])
    return X @ H.T
