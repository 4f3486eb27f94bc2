"""Scalar numerics of the oracle: rounding, float16 conversion, bit fields.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

* Round-to-nearest with ties to the even integer is the tie rule of deterministic
  write-back: [WB-zh], section "Reproduction assessment" (复现评估), states that
  half-step ties go to the nearest even index.
* float16 is the storage type of the protected rows and of every scale and zero
  point ([DAMP] "Key Points", [LBRS] "Levels and storage"). ``f16`` rounds a
  float64 value to the nearest float16 (ties to even) in one rounding; it is pinned
  against exact rational arithmetic in ``tests/test_oracle_numerics.py``.
"""
from __future__ import annotations

import numpy as np


def rne(x):
    """Round to nearest integer, ties to even (numpy's rint), float64 in and out."""
    return np.rint(np.asarray(x, dtype=np.float64))


def f16(x):
    """Nearest float16 value of float64 ``x`` (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def f16_bits(x) -> np.ndarray:
    """Bit pattern (uint16) of the nearest float16 to float64 ``x``."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_value(bits) -> np.ndarray:
    """float64 value of float16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f16_ulp(x) -> np.ndarray:
    """Spacing of float16 values at |x| (distance to the next float16 away from 0)."""
    h = np.abs(np.asarray(x, dtype=np.float64)).astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf))
    return up.astype(np.float64) - h.astype(np.float64)


def pack_fields(values: np.ndarray, width: int) -> np.ndarray:
    """Pack unsigned integers of ``width`` bits, value n at bits [n*width, (n+1)*width),
    least-significant bit first, into bytes (little-endian bit order)."""
    v = np.asarray(values, dtype=np.int64).reshape(-1)
    assert width >= 1 and np.all(v >= 0) and np.all(v < (1 << width))
    bits = ((v[:, None] >> np.arange(width)[None, :]) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bits, bitorder="little")


def unpack_fields(data: np.ndarray, width: int, count: int) -> np.ndarray:
    """Inverse of ``pack_fields``: ``count`` unsigned fields of ``width`` bits."""
    bits = np.unpackbits(np.asarray(data, dtype=np.uint8), bitorder="little")
    bits = bits[: count * width].reshape(count, width).astype(np.int64)
    return np.sum(bits << np.arange(width)[None, :], axis=1)
