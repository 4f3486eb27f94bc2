"""The integer form of stochastic rounding that the decode kernels evaluate.

[WB] "Error feedback and stochastic rounding" defines stochastic rounding as rounding up
with probability equal to the fractional part; with a 16-bit integer draw u the rule is
floor(t) + [u < frac(t) 2^16]. The tuned kernels take it as one floor conversion:
floor((ceil(t 2^16) + 2^16 - 1 - u) / 2^16), the ceiling formed as minus the floor of
-t 2^16 (float32 in the decay-aware kernels, float64 in the rotated-domain kernel), and
an arithmetic shift. These CPU checks hold that rewrite to the rule, value by value, over
random and constructed t (negative levels, exact integers, fractions on and beside
multiples of 2^-16, the largest magnitudes each kernel admits) and every draw edge.
"""
import numpy as np
import pytest


def rule(t, u):
    """floor(t) + [u < frac(t) 2^16], decided exactly: u < frac(t) 2^16 is
    floor(t) + u 2^-16 < t, and floor(t) + u 2^-16 (at most 31 significant bits here) is
    exact in float64, where t - floor(t) need not be (t in (-1/2, 0))."""
    t = np.asarray(t, np.float64)
    fl = np.floor(t)
    return (fl + (fl + u.astype(np.float64) / 65536.0 < t)).astype(np.int64)


def integer_form(t, u, dtype):
    """The kernels' evaluation: the floor of -(t 2^16) in the working precision, then
    (2^16 - 1 - z - u) >> 16 in 32-bit integers."""
    m = -(np.asarray(t, dtype) * dtype(65536.0))        # exact: a power-of-two scaling
    z = np.floor(m).astype(np.int64)
    assert np.all(np.abs(z) < 2**31)
    v = (65535 - z - u.astype(np.int64)).astype(np.int32)
    return (v >> 16).astype(np.int64)


def _cases(rng, dtype, tmax):
    n = 200_000
    t = rng.uniform(-tmax, tmax, n)
    # exact integers, exact multiples of 2^-16, and their float neighbours
    k = rng.integers(-int(tmax), int(tmax), n // 4).astype(np.float64)
    q = np.round(rng.uniform(-tmax, tmax, n // 4) * 65536.0) / 65536.0
    base = np.concatenate([k, q]).astype(dtype)
    nb = np.concatenate([base, np.nextafter(base, dtype(np.inf)), np.nextafter(base, dtype(-np.inf))])
    t = np.concatenate([t.astype(dtype), nb, np.array([0.0, -0.0, tmax * 0.999, -tmax * 0.999], dtype)])
    u = rng.integers(0, 65536, t.size).astype(np.uint32)
    # draws on the edges: 0, 65535 and the fraction's own 16-bit value
    fr = np.floor((t.astype(np.float64) - np.floor(t.astype(np.float64))) * 65536.0).astype(np.int64)
    pick = rng.integers(0, 4, t.size)
    u = np.where(pick == 0, 0, np.where(pick == 1, 65535, np.where(pick == 2, np.clip(fr, 0, 65535), u)))
    return t, u.astype(np.uint32)


@pytest.mark.parametrize("dtype,tmax", [(np.float32, 512.0), (np.float64, 16384.0)])
def test_integer_form_equals_rule(dtype, tmax):
    rng = np.random.default_rng(1234)
    t, u = _cases(rng, dtype, tmax)
    got = integer_form(t, u, dtype)
    want = rule(t.astype(np.float64), u)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (t[bad[:5]], u[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_integer_form_hand_values():
    # t = 2.25: rounds up for u < 16384 only; t = -0.5: level 0 for u < 32768, else -1;
    # an exact integer never rounds up; a zero step (t = 0) stays at 0
    t = np.array([2.25, 2.25, -0.5, -0.5, 3.0, 3.0, 0.0], np.float32)
    u = np.array([16383, 16384, 32767, 32768, 0, 65535, 0], np.uint32)
    assert integer_form(t, u, np.float32).tolist() == [3, 2, 0, -1, 3, 3, 0]
    assert rule(t, u).tolist() == [3, 2, 0, -1, 3, 3, 0]
