"""Pins of the oracle's scalar numerics: float16 rounding, ties, bit packing, Philox."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle.numerics import f16, f16_bits, pack_fields, rne, unpack_fields
from oracle.philox import philox4x32_10, sr_draws

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _exact_nearest_f16(x: float) -> float:
    """Nearest float16 by exact rational comparison of the two bracketing float16
    values (found with nextafter only); ties go to the even significand."""
    fx = Fraction(x)
    h = np.float16(x) if abs(x) < 65520 else np.float16(np.copysign(65504.0, x))
    cands = {float(h), float(np.nextafter(h, np.float16(np.inf))),
             float(np.nextafter(h, np.float16(-np.inf)))}
    cands = [c for c in cands if np.isfinite(c)]
    best = None
    for c in sorted(cands):
        d = abs(Fraction(c) - fx)
        if best is None or d < best[0]:
            best = (d, c)
        elif d == best[0]:
            even_c = int(np.float16(c).view(np.uint16)) & 1 == 0
            if even_c:
                best = (d, c)
    return best[1]


def test_f16_is_correctly_rounded():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 4, 3000))
    # exact midpoints between adjacent float16 values, and values just off them
    h = rng.standard_normal(500).astype(np.float16)
    nx = np.nextafter(h, np.float16(np.inf))
    mids = (h.astype(np.float64) + nx.astype(np.float64)) / 2
    xs += list(mids) + list(np.nextafter(mids, np.inf)) + list(np.nextafter(mids, -np.inf))
    xs += [0.0, 5.960464477539063e-08 / 2, 6.1e-5, 65504.0, 65519.99]
    for x in xs:
        assert float(f16(x)) == _exact_nearest_f16(float(x)), x


def test_f16_double_rounding_hazard():
    # a float64 value just above a float16 midpoint whose float32 rounding lands on
    # the midpoint: a float64 -> float32 -> float16 chain would round down (to even)
    lo = np.float16(1.0)
    hi = np.nextafter(lo, np.float16(2.0))
    mid = (float(lo) + float(hi)) / 2
    x = mid + 2.0 ** -40
    assert np.float32(x) == np.float32(mid)
    assert float(f16(x)) == float(hi)


def test_rne_ties_to_even():
    assert list(rne([0.5, 1.5, 2.5, -0.5, -1.5, 2.4999, 2.5001])) == [0, 2, 2, -0, -2, 2, 3]


def test_pack_fields_lsb_first():
    # 2-bit fields 1, 2, 3, 0 -> bits (lsb first) 10 01 11 00 -> 0b00111001
    assert list(pack_fields([1, 2, 3, 0], 2)) == [0x39]
    # 4-bit two fields: low nibble first
    assert list(pack_fields([0xA, 0x5], 4)) == [0x5A]
    rng = np.random.default_rng(2)
    for w in range(1, 9):
        v = rng.integers(0, 2 ** w, 128)
        assert np.array_equal(unpack_fields(pack_fields(v, w), w, 128), v)


def test_f16_bits_roundtrip():
    x = np.array([0.0, -0.0, 1.0, -2.5, 65504.0])
    assert list(f16_bits(x)) == [0x0000, 0x8000, 0x3C00, 0xC100, 0x7BFF]


def test_philox_known_answers():
    with open(os.path.join(GOLD, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        out = philox4x32_10(ctr, key)
        assert ["%08x" % w for w in out] == vec["out"]


def test_sr_draw_mapping():
    seed, H = 0x1234_5678_9ABC_DEF0, 4
    r = sr_draws(seed, 1, 2, H, 7, 3, 16)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    w0 = philox4x32_10((16 * 3 + 0, 1 * H + 2, 7, 0), key)
    w1 = philox4x32_10((16 * 3 + 1, 1 * H + 2, 7, 0), key)
    assert r[0] == w0[0] & 0xFFFF and r[1] == w0[0] >> 16
    assert r[6] == w0[3] & 0xFFFF and r[7] == w0[3] >> 16
    assert r[8] == w1[0] & 0xFFFF and r[15] == w1[3] >> 16
