"""Pins of the INT4 low tier ([DAMP] "Quantization & calibration details": per-block
asymmetric affine quantization with b = 8 for INT8 and b = 4 for INT4)."""
import numpy as np
import pytest

from oracle import layouts as L
from oracle.numerics import f16_bits
from oracle.quantizers import affine_metadata
from oracle.step import decode_step, import_state
from synth import decode_inputs


def test_int4_accounting():
    # 16 float16 rows + 112 four-bit rows + a (scale, zero) pair per 32 values
    lay = L.Layout(kind=L.MIXED, B=1, H=1, dk=128, dv=128, block=32, k_hi=16, int_bits=4)
    assert L.bits_per_value_stored(lay) == (16 * 16 + 112 * (4 + 32 / 32)) / 128 == 6.375
    lay8 = L.Layout(kind=L.MIXED, B=1, H=1, dk=128, dv=128, block=32, k_hi=16)
    assert L.bits_per_value_stored(lay8) == 9.875


@pytest.mark.parametrize("kind", [L.HAD_INT8, L.MIXED])
def test_int4_region_round_trip(kind):
    rng = np.random.default_rng(30)
    lay = L.Layout(kind=kind, B=1, H=1, dk=32, dv=128, block=32, k_hi=4, int_bits=4)
    nq, nb = lay.int8_rows, 128 // 32
    c = L.Content(codes=rng.integers(0, 16, (nq, 128)), scale_bits=f16_bits(rng.random((nq, nb))),
                  zero_bits=f16_bits(rng.standard_normal((nq, nb))),
                  hi_bits=f16_bits(rng.standard_normal((4, 128))) if kind == L.MIXED else None)
    reg = L.encode_region(lay, c)
    assert reg.size == lay.region_size()
    back = L.decode_region(lay, reg)
    assert np.array_equal(back.codes, c.codes) and np.array_equal(L.encode_region(lay, back), reg)


def test_int4_metadata_is_the_range_over_fifteen():
    x = np.linspace(-1.5, 3.0, 32)
    s, z, spre, zpre = affine_metadata(x, 4)
    assert spre == 4.5 / 15 and zpre == -1.5 and s == float(np.float16(0.3)) and z == -1.5


@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_int4_step_codes_and_rounding(mode):
    rng = np.random.default_rng(31)
    dk = dv = 128
    lay = L.Layout(kind=L.HAD_INT8, B=1, H=1, dk=dk, dv=dv, block=32, int_bits=4, mode=mode)
    reg = import_state(lay, rng.standard_normal((dk, dv)) * 0.3, L.initial_region(lay))
    inp = decode_inputs(5, 1, 1, dk, dv, 1)
    e = rng.uniform(-0.01, 0.01, (dk, dv)) if mode == "ef" else None
    r = decode_step(lay, reg, e, inp["q"][0, 0, 0], inp["k"][0, 0, 0], inp["v"][0, 0, 0], inp["beta"][0, 0, 0],
                    inp["s"][0, 0], 3, 0, 0)
    c = L.decode_region(lay, r.wb.region)
    assert c.codes.min() >= 0 and c.codes.max() == 15
    step = np.repeat(c.scale, 32, axis=1)
    zerr = np.abs(np.repeat(c.zero, 32, axis=1) - np.repeat(r.wb.meta_pre["zero"], 32, axis=1))
    err = np.abs(L.stored_values(lay, c) - r.wb.X)
    bound = step * (1.0 if mode == "sr" else 0.5) + (step if mode == "ef" else 0) + 2 * zerr + 16 * step * 2 ** -10
    assert np.all(err <= bound)
