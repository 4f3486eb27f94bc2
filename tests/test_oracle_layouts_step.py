"""Pins of the storage layouts, the teacher-forced step, prefill cadence and DAMP."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import layouts as L
from oracle.damp import calibration_samples, risk_scores, row_error_energy, select_permutation
from oracle.hadamard import sylvester
from oracle.numerics import f16_bits
from oracle.recurrence import delta_step, unrolled
from oracle.step import allocate_region, decode_step, export_state, import_state, prefill
from synth import decode_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def lay(kind, mode="rtn", dk=128, dv=128, **kw):
    base = dict(kind=kind, B=1, H=1, dk=dk, dv=dv, mode=mode)
    if kind == L.HAD_INT8:
        base["block"] = 128 if dv >= 128 else dv
    base.update(kw)
    return L.Layout(**base)


def test_layout_accounting():
    with open(os.path.join(GOLD, "layout_accounting.json")) as f:
        g = json.load(f)
    mixed = lay(L.MIXED)
    assert mixed.region_size() == 20224
    assert Fraction(mixed.region_size() * 8, 128 * 128) == Fraction(g["mixed_bits_per_element"])
    assert round(100 * (1 - g["mixed_bits_per_element"] / 32), 1) == g["storage_reduction_percent"]
    # the page's count: 4-bit mean codes + f16 scale + width field per row of dv values
    dv = 128
    assert round(4 + Fraction(g["row_meta_bits_4bit_width"], dv), 3) == Fraction(4156, 1000)
    assert Fraction(16 + 3, dv) == Fraction(g["row_meta_bits_3bit_width"], dv)
    bal = lay(L.BITALLOC)
    assert bal.region_size() == 8192 + 256 + 128
    assert lay(L.HAD_INT8).region_size() == 16896
    assert lay(L.UNIFORM, dk=16, dv=16).region_size() == 128
    for k in L.KINDS:
        assert lay(k).region_stride() % 256 == 0


@pytest.mark.parametrize("kind", L.KINDS)
def test_encode_decode_roundtrip(kind):
    rng = np.random.default_rng(20)
    la = lay(kind, dk=32, dv=128, k_hi=4)
    dk, dv = la.dk, la.dv
    if kind == L.FP32:
        c = L.Content(S32=rng.standard_normal((dk, dv)).astype(np.float32).astype(np.float64))
    elif kind == L.UNIFORM:
        c = L.Content(kappa=rng.integers(-8, 8, (dk, dv)))
    elif kind in (L.HAD_INT8, L.MIXED):
        nq = la.int8_rows
        nb = dv // la.block
        c = L.Content(codes=rng.integers(0, 256, (nq, dv)),
                      scale_bits=f16_bits(rng.random((nq, nb))),
                      zero_bits=f16_bits(rng.standard_normal((nq, nb))),
                      hi_bits=f16_bits(rng.standard_normal((la.k_hi, dv))) if kind == L.MIXED else None)
    elif kind == L.HEADALLOC:
        b = 5
        ng = dk // L.HA_GROUP
        c = L.Content(kappa=rng.integers(-(2 ** (b - 1) - 1), 2 ** (b - 1), (dk, dv)), width=b,
                      fit=rng.integers(0, 16, (ng, dv)), delta_bits=f16_bits(rng.random((ng, dv))))
    else:
        w = np.full(dk, 4)
        w[:8] = [2, 8, 3, 5, 6, 2, 3, 3]        # sums to 32: same as eight rows of 4
        assert w.sum() == 4 * dk
        kap = np.stack([rng.integers(-(2 ** (b - 1) - 1), 2 ** (b - 1), dv) for b in w])
        c = L.Content(kappa=kap, widths=w, fit=rng.integers(0, 16, dk),
                      delta_bits=f16_bits(rng.random(dk)))
    reg = L.encode_region(la, c)
    assert reg.size == la.region_size()
    d = L.decode_region(la, reg)
    assert np.array_equal(L.encode_region(la, d), reg)


def test_storage_transforms_are_inverse():
    rng = np.random.default_rng(21)
    perm = rng.permutation(128)
    for kind in (L.HAD_INT8, L.MIXED):
        la = lay(kind)
        S = rng.standard_normal((128, 128))
        assert np.allclose(L.to_logical(la, L.to_stored(la, S, perm), perm), S, atol=1e-12)


def test_identity_write_back_equals_unrolled_recurrence():
    la = lay(L.FP32, dk=8, dv=8)
    inp = decode_inputs(1, 1, 1, 8, 8, 6)
    reg = L.initial_region(la)
    S = np.zeros((8, 8))
    for t in range(6):
        r = decode_step(la, reg, None, inp["q"][t, 0, 0], inp["k"][t, 0, 0], inp["v"][t, 0, 0],
                        inp["beta"][t, 0, 0], inp["s"][0, 0], t, 0, 0)
        reg = r.wb.region
    ref = unrolled(np.zeros((8, 8)), [inp["k"][t, 0, 0] for t in range(6)],
                   [inp["v"][t, 0, 0] for t in range(6)],
                   [inp["beta"][t, 0, 0] for t in range(6)], [inp["s"][0, 0]] * 6)
    got = export_state(la, reg)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6)


def _run_uniform(mode, T=256):
    la = lay(L.UNIFORM, mode=mode, dk=16, dv=16, bits=4)
    inp = decode_inputs(0, 1, 1, 16, 16, T)
    reg = L.initial_region(la)
    e = np.zeros((16, 16)) if mode == "ef" else None
    hist = []
    for t in range(T):
        r = decode_step(la, reg, e, inp["q"][t, 0, 0], inp["k"][t, 0, 0], inp["v"][t, 0, 0],
                        inp["beta"][t, 0, 0], inp["s"][0, 0], t, 0, 0)
        hist.append((reg, r))
        reg, e = r.wb.region, r.wb.e_new
    return la, hist


def test_tiny_uniform_dead_zone_invariant():
    """Every element whose margin M = 2|h_t - q_{t-1}| / Delta is below 1, on an
    interior level, keeps its stored level (RTN, the tiny 16 x 16 configuration)."""
    la, hist = _run_uniform("rtn")
    d = 0.125
    n_dead = 0
    for reg, r in hist:
        prev = L.decode_region(la, reg).kappa
        new = L.decode_region(la, r.wb.region).kappa
        M = 2 * np.abs(r.S_new - prev * d) / d
        interior = (prev > -8) & (prev < 7)
        sel = (M < 1) & interior
        n_dead += sel.sum()
        assert np.array_equal(new[sel], prev[sel])
    assert n_dead > 1000


def test_tiny_uniform_error_feedback_bounds():
    la, hist = _run_uniform("ef")
    for _, r in hist:
        assert np.all(np.abs(r.wb.e_new) <= 0.125)


@pytest.mark.parametrize("kind", L.KINDS)
@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_step_rounds_within_half_a_step(kind, mode):
    dk, dv = 32, 128
    la = lay(kind, mode=mode, dk=dk, dv=dv, k_hi=4, H=2, seed=99)
    rng = np.random.default_rng(22)
    perm = rng.permutation(dk)
    inp = decode_inputs(3, 1, 2, dk, dv, 1)
    S0 = rng.standard_normal((dk, dv)) * 0.3
    reg = import_state(la, S0, L.initial_region(la), perm)
    e = rng.uniform(-0.001, 0.001, (dk, dv)) if mode == "ef" else None
    r = decode_step(la, reg, e, inp["q"][0, 0, 1], inp["k"][0, 0, 1], inp["v"][0, 0, 1],
                    inp["beta"][0, 0, 1], inp["s"][0, 1], 5, 0, 1, perm)
    Xhat = L.stored_values(la, L.decode_region(la, r.wb.region))
    err = np.abs(Xhat - r.wb.X)
    if kind == L.FP32:
        assert np.all(err <= np.abs(r.wb.X) * 2 ** -24)
        return
    rot = L.rotated_rows(la)
    if kind == L.UNIFORM:
        step = np.full((dk, dv), 0.125)
    elif kind in (L.HAD_INT8, L.MIXED):
        c = L.decode_region(la, r.wb.region)
        q0 = dk - la.int8_rows
        step = np.zeros((dk, dv))
        step[q0:] = np.repeat(c.scale, la.block, axis=1)
        zero_err = np.abs(np.repeat(c.zero, la.block, axis=1) - np.repeat(r.wb.meta_pre["zero"], la.block, axis=1))
        step[q0:] += 2 * zero_err
        if kind == L.MIXED:
            step[:q0] = np.abs(r.wb.X[:q0]) * 2 ** -10 + 2 ** -24
    elif kind == L.HEADALLOC:
        c = L.decode_region(la, r.wb.region)
        step = np.repeat(c.delta, L.HA_GROUP, axis=0)
    else:
        c = L.decode_region(la, r.wb.region)
        step = np.repeat(c.delta[:, None], dv, axis=1)
    unclipped = np.isfinite(r.wb.boundary) & (np.abs(r.wb.tau) < 2 ** 30)
    if kind == L.UNIFORM:
        unclipped &= (r.wb.X > -1) & (r.wb.X < 0.875)
    if kind == L.BITALLOC:
        n = (2 ** (c.widths - 1) - 1)[:, None]
        unclipped &= np.abs(r.wb.X) <= n * step
    if kind == L.HEADALLOC:
        unclipped &= np.abs(r.wb.X) <= (2 ** (c.width - 1) - 1) * step
    bound = step * (1.0 if mode == "sr" else 0.5) + (step if mode == "ef" else 0)
    assert np.all(err[unclipped] <= bound[unclipped] * (1 + 1e-9) + 1e-12)
    assert rot.sum() == (0 if kind in (L.FP32, L.UNIFORM, L.BITALLOC, L.HEADALLOC) else la.int8_rows)


def test_prefill_with_cadence_one_equals_decode_steps():
    la = lay(L.MIXED, mode="rtn", dk=32, dv=128, k_hi=4)
    perm = np.random.default_rng(23).permutation(32)
    inp = decode_inputs(4, 1, 1, 32, 128, 5)
    reg0 = L.initial_region(la)
    sl = lambda a: a[:, 0, 0]
    reg_p, _, outs = prefill(la, reg0, None, sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                             sl(inp["beta"]), [inp["s"][0, 0]] * 5, 0, 1, 0, 0, perm)
    reg = reg0
    for t in range(5):
        r = decode_step(la, reg, None, inp["q"][t, 0, 0], inp["k"][t, 0, 0], inp["v"][t, 0, 0],
                        inp["beta"][t, 0, 0], inp["s"][0, 0], t, 0, 0, perm)
        assert np.allclose(r.o, outs[t], rtol=0, atol=0)
        reg = r.wb.region
    assert np.array_equal(reg, reg_p)


def test_prefill_deferred_write_back_keeps_unquantized_state_between():
    la = lay(L.UNIFORM, dk=16, dv=16)
    inp = decode_inputs(5, 1, 1, 16, 16, 8)
    sl = lambda a: a[:, 0, 0]
    _, _, outs = prefill(la, L.initial_region(la), None, sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                         sl(inp["beta"]), [inp["s"][0, 0]] * 8, 0, 8, 0, 0)
    S = np.zeros((16, 16))
    for t in range(8):
        S, o = delta_step(S, inp["q"][t, 0, 0], inp["k"][t, 0, 0], inp["v"][t, 0, 0],
                          inp["beta"][t, 0, 0], inp["s"][0, 0])
        assert np.allclose(o, outs[t], atol=0)


def test_allocation_pass_keeps_region_and_budget():
    la = lay(L.BITALLOC)
    rng = np.random.default_rng(24)
    S = rng.standard_normal((128, 128)) * np.exp(rng.uniform(-3, 1, 128))[:, None]
    reg = import_state(la, S, L.initial_region(la))
    s = np.exp(rng.uniform(np.log(1e-3), 0, 128))
    reg2, alloc = allocate_region(la, reg, s, np.full(128, 1 / 384))
    c = L.decode_region(la, reg2)
    assert reg2.size == reg.size and c.widths.sum() == 512
    assert np.array_equal(c.widths, alloc["widths"]) and np.array_equal(c.fit, alloc["fit"])
    # stored values are re-rounded from the previous stored values at the new widths
    Y = L.stored_values(la, L.decode_region(la, reg))
    Y2 = L.stored_values(la, c)
    n = (2 ** (c.widths - 1) - 1)[:, None]
    inside = np.abs(Y) <= n * c.delta[:, None]
    assert np.all(np.abs(Y2 - Y)[inside] <= (c.delta[:, None] / 2 * np.ones_like(Y))[inside] * (1 + 1e-12))


def test_export_import_roundtrip_is_idempotent():
    rng = np.random.default_rng(25)
    perm = rng.permutation(128)
    for kind in L.KINDS:
        la = lay(kind, k_hi=16)
        S = rng.standard_normal((128, 128)) * 0.2
        reg = import_state(la, S, L.initial_region(la), perm)
        S1 = export_state(la, reg, perm)
        reg2 = import_state(la, S1, reg, perm)
        if kind in (L.HAD_INT8, L.MIXED):
            # the rotation round trip perturbs values by ~1e-16; codes stay equal
            S2 = export_state(la, reg2, perm)
            assert np.allclose(S2, S1, atol=1e-12)
        else:
            assert np.array_equal(reg2, reg), kind


def test_damp_error_energy_and_selection():
    rng = np.random.default_rng(26)
    x = rng.standard_normal(64)
    Hm = sylvester(64)
    e_direct = row_error_energy(x, 32)
    # orthonormal rotation: the error energy equals the rotated-domain error energy
    from oracle.quantizers import affine_metadata, affine_round
    y = Hm @ x
    e_rot = 0.0
    for g in range(0, 64, 32):
        sc, ze, _, _ = affine_metadata(y[g:g + 32])
        e_rot += np.sum((y[g:g + 32] - affine_round(y[g:g + 32], sc, ze, "rtn").xhat) ** 2)
    assert abs(e_direct - e_rot) < 1e-12 * max(e_rot, 1e-300) + 1e-30
    # synthetic calibration: the slowest rows reach the persistence cap and win
    inp = decode_inputs(7, 4, 1, 32, 32, 64)
    samples = calibration_samples(inp, 0, every=8)
    E, P, C = risk_scores(samples, inp["s"][0, 0], 0.01, 32)
    perm = select_permutation(C, 4)
    assert sorted(perm) == list(range(32))
    top = perm[:4]
    assert np.all(np.diff(top) > 0) and np.all(np.diff(perm[4:]) > 0)
    assert set(top) == set(np.argsort(-C, kind="stable")[:4])
    s = inp["s"][0, 0]
    assert np.mean(s[top]) < np.mean(s)
    assert np.allclose(P, 1 / np.maximum(1 - np.exp(-2 * s.astype(np.float64)), 0.01))
