"""Pins of the per-head allocation unit with block scales ([LBRS] "Allocation units",
"Levels and storage")."""
import itertools

import numpy as np

from oracle import layouts as L
from oracle.allocation import allocate_heads, fit_row, proxy_cost
from oracle.quantizers import levels_n
from oracle.recurrence import persistence_factor
from oracle.step import allocate_headalloc_regions, write_back


def _heads(rng, H, dk=64, dv=8):
    return [rng.standard_normal((dk, dv)) * np.exp(rng.uniform(-2, 0.5, (dk, 1))) for _ in range(H)]


def test_two_bit_mean_is_uniform_block_quantization():
    rng = np.random.default_rng(1)
    Ys = _heads(rng, 3)
    s = [np.full(64, v) for v in (1e-3, 0.1, 1.0)]
    al = allocate_heads(Ys, s, [0.01] * 3, bbar=2, bmin=2, bmax=8)
    assert al["widths"].tolist() == [2, 2, 2]
    for h in range(3):
        assert set(np.unique(al["kappa"][h])) <= {-1, 0, 1}


def test_decay_alone_sets_the_widths():
    rng = np.random.default_rng(2)
    Y = _heads(rng, 1)[0]
    s = [np.full(64, v) for v in (1e-3, 0.03, 1.0)]
    b = allocate_heads([Y, Y, Y], s, [0.01] * 3, bbar=4, bmin=2, bmax=8)["widths"]
    assert b.sum() == 12 and b[0] >= b[1] >= b[2] and b[0] > b[2]
    # the ranges of a head do not matter (R~ = 1)
    b2 = allocate_heads([Y, 100 * Y, 0.01 * Y], s, [0.01] * 3, bbar=4, bmin=2, bmax=8)["widths"]
    assert np.array_equal(b, b2)


def test_head_widths_are_the_brute_force_optimum_of_the_summed_costs():
    rng = np.random.default_rng(3)
    for _ in range(30):
        H = 3
        s = [np.exp(rng.uniform(np.log(1e-3), 0.0, 64)) for _ in range(H)]
        r = [np.full(64, 0.005)] * H
        al = allocate_heads(_heads(rng, H), s, r, bbar=4, bmin=2, bmax=8)
        c = np.array([np.sum(persistence_factor(s[h], r[h])) for h in range(H)])
        best = min(proxy_cost(c, np.array(w)) for w in itertools.product(range(2, 9), repeat=H) if sum(w) == 4 * H)
        assert np.isclose(proxy_cost(c, al["widths"]), best, rtol=1e-12)


def test_group_fit_and_step_follow_the_row_rule_on_32_values():
    rng = np.random.default_rng(4)
    Y = _heads(rng, 1)[0]
    al = allocate_heads([Y, Y], [np.full(64, 0.01), np.full(64, 0.5)], [0.01] * 2, bbar=4, bmin=2, bmax=8)
    for h in range(2):
        b = int(al["widths"][h])
        for g in range(2):
            for j in range(8):
                x = Y[32 * g: 32 * g + 32, j]
                k, _ = fit_row(x, float(np.max(np.abs(x))), b)
                assert al["fit"][h][g, j] == k
                d = al["delta"][h][g, j]
                assert np.all(np.abs(al["kappa"][h][32 * g: 32 * g + 32, j]) <= levels_n(b))
                assert np.all(np.abs(x - d * al["kappa"][h][32 * g: 32 * g + 32, j]) <= 0.5 * d + 1e-15 + (
                    np.abs(x) - levels_n(b) * d).clip(0))


def test_region_round_trip_and_write_back_idempotence():
    rng = np.random.default_rng(5)
    dk, dv, H = 64, 16, 3
    lay = L.Layout(kind=L.HEADALLOC, B=1, H=H, dk=dk, dv=dv, bbar=4, bmin=2, bmax=8)
    assert lay.region_size() == dk * dv + 3 * (dk // 32) * dv + 16
    regs = [L.initial_region(lay) for _ in range(H)]
    c0 = L.decode_region(lay, regs[0])
    assert c0.width == 4 and np.all(c0.fit == 15) and np.all(c0.kappa == 0)
    # import three states into the zero state's metadata, then one allocation pass
    Ys = _heads(rng, H, dk, dv)
    regs = [write_back(lay, Ys[h], None, 0, 0, h, prev=c0).region for h in range(H)]
    new, al = allocate_headalloc_regions(lay, regs, [np.full(dk, v) for v in (1e-3, 0.05, 1.0)], [0.01] * H)
    for h in range(H):
        c = L.decode_region(lay, new[h])
        assert c.width == al["widths"][h] and np.array_equal(L.encode_region(lay, c), new[h])
        used = dk * dv * c.width // 8
        assert np.all(new[h][used: lay.code_capacity] == 0)
        # stored values written back with the fits that put every group maximum on a
        # level (f = 1, k = 15) come back unchanged
        c15 = L.Content(kappa=c.kappa, width=c.width, fit=np.full_like(c.fit, 15), delta_bits=c.delta_bits,
                        delta=c.delta)
        Yh = L.stored_values(lay, c15)
        Rg = np.max(np.abs(Yh.reshape(dk // 32, 32, dv)), axis=1)
        n = levels_n(c.width)
        on_level = np.isclose(Rg, n * c.delta, rtol=0, atol=0)
        wb = write_back(lay, Yh, None, 0, 0, h, prev=c15)
        back = L.decode_region(lay, wb.region)
        cols = np.repeat(on_level, 32, axis=0)
        assert np.array_equal(back.kappa[cols], c.kappa[cols]) and on_level.any()
    assert len(set(int(w) for w in al["widths"])) > 1
