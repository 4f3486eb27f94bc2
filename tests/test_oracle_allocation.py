"""Pins of the decay-aware bit allocation."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.allocation import (allocate_head, default_r, fit_row, integer_widths,
                               proxy_cost, real_widths, row_costs)
from oracle.recurrence import persistence

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    with open(os.path.join(GOLD, "worked_example_allocation.json")) as f:
        g = json.load(f)
    wA = float(persistence(g["s_row_A"]))
    wB = float(persistence(g["s_row_B"]))
    assert round(wA, 1) == g["persistence_A"]
    assert round(wB, 3) == g["persistence_B"]
    # "about 315": the ratio of the printed (rounded) weights; the exact ratio is 316.3
    assert abs(wA / wB - g["cost_ratio_about"]) / g["cost_ratio_about"] < 0.01
    c = np.array([wA, wB])                      # equal ranges: c = persistence
    bstar = real_widths(c, g["mean_bits"])
    assert round(bstar[0] - bstar[1], 2) == g["extra_bits_A_over_B"]
    b = integer_widths(c, bstar, g["mean_bits"], 1, 16)
    assert list(b) == [g["bits_A"], g["bits_B"]]
    uni = proxy_cost(c, [4, 4])
    alloc = proxy_cost(c, b)
    assert round(uni, 3) == g["proxy_uniform"]
    assert round(alloc, 3) == g["proxy_allocated"]
    assert round(uni / alloc) == g["gain_about"]


def test_real_widths_keep_the_mean_and_give_am_over_gm():
    rng = np.random.default_rng(14)
    for _ in range(50):
        c = np.exp(rng.uniform(-8, 8, 64))
        bstar = real_widths(c, 4.0)
        assert abs(np.mean(bstar) - 4.0) < 1e-12
        am = np.mean(c)
        gm = np.exp(np.mean(np.log(c)))
        gain = proxy_cost(c, np.full(64, 4.0)) / proxy_cost(c, bstar)
        assert abs(gain - am / gm) < 1e-9 * am / gm


@pytest.mark.parametrize("n", [3, 4])
def test_integer_widths_reach_the_brute_force_optimum(n):
    rng = np.random.default_rng(15 + n)
    bbar, bmin, bmax = 4, 2, 8
    for _ in range(300):
        c = np.exp(rng.uniform(-12, 12, n))
        b = integer_widths(c, real_widths(c, bbar), bbar, bmin, bmax)
        assert b.sum() == bbar * n and b.min() >= bmin and b.max() <= bmax
        best = min(proxy_cost(c, w) for w in itertools.product(range(bmin, bmax + 1), repeat=n)
                   if sum(w) == bbar * n)
        assert proxy_cost(c, b) <= best * (1 + 1e-12)


def test_range_normalisation_and_costs():
    rng = np.random.default_rng(16)
    Y = rng.standard_normal((128, 128)) * np.exp(rng.uniform(-3, 3, 128))[:, None]
    s = np.exp(rng.uniform(np.log(1e-3), 0, 128))
    R, Rt, G, c = row_costs(Y, s, default_r(128))
    assert np.allclose(R, np.max(np.abs(Y), axis=1))
    assert abs(np.sqrt(np.mean(Rt ** 2)) - 1.0) < 1e-12
    assert np.allclose(c, G * Rt ** 2)
    assert abs(default_r(128) - 1.0 / 384.0) < 1e-18


def test_allocate_head_budget_and_guards():
    rng = np.random.default_rng(17)
    Y = rng.standard_normal((128, 128)) * np.exp(rng.uniform(-3, 3, 128))[:, None]
    s = np.exp(rng.uniform(np.log(1e-3), 0, 128))
    a = allocate_head(Y, s, default_r(128))
    assert a["widths"].sum() == 512
    assert a["widths"].min() >= 2 and a["widths"].max() <= 8
    # slower rows of equal range get at least as many bits
    Yeq = np.ones((128, 128))
    a2 = allocate_head(Yeq, np.sort(s), default_r(128))
    assert np.all(np.diff(a2["widths"]) <= 0)
    z = allocate_head(np.zeros((128, 128)), s, default_r(128))
    assert np.all(z["widths"] == 4)


def test_fit_prefers_exact_grid():
    # values exactly on the f = 1 grid of width 4 have zero error at k = 15
    n = 7
    d = 0.125
    x = np.arange(-n, n + 1) * d
    k, errs = fit_row(np.tile(x, 9)[:128], n * d, 4)
    assert k == 15 and errs[15] == 0.0
    # a dense row with one moderate outlier: clipping it lowers the squared error
    rng = np.random.default_rng(18)
    x = rng.uniform(-1, 1, 128)
    x[0] = 1.6
    k, errs = fit_row(x, 1.6, 3)
    assert k < 15 and errs[k] == errs.min() and errs[k] < errs[15]
