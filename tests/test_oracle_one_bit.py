"""Pins of one-bit rows ([LBRS] "Levels and storage": one bit stores the sign times the
mean absolute value) for the per-row allocation with b_min = 1."""
import itertools

import numpy as np

from oracle import layouts as L
from oracle.allocation import allocate_head, proxy_cost
from oracle.quantizers import one_bit_round, one_bit_step
from oracle.step import decode_step


def test_sign_times_mean_absolute_value():
    x = np.array([0.3, -0.1, 0.2, -0.4, 0.0])
    d, pre = one_bit_step(x)
    assert pre == 0.2 and d == float(np.float16(0.2))
    rr = one_bit_round(x, d, "rtn")
    # an exact zero is the half-step tie of the grid -Delta + k 2 Delta: the even index
    assert rr.kappa.tolist() == [1, -1, 1, -1, -1]
    # for fixed signs the mean absolute value is the least-squares scale
    a = np.abs(x)
    err = lambda s: np.sum((a - s) ** 2)
    assert err(pre) < err(pre * 1.01) and err(pre) < err(pre * 0.99)


def test_one_bit_floor_is_the_brute_force_optimum():
    rng = np.random.default_rng(7)
    for _ in range(20):
        Y = rng.standard_normal((4, 16)) * np.exp(rng.uniform(-4, 0.5, (4, 1)))
        s = np.exp(rng.uniform(np.log(1e-3), 1.0, 4))
        a = allocate_head(Y, s, 0.01, bbar=3, bmin=1, bmax=8)
        c = a["c"]
        best = min(proxy_cost(c, np.array(w)) for w in itertools.product(range(1, 9), repeat=4) if sum(w) == 12)
        assert a["widths"].sum() == 12 and np.isclose(proxy_cost(c, a["widths"]), best, rtol=1e-12)


def test_one_bit_rows_in_the_region_and_the_step():
    rng = np.random.default_rng(8)
    dk, dv = 16, 32
    lay = L.Layout(kind=L.BITALLOC, B=1, H=1, dk=dk, dv=dv, bbar=3, bmin=1, bmax=8, mode="rtn")
    w = np.array([1, 5, 1, 3, 2, 4, 1, 7, 3, 3, 2, 1, 4, 3, 4, 4])
    assert w.sum() == 3 * dk
    kap = np.stack([rng.choice([-1, 1], dv) if b == 1 else rng.integers(-(2 ** (b - 1) - 1), 2 ** (b - 1), dv)
                    for b in w])
    c = L.Content(kappa=kap, widths=w, fit=np.full(dk, 15), delta_bits=L.f16_bits(rng.random(dk)))
    reg = L.encode_region(lay, c)
    back = L.decode_region(lay, reg)
    assert np.array_equal(back.kappa, kap) and np.array_equal(back.widths, w)
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    r = decode_step(lay, reg, None, k, k, rng.standard_normal(dv), 0.6, np.full(dk, 0.05), 0, 0, 0)
    out = L.decode_region(lay, r.wb.region)
    for i in np.argwhere(w == 1).ravel():
        h = r.wb.X[i]
        assert out.delta[i] == float(np.float16(np.mean(np.abs(h))))
        assert np.array_equal(out.kappa[i], np.where(h > 0, 1, -1))
