"""Pins of the recurrence, readout, persistence and erasure-rate functions."""
import json
import os

import numpy as np
import pytest

from oracle.hadamard import fwht, rotate_rows, sylvester
from oracle.recurrence import (delta_step, erasure_r, erasure_rate_approx,
                               exact_gramian_diag, persistence, transition, unrolled)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, n):
    g = rng.standard_normal(n)
    return g / np.linalg.norm(g)


@pytest.mark.parametrize("s", [1e-3, 1e-2, 0.1, 1.0])
def test_persistence_closed_form_vs_brute_force(s):
    # Low-Bit Recurrent States, "Proof sketch": sum_{l>=1} e^{-2 s l} = 1/expm1(2 s)
    lags = int(60.0 / (2 * s)) + 10
    l = np.arange(1, lags + 1, dtype=np.float64)
    brute = np.sum(np.exp(-2.0 * s * l)[::-1])
    assert abs(brute - persistence(s)) <= 1e-13 * persistence(s)


def test_step_matches_unrolled_product():
    rng = np.random.default_rng(3)
    dk, dv, T = 6, 5, 7
    S0 = rng.standard_normal((dk, dv))
    ks = [_unit(rng, dk) for _ in range(T)]
    vs = [rng.standard_normal(dv) for _ in range(T)]
    bs = list(rng.random(T))
    ss = [np.exp(rng.uniform(np.log(1e-3), 0, dk)) for _ in range(T)]
    S = S0
    for t in range(T):
        S, _ = delta_step(S, np.zeros(dk), ks[t], vs[t], bs[t], ss[t])
    assert np.max(np.abs(S - unrolled(S0, ks, vs, bs, ss))) < 1e-12


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((4, 3))
    s = np.array([0.1, 0.01, 1.0, 0.5])
    S = S0
    for _ in range(5):
        S, _ = delta_step(S, np.zeros(4), _unit(rng, 4), rng.standard_normal(3), 0.0, s)
    assert np.allclose(S, np.exp(-5 * s)[:, None] * S0, rtol=1e-14, atol=0)


def test_beta_one_overwrites_and_readout_uses_new_state():
    # with beta = 1 and a unit key the delta rule stores v exactly along k, for any
    # prior state; reading with q = k therefore returns v only if the readout is
    # taken from the updated state
    rng = np.random.default_rng(5)
    for _ in range(5):
        S0 = rng.standard_normal((8, 6)) * 3
        k = _unit(rng, 8)
        v = rng.standard_normal(6)
        s = np.exp(rng.uniform(-7, 0, 8))
        S, o = delta_step(S0, k, k, v, 1.0, s)
        assert np.allclose(S.T @ k, v, atol=1e-13)
        assert np.allclose(o, v, atol=1e-13)


def test_update_spectrum():
    rng = np.random.default_rng(6)
    k = _unit(rng, 5)
    beta = 0.37
    F = transition(k, beta, np.zeros(5), 5)
    ev = np.sort(np.linalg.eigvalsh((F + F.T) / 2))
    assert np.allclose(ev, sorted([1 - beta] + [1.0] * 4), atol=1e-14)
    assert np.linalg.norm(F, 2) <= 1 + 1e-14


def test_one_step_erasure_identity():
    # ||F e_i||^2 = e^{-2 s_i} (1 - beta (2 - beta) k_i^2) for a unit key; this is
    # the per-step erasure that r_i averages
    rng = np.random.default_rng(7)
    k = _unit(rng, 6)
    beta = 0.8
    s = np.exp(rng.uniform(-7, 0, 6))
    F = transition(k, beta, s, 6)
    lhs = np.sum(F * F, axis=0)
    rhs = np.exp(-2 * s) * (1 - beta * (2 - beta) * k ** 2)
    assert np.allclose(lhs, rhs, rtol=1e-13)


def test_erasure_rate_page_example():
    with open(os.path.join(GOLD, "erasure_rate_example.json")) as f:
        g = json.load(f)
    k = np.array([1.0, 1.0]) / np.sqrt(2.0)
    F = transition(k, g["beta"], g["s"], 2)
    exact = exact_gramian_diag(F, 20000)
    r = erasure_r([g["beta"]], [k])
    approx = erasure_rate_approx(g["s"], r, 1.0, g["C"])
    assert np.allclose(np.round(exact, 1), g["exact_gamma"])
    assert np.allclose(np.round(approx, 2), g["approx_gamma"])


def test_erasure_rate_reduces_to_persistence_without_writes():
    s = np.array([0.01, 1.0])
    assert np.allclose(erasure_rate_approx(s, 0.0), persistence(s), rtol=1e-15)
    F = transition(np.zeros(2), 0.0, s, 2)
    assert np.allclose(exact_gramian_diag(F, 5000), persistence(s), rtol=1e-12)


def test_hadamard_orthonormal_and_forms_agree():
    for n in (2, 4, 16, 128):
        Hm = sylvester(n)
        assert np.allclose(Hm @ Hm.T, np.eye(n), atol=1e-14)
        assert np.array_equal(Hm, Hm.T)
        assert np.allclose(np.abs(Hm), 1 / np.sqrt(n))
        x = np.random.default_rng(n).standard_normal((3, n))
        assert np.allclose(fwht(x), x @ Hm.T, atol=1e-13)
        assert np.allclose(rotate_rows(x), fwht(x), atol=1e-13)
    assert np.allclose(sylvester(2) * np.sqrt(2), [[1, 1], [1, -1]])
    assert np.allclose(sylvester(4) * 2, [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


def test_rotated_domain_update_identity():
    """The GPU keeps Hadamard rows rotated: with Y = S H (rows y_i = H x_i),
    u = sum_P k_i a_i S_i + H sum_Q k_i a_i Y_i, w = beta (v - u),
    float16 rows S_i' = a_i S_i + k_i w, rotated rows Y_i' = a_i Y_i + k_i H w,
    o = sum_P q_i S_i' + H sum_Q q_i Y_i'. Check against the plain step."""
    rng = np.random.default_rng(8)
    dk, dv, khi = 16, 128, 4
    Hm = sylvester(dv)
    S = rng.standard_normal((dk, dv))
    q, k = _unit(rng, dk), _unit(rng, dk)
    v = rng.standard_normal(dv)
    beta = 0.7
    s = np.exp(rng.uniform(-7, 0, dk))
    a = np.exp(-s)
    S_new, o = delta_step(S, q, k, v, beta, s)
    P, Q = slice(0, khi), slice(khi, dk)
    Y = S[Q] @ Hm.T
    u = (k[P] * a[P]) @ S[P] + Hm @ ((k[Q] * a[Q]) @ Y)
    w = beta * (v - u)
    SP = a[P, None] * S[P] + np.outer(k[P], w)
    YQ = a[Q, None] * Y + np.outer(k[Q], Hm @ w)
    o2 = q[P] @ SP + Hm @ (q[Q] @ YQ)
    assert np.max(np.abs(SP - S_new[P])) < 1e-12
    assert np.max(np.abs(YQ - S_new[Q] @ Hm.T)) < 1e-12
    assert np.max(np.abs(o2 - o)) < 1e-12
