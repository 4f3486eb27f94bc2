"""Pins of the write-back rules and grids."""
import json
import os

import numpy as np

from oracle.numerics import f16
from oracle.quantizers import (affine_metadata, affine_round, fit_fraction, levels_n,
                               row_step, sym_round, uniform_round, uniform_step,
                               write_margin)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_uniform_grid_constants():
    with open(os.path.join(GOLD, "layout_accounting.json")) as f:
        g = json.load(f)
    assert uniform_step(4) == g["delta_4"]
    assert uniform_step(4) / 2 == g["half_step_4"]
    # rails: two's-complement 4-bit levels cover [-1, 1 - Delta]
    r = uniform_round(np.array([1.0, 5.0, -1.0, -7.0, 0.875]), 4, "rtn")
    assert list(r.kappa) == [7, 7, -8, -8, 7]
    assert list(r.xhat) == [0.875, 0.875, -1.0, -1.0, 0.875]


def test_uniform_ties_go_to_even_index():
    d = uniform_step(4)
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 3.5]) * d
    assert list(uniform_round(x, 4, "rtn").kappa) == [0, 2, 2, 0, -2, 4]


def test_dead_zone():
    """Margin M = 2|h - q_prev| / Delta < 1 keeps an interior stored level; M > 1
    moves it (When Quantization Breaks Memory, Methods / Diagnostics)."""
    rng = np.random.default_rng(9)
    B = 4
    d = uniform_step(B)
    kprev = rng.integers(-7, 7, 20000)                 # interior levels
    qprev = kprev * d
    h = qprev + rng.uniform(-1.5, 1.5, kprev.size) * d
    M = write_margin(h, qprev, B)
    k_new = uniform_round(h, B, "rtn").kappa
    inside = M < 1
    assert np.all(k_new[inside] == kprev[inside])
    assert np.all(k_new[M > 1] != kprev[M > 1])


def test_error_feedback_bounds_and_telescoping():
    rng = np.random.default_rng(10)
    B = 4
    d = uniform_step(B)
    e = np.zeros(50)
    total = np.zeros(50)
    for _ in range(300):
        h = rng.uniform(-0.6, 0.6, 50)          # away from the rails: no clip fires
        r = uniform_round(h, B, "ef", e=e)
        assert np.all(np.abs(r.e_new) <= d)
        total += h - r.xhat
        e = r.e_new
    assert np.allclose(total, e, atol=1e-12)      # sum (h_t - q_t) = e_T - e_0


def test_error_feedback_clips_at_rails():
    r = uniform_round(np.array([3.0]), 4, "ef", e=np.array([0.05]))
    assert r.kappa[0] == 7 and r.e_new[0] == uniform_step(4)


def test_stochastic_rounding_unbiased():
    rng = np.random.default_rng(11)
    x = rng.uniform(-0.8, 0.8, 64)
    n = 4000
    acc = np.zeros_like(x)
    up = np.zeros_like(x)
    for _ in range(n):
        r16 = rng.integers(0, 65536, x.size)
        rr = uniform_round(x, 4, "sr", r16=r16)
        acc += rr.xhat
        up += rr.kappa > np.floor(rr.tau)
    d = uniform_step(4)
    frac = x / d - np.floor(x / d)
    # E[q] = x and P(up) = frac (binomial error bars, 5 sigma)
    sig = np.sqrt(frac * (1 - frac) / n)
    assert np.all(np.abs(up / n - frac) <= 5 * sig + 2 ** -16)
    assert np.all(np.abs(acc / n - x) <= 5 * sig * d + d * 2 ** -16)


def test_affine_block_metadata_and_idempotence():
    rng = np.random.default_rng(12)
    for _ in range(200):
        blk = rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 1)
        scale, zero, spre, zpre = affine_metadata(blk)
        assert scale == f16(spre) and zero == f16(zpre)
        r = affine_round(blk, scale, zero, "rtn")
        assert r.kappa.min() == 0 and r.kappa.max() == 255
        assert np.all(np.abs(r.xhat - blk) <= scale / 2 * (1 + 1e-9) + abs(zero - zpre) + 1e-300)
        s2, z2, _, _ = affine_metadata(r.xhat)
        assert (s2, z2) == (scale, zero)
        r2 = affine_round(r.xhat, s2, z2, "rtn")
        assert np.array_equal(r2.kappa, r.kappa)


def test_affine_degenerate_block():
    blk = np.full(32, 0.3)
    scale, zero, _, _ = affine_metadata(blk)
    assert scale == 0.0
    r = affine_round(blk, scale, zero, "ef", e=np.full(32, 0.01))
    assert np.all(r.kappa == 0) and np.all(r.xhat == zero) and np.all(r.e_new == 0)


def test_symmetric_row_levels():
    assert [levels_n(b) for b in range(2, 9)] == [1, 3, 7, 15, 31, 63, 127]
    fr = [fit_fraction(k) for k in range(16)]
    assert fr[0] == 0.25 and fr[-1] == 1.0 and len(set(fr)) == 16
    rng = np.random.default_rng(13)
    for b in range(2, 9):
        x = rng.standard_normal(128)
        R = np.max(np.abs(x))
        d, pre = row_step(R, b, 15)
        r = sym_round(x, d, levels_n(b), "rtn")
        assert np.abs(r.kappa).max() == levels_n(b)
        # idempotence at f = 1: the extreme value maps to +-n, so the refit is equal
        d2, _ = row_step(np.max(np.abs(r.xhat)), b, 15)
        assert d2 == d
        assert np.array_equal(sym_round(r.xhat, d2, levels_n(b), "rtn").kappa, r.kappa)
    z = sym_round(np.zeros(8), 0.0, 7, "rtn")
    assert np.all(z.kappa == 0)


# ---- temporal-memory rules on the uniform grid (direction / residual memory) ----------
# The expected values follow the rule text directly: the vote band Delta/8 < |delta| <
# Delta/2 with strict edges, a one-level move when the counter reaches 2^(k-1), the
# counter reset at every stored-level change, moves clipped at the rails; the residual
# of error feedback kept on the k-bit grid j Delta / 2^(k-1), j in [-2^(k-1), 2^(k-1)).

from oracle.quantizers import residual_quantize, uniform_memory_round, write_activity  # noqa: E402


def _dir(x, kp, c, k=2, B=4):
    return uniform_memory_round(np.array(x, float), B, "dir", np.array(kp), np.array(c, float), k)


def _act(x, kp, r, B=4):
    """[dead-zone, changes, votes, triggers] of one step from no previous vote."""
    n = len(x)
    return write_activity(np.array(x, float), np.array(kp), r.kappa, B, r.triggers, np.zeros(n))[0][:4].tolist()


def test_direction_memory_votes_trigger_and_reset():
    d = uniform_step(4)                       # 0.125: vote band (0.015625, 0.0625)
    # one vote up, counter 0 -> 1, no move (T = 2 for k = 2)
    r = _dir([0.03], [0], [0])
    assert r.kappa.tolist() == [0] and r.side_new.tolist() == [1.0]
    # the second same-sign vote reaches T: one level up, counter reset
    r = _dir([0.03], [0], [1])
    assert r.kappa.tolist() == [1] and r.side_new.tolist() == [0.0]
    assert _act([0.03], [0], r) == [1, 1, 1, 1]
    # an opposite vote takes the counter back, no move
    r = _dir([-0.03], [0], [1])
    assert r.kappa.tolist() == [0] and r.side_new.tolist() == [0.0]
    # below the band: neither vote nor reset
    r = _dir([0.01], [0], [1])
    assert r.kappa.tolist() == [0] and r.side_new.tolist() == [1.0]
    assert _act([0.01], [0], r) == [1, 0, 0, 0]
    # an ordinary write (nearest level changes) stores it and resets the counter
    r = _dir([0.07], [0], [-1])
    assert r.kappa.tolist() == [1] and r.side_new.tolist() == [0.0]
    assert _act([0.07], [0], r) == [0, 1, 0, 0]
    # the band edges are excluded: |delta| = Delta/8 and |delta| = Delta/2 (a tie that
    # rounds back to the even level 0) do not vote
    r = _dir([d / 8, d / 2, -d / 8], [0, 0, 0], [1, 1, 1])
    assert r.kappa.tolist() == [0, 0, 0] and r.side_new.tolist() == [1.0, 1.0, 1.0]
    # proposals relative to a nonzero stored level
    r = _dir([3 * d + 0.03, -5 * d - 0.03], [3, -5], [1, -1])
    assert r.kappa.tolist() == [4, -6] and r.side_new.tolist() == [0.0, 0.0]


def test_direction_memory_rails_and_counter_range():
    d = uniform_step(4)
    # at the upper rail a trigger cannot move the level; the counter still resets
    r = _dir([7 * d + 0.03, -8 * d - 0.03], [7, -8], [1, -1])
    assert r.kappa.tolist() == [7, -8] and r.side_new.tolist() == [0.0, 0.0]
    assert _act([7 * d + 0.03, -8 * d - 0.03], [7, -8], r) == [2, 0, 2, 2]
    # k = 3: T = 4, the counter runs through -3 .. 3 before a move
    c, kp = 0.0, 0
    seen = []
    for _ in range(4):
        r = _dir([kp * d + 0.03], [kp], [c], k=3)
        kp, c = int(r.kappa[0]), float(r.side_new[0])
        seen.append((kp, c))
    assert seen == [(0, 1.0), (0, 2.0), (0, 3.0), (1, 0.0)]
    for _ in range(3):
        r = _dir([kp * d - 0.03], [kp], [c], k=3)
        kp, c = int(r.kappa[0]), float(r.side_new[0])
    assert (kp, c) == (1, -3.0)


def test_residual_memory_grid_and_carry():
    d = uniform_step(4)
    # k = 2: residual points {-d, -d/2, 0, d/2}; ties to the even index
    v, j, _ = residual_quantize(np.array([0.03, 0.04, -d, d, d / 4, 3 * d / 4]), d, 2)
    assert j.tolist() == [0, 1, -2, 1, 0, 1]
    assert v.tolist() == [0.0, d / 2, -d, d / 2, 0.0, d / 2]
    # a sub-threshold proposal is remembered on the k-bit grid and later written
    x = np.array([0.04])
    r1 = uniform_memory_round(x, 4, "resq", np.array([0]), np.array([0.0]), 2)
    assert r1.kappa.tolist() == [0] and r1.side_new.tolist() == [d / 2]
    r2 = uniform_memory_round(x, 4, "resq", r1.kappa, r1.side_new, 2)
    assert r2.kappa.tolist() == [1]
    assert np.isclose(r2.side_new[0], 0.0)           # residual 0.04 + d/2 - d = -0.0225
    # with many residual bits the rule is error feedback (residual clipped to +-d)
    rng = np.random.default_rng(3)
    xs = rng.uniform(-1.2, 1.2, 200)
    es = rng.uniform(-d, d, 200)
    r = uniform_memory_round(xs, 4, "resq", np.zeros(200, np.int64), es, 30)
    ef = uniform_round(xs, 4, "ef", es)
    assert np.array_equal(r.kappa, ef.kappa)
    assert np.allclose(r.side_new, ef.e_new, atol=d * 2.0 ** -28)


def _run_sequence(xs_rel, k=3, B=4, mode="dir"):
    """Drive one element through proposals given relative to its stored level; returns
    the summed eight counts and the per-step (vote sign, level changed or triggered)."""
    d = uniform_step(B)
    kp, side, vs = 0, 0.0, np.zeros(1)
    total = np.zeros(8, np.int64)
    events = []
    for rel in xs_rel:
        x = np.array([kp * d + rel])
        if mode in ("dir", "resq"):
            r = uniform_memory_round(x, B, mode, np.array([kp]), np.array([side]), k)
            kn, side, trig = r.kappa, float(r.side_new[0]), r.triggers
        else:
            rr = uniform_round(x, B, mode, np.array([side]))
            kn, trig = rr.kappa, np.zeros(1, bool)
            side = float(rr.e_new[0]) if mode == "ef" else 0.0
        cnt, vs = write_activity(x, np.array([kp]), kn, B, trig, vs)
        total += cnt
        a = abs(rel) / d
        sign = (1 if rel > 0 else -1) if 0.125 < a < 0.5 else 0
        events.append((sign, bool(kn[0] != kp or trig[0])))
        kp = int(kn[0])
    return total, events


def test_vote_persistence_hand_sequence():
    # k = 3 (T = 4), Delta = 0.125, vote band (0.015625, 0.0625) around the stored level:
    # + + - (small) + + +(trigger: level 0 -> 1) +
    total, _ = _run_sequence([0.03, 0.03, -0.03, 0.01, 0.03, 0.03, 0.03, 0.03])
    # dead 8, changes 1, votes 7, triggers 1, sub-threshold writes 1 (the trigger),
    # same-sign pairs 4 (steps 1, 5, 6, 7), opposite 1 (step 2), runs 4:
    # [0, 1], [2], [4, 5, 6], [7] -- the trigger ends the third run
    assert total.tolist() == [8, 1, 7, 1, 1, 4, 1, 4]


def test_vote_persistence_matches_brute_force_runs():
    """Runs split by a second method: maximal groups of equal nonzero sign on consecutive
    steps, cut again after every step that changed the level or triggered."""
    import itertools
    rng = np.random.default_rng(11)
    d = uniform_step(4)
    for mode, k in (("dir", 2), ("dir", 3), ("rtn", 0), ("ef", 0), ("resq", 2)):
        rel = rng.choice([-0.7, -0.4, -0.03, -0.01, 0.0, 0.01, 0.03, 0.05, 0.4, 0.7], size=400) * d * 8
        total, ev = _run_sequence(rel, k=max(k, 1), mode=mode)
        runs = 0
        for sgn, grp in itertools.groupby(ev, key=lambda e: e[0]):
            if sgn == 0:
                continue
            g = list(grp)
            runs += 1 + sum(1 for e in g[:-1] if e[1])
        pairs = list(zip(ev, ev[1:]))
        same = sum(1 for a, b in pairs if a[0] != 0 and a[0] == b[0])
        opp = sum(1 for a, b in pairs if a[0] != 0 and b[0] != 0 and a[0] != b[0])
        votes = sum(1 for e in ev if e[0] != 0)
        assert (total[2], total[5], total[6], total[7]) == (votes, same, opp, runs), mode
        assert votes > 50 and runs < votes and opp > 0
        # nearest-level writing never changes a level below the write margin; under
        # direction memory only a trigger that is not held at a rail does
        if mode == "rtn":
            assert total[4] == 0 and total[3] == 0
        if mode == "dir":
            assert 0 < total[4] <= total[3]
