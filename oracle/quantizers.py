"""Write-back rules and the grids they round onto.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Write-back maps the computed state h_t to the stored q_t ([WB] "Post-training
write-back interventions and diagnostics"; [WB-zh] "Core method" 核心方法 and
"Method steps" 方法步骤详情):
  * continuous propagation (identity): q_t = h_t;
  * deterministic B-bit: nearest level of a grid of spacing Delta_B, half-step ties
    to the even index, clipped at the grid rails ([WB-zh] "Reproduction assessment"
    复现评估);
  * stochastic rounding: one of the two adjacent levels, chosen with probability
    given by the relative position, so unbiased in expectation ([WB-zh] "Error
    feedback and stochastic rounding" 误差反馈与随机舍入);
  * error feedback: q_t = Q_B(h_t + e_{t-1}) with the residual e_t clipped to
    +-Delta_B (same section of [WB-zh]); e is an auxiliary write-back state.

Temporal-memory rules on the fixed uniform grid ([WB] "Interventions", "Post-training
write-back interventions and diagnostics", "Trajectory analysis"; [WB-zh] "Core
method"), the readings of this module:
  * quantized residual memory (k bits): error feedback whose carried residual is itself
    stored on a k-bit grid -- the clipped residual r in [-Delta_B, Delta_B] rounds to
    the nearest of j * Delta_B / 2^(k-1), j in [-2^(k-1), 2^(k-1) - 1] (ties to even j);
  * direction memory (k bits): a signed counter c per element. With q_{t-1} on level
    kappa_{t-1} and delta = h_t - q_{t-1}: if the nearest level of h_t differs from
    kappa_{t-1} the write is ordinary (stored, counter reset); otherwise a proposal with
    Delta_B/8 < |delta| < Delta_B/2 votes c += sign(delta) and, when |c| reaches
    T = 2^(k-1), the stored level moves one step in that direction (clipped at the grid
    rails) and the counter resets; smaller proposals leave level and counter unchanged.
    The counter therefore takes the 2^k - 1 values -(T-1) .. T-1.
Write activity of one step (per head; [WB] "Direction-memory events", "Persistence
metrics", "State diagnostics", "Write-back behavior"), read as eight counts:
  0 dead-zone elements (write margin M < 1);
  1 elements whose stored level changed;
  2 eligible votes: proposals with Delta_B/8 < |delta| < Delta_B/2, signed by delta
    (counted under every rule, whether or not a direction memory consumes them);
  3 direction-memory triggers (a trigger at a rail moves nothing);
  4 sub-threshold writes: M < 1 and the stored level changed anyway;
  5 / 6 same-sign / opposite-sign vote transitions: an eligible vote whose element
    also cast an eligible vote on the previous step, with the same / the other sign;
  7 runs started: an eligible vote that does not continue a run. A run is a string of
    eligible votes of one sign on consecutive steps; it ends at a reversal, an
    ineligible step, or a step whose vote changed the stored level or triggered (the
    ordinary write and the trigger that end runs). Every vote belongs to one run, so
    the mean run length over a sequence is count 2 / count 7, runs still open at its
    end included (they end at sequence termination).
The per-element state this needs between steps is one byte: 0 (no eligible vote),
1 / 2 (a positive / negative vote, run open), 5 / 6 (the same vote, run closed).

Every grid here is "offset + kappa * step" with integer kappa in [lo, hi]; a rule
works on the grid coordinate tau = (x - offset) / step.
  * uniform B-bit grid: offset 0, step Delta_B = 2^(1-B), kappa in
    [-2^(B-1), 2^(B-1) - 1]; Delta_4 = 0.125 ([WB-zh] "Core method").
  * per-block asymmetric affine INT8 ([DAMP] "Quantization & calibration details"):
    offset = f16(min), step = f16((max - min) / 255), kappa in [0, 255].
  * symmetric per-row levels {-n..n} Delta, n = 2^(b-1) - 1, Delta = f16(f R / n)
    ([LBRS] "Levels and storage").
Stochastic rounding compares a 16-bit uniform draw r with the fractional part:
kappa = floor(tau) + [r < frac(tau) * 2^16]; the rounding boundary is floor(tau) +
r / 2^16. A zero step (degenerate block or all-zero row) stores kappa = 0 and, with
error feedback, a zero residual.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import f16, rne

RTN, SR, EF, DIR, RESQ = "rtn", "sr", "ef", "dir", "resq"


@dataclass
class Rounded:
    kappa: np.ndarray      # integer level index (int64)
    xhat: np.ndarray       # dequantized value offset + kappa * step (float64)
    e_new: np.ndarray      # new error-feedback residual (zeros unless EF)
    tau: np.ndarray        # pre-rounding grid coordinate
    boundary: np.ndarray   # distance of tau to the rule's rounding boundary (grid units)


def round_on_grid(x, step, offset, lo, hi, mode, e=None, r16=None) -> Rounded:
    """Apply one write-back rule to values ``x`` on the grid offset + kappa * step.

    ``step`` and ``offset`` broadcast against ``x``; ``e`` is the incoming
    error-feedback residual (EF only); ``r16`` the 16-bit draws (SR only).
    """
    x = np.asarray(x, dtype=np.float64)
    step = np.broadcast_to(np.asarray(step, dtype=np.float64), x.shape)
    offset = np.broadcast_to(np.asarray(offset, dtype=np.float64), x.shape)
    target = x + (np.asarray(e, dtype=np.float64) if mode == EF else 0.0)
    zero_step = step == 0.0
    safe = np.where(zero_step, 1.0, step)
    tau = (target - offset) / safe
    if mode == SR:
        r = np.asarray(r16, dtype=np.float64).reshape(x.shape)
        fl = np.floor(tau)
        frac = tau - fl
        kappa = fl + (r < frac * 65536.0)
        boundary = np.abs(frac - r / 65536.0)
    else:
        kappa = rne(tau)
        boundary = np.abs(np.abs(tau - np.floor(tau) - 0.5))
    kappa = np.clip(kappa, lo, hi)
    kappa = np.where(zero_step, 0.0, kappa)
    boundary = np.where(zero_step, np.inf, boundary)
    xhat = offset + kappa * step
    if mode == EF:
        e_new = np.clip(target - xhat, -step, step)
    else:
        e_new = np.zeros_like(x)
    return Rounded(kappa.astype(np.int64), xhat, e_new, tau, boundary)


# ----- uniform B-bit grid ---------------------------------------------------

def uniform_step(B: int) -> float:
    return 2.0 ** (1 - B)


def uniform_round(x, B: int, mode: str, e=None, r16=None) -> Rounded:
    lo, hi = -(2 ** (B - 1)), 2 ** (B - 1) - 1
    return round_on_grid(x, uniform_step(B), 0.0, lo, hi, mode, e, r16)


def residual_quantize(r, step, kbits: int):
    """Nearest point of the k-bit residual grid j * step / 2^(k-1), j in
    [-2^(k-1), 2^(k-1) - 1], ties to even j. Returns (value, j, distance of r /
    (step / 2^(k-1)) to the rounding boundary)."""
    r = np.asarray(r, dtype=np.float64)
    step = np.broadcast_to(np.asarray(step, dtype=np.float64), r.shape)
    h = 2 ** (kbits - 1)
    sub = np.where(step == 0.0, 1.0, step / h)
    u = r / sub
    j = np.clip(rne(u), -h, h - 1)
    j = np.where(step == 0.0, 0.0, j)
    bnd = np.where(step == 0.0, np.inf, np.abs(np.abs(u - np.floor(u)) - 0.5))
    return j * np.where(step == 0.0, 0.0, sub), j.astype(np.int64), bnd


@dataclass
class MemoryRounded:
    kappa: np.ndarray       # stored level index (int64)
    side_new: np.ndarray    # new residual value (residual memory) or counter (direction memory)
    tau: np.ndarray         # grid coordinate of the value rounded (h or h + e)
    boundary: np.ndarray    # distance (grid units) to the nearest decision boundary
    triggers: np.ndarray    # direction-memory triggers (bool)


def uniform_memory_round(x, B: int, mode: str, kappa_prev, side, kbits: int) -> MemoryRounded:
    """Residual memory (mode RESQ, ``side`` = carried k-bit residual value) or direction
    memory (mode DIR, ``side`` = counter) on the uniform B-bit grid; ``kappa_prev`` are
    the stored levels entering the step."""
    x = np.asarray(x, dtype=np.float64)
    step = uniform_step(B)
    lo, hi = -(2 ** (B - 1)), 2 ** (B - 1) - 1
    kp = np.asarray(kappa_prev, dtype=np.int64)
    side = np.asarray(side, dtype=np.float64)
    q_prev = kp * step
    delta = x - q_prev
    ad = np.abs(delta) / step                              # |delta| in grid units
    tau_h = x / step
    near = np.clip(rne(tau_h), lo, hi)
    dead = 2.0 * ad < 1.0
    vote = (ad > 0.125) & (ad < 0.5)
    bnd_h = np.abs(np.abs(tau_h - np.floor(tau_h)) - 0.5)
    if mode == RESQ:
        target = x + side
        tau = target / step
        kappa = np.clip(rne(tau), lo, hi)
        r = np.clip(target - kappa * step, -step, step)
        e_val, _, bnd_e = residual_quantize(r, step, kbits)
        side_new = e_val
        boundary = np.minimum(np.abs(np.abs(tau - np.floor(tau)) - 0.5), bnd_e)
        moves = np.zeros_like(x, dtype=bool)
    elif mode == DIR:
        T = 2 ** (kbits - 1)
        ordinary = near != kp
        sgn = np.sign(delta)
        c = side + np.where(~ordinary & vote, sgn, 0.0)
        moves = ~ordinary & vote & (np.abs(c) >= T)
        kappa = np.where(ordinary, near, np.where(moves, np.clip(kp + sgn, lo, hi), kp))
        side_new = np.where(ordinary | moves, 0.0, c)
        tau = tau_h
        # decisions: the nearest level (half-integers of tau) and the vote band edges
        boundary = np.minimum(bnd_h, np.minimum(np.abs(ad - 0.125), np.abs(ad - 0.5)))
    else:
        raise ValueError(mode)
    return MemoryRounded(kappa.astype(np.int64), side_new, tau, boundary, moves)


def write_activity(x, kappa_prev, kappa_new, B: int, triggers, votes_prev):
    """The eight write-activity counts of one step on the uniform B-bit grid (h_t = x,
    levels entering and leaving the step, direction-memory triggers, the vote state of
    the previous step) and the new vote state; states and counts as described in the
    module docstring."""
    x = np.asarray(x, np.float64)
    kp = np.asarray(kappa_prev, np.int64)
    kn = np.asarray(kappa_new, np.int64)
    trig = np.asarray(triggers, bool)
    vp = np.asarray(votes_prev, np.int64)
    step = uniform_step(B)
    delta = x - kp * step
    ad = np.abs(delta) / step
    dead = 2.0 * ad < 1.0
    change = kn != kp
    vote = (ad > 0.125) & (ad < 0.5)
    sign = np.where(vote, np.where(delta > 0, 1, 2), 0)
    prev_sign = vp & 3
    same = vote & (prev_sign == sign)
    opposite = vote & (prev_sign != 0) & (prev_sign != sign)
    continues = vote & (vp == sign)                  # same sign, previous run still open
    closed = change | trig
    votes_new = np.where(vote, sign | np.where(closed, 4, 0), 0)
    counts = np.array([dead.sum(), change.sum(), vote.sum(), trig.sum(), (dead & change).sum(),
                       same.sum(), opposite.sum(), (vote & ~continues).sum()], dtype=np.int64)
    return counts, votes_new.astype(np.uint8)


def write_margin(h, q_prev, B: int):
    """M = 2 |h - q_prev| / Delta_B ([WB] "Methods", Diagnostics; [WB-zh] the margin
    M_{t,j} = 2|delta| / Delta_B of "Core method")."""
    return 2.0 * np.abs(np.asarray(h, np.float64) - np.asarray(q_prev, np.float64)) / uniform_step(B)


# ----- per-block asymmetric affine INT8 ---------------------------------------

def affine_metadata(x_block, bits: int = 8):
    """Returns (scale, zero, scale_pre, zero_pre): float16 values and their float64
    pre-rounding values, for one block of values; b-bit codes 0 .. 2^b - 1 ([DAMP]
    "Quantization & calibration details": b = 8 for INT8, b = 4 for INT4)."""
    x_block = np.asarray(x_block, dtype=np.float64)
    mn = float(np.min(x_block))
    mx = float(np.max(x_block))
    scale_pre = max(mx - mn, 0.0) / float(2 ** bits - 1)
    return float(f16(scale_pre)), float(f16(mn)), scale_pre, mn


def affine_round(x, scale, zero, mode, e=None, r16=None, bits: int = 8) -> Rounded:
    return round_on_grid(x, scale, zero, 0, 2 ** bits - 1, mode, e, r16)


# ----- symmetric per-row levels (decay-aware allocation) ---------------------

def fit_fraction(kfit: int) -> float:
    """Clipping fraction f_k = 1/4 + k/20, k = 0..15: sixteen values on [1/4, 1]
    ([LBRS] "Levels and storage")."""
    return 0.25 + kfit / 20.0


def levels_n(b: int) -> int:
    return 2 ** (b - 1) - 1


def row_step(R: float, b: int, kfit: int):
    """Delta = f16(f R / n) and its float64 pre-rounding value."""
    pre = fit_fraction(kfit) * R / levels_n(b)
    return float(f16(pre)), pre


def one_bit_step(x):
    """One-bit row ([LBRS] "Levels and storage": one bit stores the sign times the mean
    absolute value): Delta = f16(mean |x|) and its float64 pre-rounding value."""
    pre = float(np.mean(np.abs(np.asarray(x, np.float64))))
    return float(f16(pre)), pre


def one_bit_round(x, step, mode, e=None, r16=None) -> Rounded:
    """The rules on the two levels -Delta, +Delta: the grid -Delta + kappa' * 2 Delta,
    kappa' in {0, 1} (RTN: the sign, an exact zero being the half-step tie that goes to
    the even index, -Delta). Returns kappa = 2 kappa' - 1 in {-1, +1}."""
    step = np.broadcast_to(np.asarray(step, dtype=np.float64), np.shape(x))
    rr = round_on_grid(x, 2.0 * step, -step, 0, 1, mode, e, r16)
    return Rounded(kappa=2 * rr.kappa - 1, xhat=rr.xhat, e_new=rr.e_new, tau=rr.tau, boundary=rr.boundary)


def sym_round(x, step, n, mode, e=None, r16=None) -> Rounded:
    return round_on_grid(x, step, 0.0, -n, n, mode, e, r16)
