"""Online decay and erasure estimators that feed the bit allocation.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

[LBRS] "State bit allocation": at each write-back the allocation takes
  s-hat_i = -1/2 log EMA_64(e^{2 g_{t,i}})   (g = -s the log decay of row i), and
  r_i     = 1/2 EMA_64[beta_t (2 - beta_t) k_{t,i}^2],
with an exponential moving average of target span 64 tokens that is chunk-aware.

Readings (the pages give no formula for the average):
  * span S means alpha = 2 / (S + 1) per token (the usual span convention), so
    alpha = 2/65;
  * the average is normalised by its weight sum: after tokens 1..n with values x_t,
    EMA = sum_t (1 - alpha)^(n - t) x_t / sum_t (1 - alpha)^(n - t), so a constant
    stream is reproduced exactly from the first token on (no start-up bias);
  * "chunk-aware": the tokens of a chunk enter one by one with their own weights, so a
    write-back after C tokens sees the same average as C single-token updates;
  * the decay average is kept as the average of 1 - e^{2g} = -expm1(-2 s) (the same
    information, without the cancellation of 1 - EMA near 1), and
    s-hat = -1/2 log(1 - EMA(1 - e^{2g})) = -1/2 log1p(-m);
  * with no token folded in yet (weight sum 0) there is no estimate; the allocation
    then gives every row the same persistence factor (range alone decides).
The state of one head is (N_a [dk], N_r [dk], W): the unnormalised averages and the
weight sum, all starting at 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SPAN = 64


def ema_alpha(span: int = SPAN) -> float:
    return 2.0 / (span + 1.0)


@dataclass
class EmaState:
    Na: np.ndarray                     # sum of weights times (1 - e^{2 g}) per row
    Nr: np.ndarray                     # sum of weights times beta (2 - beta) k_i^2 per row
    W: float = 0.0                     # sum of weights
    n: int = field(default=0)          # tokens folded in


def ema_init(dk: int) -> EmaState:
    return EmaState(Na=np.zeros(dk), Nr=np.zeros(dk), W=0.0, n=0)


def ema_fold(st: EmaState, s_rows, beta: float, k, span: int = SPAN) -> EmaState:
    """Fold one token in: every earlier weight shrinks by (1 - alpha), the new token
    enters with weight alpha."""
    a = ema_alpha(span)
    s_rows = np.asarray(s_rows, np.float64)
    k = np.asarray(k, np.float64)
    xa = -np.expm1(-2.0 * s_rows)
    xr = float(beta) * (2.0 - float(beta)) * k ** 2
    return EmaState(Na=(1.0 - a) * st.Na + a * xa, Nr=(1.0 - a) * st.Nr + a * xr,
                    W=(1.0 - a) * st.W + a, n=st.n + 1)


def ema_estimates(Na, Nr, W):
    """(s-hat, r) per row from the unnormalised averages, or (None, None) when no token
    has been folded in."""
    if W == 0.0:
        return None, None
    m = np.asarray(Na, np.float64) / W
    return -0.5 * np.log1p(-m), 0.5 * np.asarray(Nr, np.float64) / W
