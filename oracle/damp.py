"""DAMP risk score and the static per-head row permutation of the mixed layout.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

[DAMP] "Risk scoring and selection": for each key channel u,
  E_u      mean squared quantization-error energy of the row under the low-precision
           mapping (here: Hadamard rotation, then per-block asymmetric affine INT8
           with 32-value blocks, round to nearest, dequantize, rotate back);
  a_eff,u  geometric mean of the per-step retention, exp(E[log a_u]);
  P_u      1 / max(1 - a_eff,u^2, tau), the capped persistence;
  C_u      E_u * P_u; the K_hi = 16 highest-cost rows of each head stay in float16.
[DAMP] "Implementation": a per-head permutation places the protected rows
contiguously; it is computed once, offline. [DAMP] "Quantization & calibration
details": states are sampled every 8 tokens of a calibration stream.

The pages calibrate on text; with no model or corpus here, the calibration stream is
the synthetic one (a separate seed), run through the unquantized recurrence.
Ties in C_u go to the lower row index; perm lists the selected rows in ascending
order, then the others in ascending order.
"""
from __future__ import annotations

import numpy as np

from .hadamard import sylvester
from .quantizers import affine_metadata, affine_round
from .recurrence import delta_step


def row_error_energy(x, G: int = 32) -> float:
    """||x - H^-1 deQ(Q(H x))||^2 for one row x."""
    x = np.asarray(x, dtype=np.float64)
    Hm = sylvester(x.size)
    y = Hm @ x
    yhat = np.zeros_like(y)
    for g in range(0, y.size, G):
        scale, zero, _, _ = affine_metadata(y[g:g + G])
        yhat[g:g + G] = affine_round(y[g:g + G], scale, zero, "rtn").xhat
    xhat = Hm @ yhat
    return float(np.sum((x - xhat) ** 2))


def risk_scores(samples, s_rows, tau: float = 0.01, G: int = 32):
    """(E, P, C) per row from sampled states of one head [N][dk][dv]."""
    samples = np.asarray(samples, dtype=np.float64)
    N, dk, _ = samples.shape
    E = np.zeros(dk)
    for n in range(N):
        for u in range(dk):
            E[u] += row_error_energy(samples[n, u], G)
    E /= N
    a = np.exp(-np.broadcast_to(np.asarray(s_rows, np.float64), (dk,)))
    a_eff = np.exp(np.log(a))          # constant decay: the geometric mean is a itself
    P = 1.0 / np.maximum(1.0 - a_eff ** 2, tau)
    return E, P, E * P


def select_permutation(C, k_hi: int = 16):
    C = np.asarray(C, dtype=np.float64)
    order = sorted(range(C.size), key=lambda u: (-C[u], u))
    top = sorted(order[:k_hi])
    rest = sorted(order[k_hi:])
    return np.array(top + rest, dtype=np.int64)


def calibration_samples(inputs, h: int, every: int = 8):
    """Unquantized states of head h, sampled after every ``every``-th token, for each
    sequence of a calibration stream (inputs as produced by ``synth.decode_inputs``)."""
    q, k, v, beta, s = inputs["q"], inputs["k"], inputs["v"], inputs["beta"], inputs["s"]
    T, B = beta.shape[0], beta.shape[1]
    dk, dv = k.shape[-1], v.shape[-1]
    out = []
    for b in range(B):
        S = np.zeros((dk, dv))
        for t in range(T):
            S, _ = delta_step(S, q[t, b, h], k[t, b, h], v[t, b, h], beta[t, b, h], s[b, h])
            if (t + 1) % every == 0:
                out.append(S.copy())
    return np.stack(out)
