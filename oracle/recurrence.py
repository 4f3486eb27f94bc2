"""The gated delta rule, its readout, and the persistence quantities built on it.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

State S is dk x dv for one head; row i belongs to key channel i.

* Step ([LBRS] "Accumulated readout error": the transition between write-backs is
  F_t = (I - k_t a_t^T) D_t with a_t = beta_t k_t; [DAMP] "Error propagation model";
  [LBRS-x]: each row is multiplied by its decay e^{-s} before new information is
  written, with one s per row in KDA):
      S_t = (I - beta k k^T) Diag(e^{-s}) S_{t-1} + beta k v^T
  evaluated in its plain order: D = Diag(e^{-s}); u = k^T (D S); w = beta (v - u);
  S_t = D S + k w^T.
* Readout o_t = S_t^T q_t is taken from the unquantized S_t, before write-back
  ([LBRS] "Accumulated readout error": outputs precede quantization).
* Persistence sum: sum_{l>=1} e^{-2 s l} = 1 / expm1(2 s) ([LBRS] "Proof sketch").
* Approximate erasure rate Gamma_i ~ rho_i / [C expm1(2 (s_i + r_i))] with
  r_i = E[beta (2 - beta) k_i^2] / 2 ([LBRS] "Approximate erasure rate").
* Exact observability-Gramian diagonal Gamma_i = sum_{l>=1} ||F^l e_i||^2, which the
  same paragraph compares against the approximation ([LBRS-x] calls Gamma-hat an
  estimate of a diagonal entry of the observability Gramian).
"""
from __future__ import annotations

import numpy as np


def decay_factors(s, dk: int) -> np.ndarray:
    """a_i = e^{-s_i}; a scalar (per-head) s is broadcast to every row."""
    s = np.asarray(s, dtype=np.float64)
    return np.exp(-np.broadcast_to(s, (dk,)).astype(np.float64))


def delta_step(S, q, k, v, beta, s):
    """One gated delta-rule step; returns (S_t, o_t) in float64."""
    S = np.asarray(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = float(beta)
    a = decay_factors(s, S.shape[0])
    DS = a[:, None] * S
    u = k @ DS
    w = beta * (v - u)
    S_new = DS + np.outer(k, w)
    o = S_new.T @ q
    return S_new, o


def transition(k, beta, s, dk: int) -> np.ndarray:
    """F = (I - beta k k^T) Diag(e^{-s}) as an explicit dk x dk matrix."""
    k = np.asarray(k, dtype=np.float64)
    return (np.eye(dk) - float(beta) * np.outer(k, k)) @ np.diag(decay_factors(s, dk))


def unrolled(S0, ks, vs, betas, ss):
    """Product form: S_T = F_T ... F_1 S_0 + sum_t F_T ... F_{t+1} beta_t k_t v_t^T."""
    S0 = np.asarray(S0, dtype=np.float64)
    dk = S0.shape[0]
    T = len(ks)
    Fs = [transition(ks[t], betas[t], ss[t], dk) for t in range(T)]
    total = np.eye(dk)
    for F in Fs:
        total = F @ total
    S = total @ S0
    for t in range(T):
        tail = np.eye(dk)
        for F in Fs[t + 1:]:
            tail = F @ tail
        S = S + tail @ (float(betas[t]) * np.outer(ks[t], vs[t]))
    return S


def persistence(s):
    """Closed form of sum_{l>=1} e^{-2 s l}."""
    return 1.0 / np.expm1(2.0 * np.asarray(s, dtype=np.float64))


def erasure_rate_approx(s, r, rho=1.0, C=1):
    """Gamma-hat_i = rho_i / [C expm1(2 (s_i + r_i))]."""
    s = np.asarray(s, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.asarray(rho, dtype=np.float64) / (C * np.expm1(2.0 * (s + r)))


GAMMA_ERASURE, GAMMA_W1, GAMMA_HC = "erasure", "w1", "hC"


def persistence_factor(s, r, kind: str = GAMMA_ERASURE, C: int = 1):
    """The persistence factor of each row that weights its range in the allocation
    ([LBRS] "Approximate erasure rate", "Choice of persistence factor", "Related work"):
      erasure  rho / [C expm1(2 (s + r))]  with rho = 1 (the default);
      w1       1 / (1 - a^2), a = e^{-s}: DAMP's factor, uncapped;
      hC       1 / (1 - e^{-2 C s}): the write-back-time factor.
    w1 and hC do not use r."""
    s = np.asarray(s, dtype=np.float64)
    if kind == GAMMA_ERASURE:
        return erasure_rate_approx(s, r, 1.0, C)
    a = np.exp(-s)
    if kind == GAMMA_W1:
        return 1.0 / (1.0 - a ** 2)
    if kind == GAMMA_HC:
        return 1.0 / (1.0 - np.exp(-2.0 * C * s))
    raise ValueError(kind)


def erasure_r(betas, ks):
    """r_i = E[beta (2 - beta) k_i^2] / 2 as a sample mean over a stream of tokens."""
    betas = np.asarray(betas, dtype=np.float64)
    ks = np.asarray(ks, dtype=np.float64)
    return 0.5 * np.mean((betas * (2.0 - betas))[:, None] * ks ** 2, axis=0)


def exact_gramian_diag(F, lags: int) -> np.ndarray:
    """Gamma_i = sum_{l=1..lags} ||F^l e_i||^2 for a fixed transition F (brute force)."""
    F = np.asarray(F, dtype=np.float64)
    n = F.shape[0]
    P = np.eye(n)
    g = np.zeros(n)
    for _ in range(lags):
        P = F @ P
        g += np.sum(P * P, axis=0)
    return g
