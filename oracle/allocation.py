"""Decay-aware per-row bit allocation for one head.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

[LBRS] "State bit allocation", "Range normalization", "Approximate erasure rate",
"Allocation units", "Levels and storage"; [LBRS-x] (the cost c = Gamma-hat * R~^2 and
the rule "mean budget plus half log2 of cost over its geometric mean"):

  R_i     row absolute maximum of the currently stored (dequantized) state;
  R~_i    R_i / RMS_j R_j over the normalisation group (one head for KDA);
  Gamma_i the persistence factor: 1 / [C expm1(2 (s_i + r_i))] (rho_i = 1) by default,
          or DAMP's uncapped 1 / (1 - a_i^2), or 1 / (1 - e^{-2 C s_i})
          ([LBRS] "Choice of persistence factor"); with no decay estimate (online
          estimators that have seen no token) every row gets the same factor;
  c_i     Gamma_i * R~_i^2;
  b*_i    bbar + 0.5 * log2(c_i / GM(c))  -- the real-valued minimiser of
          sum_i c_i 2^{-2 b_i} at mean bbar (the displayed equation is missing from
          the extracted page; the explainer states the rule in words);
  b_i     round (ties to even), clip to [bmin, bmax], then adjust one bit at a time
          until sum b_i = bbar * dk: while short, +1 to the row of largest marginal
          gain (3/4) c_i 2^{-2 b_i} among b_i < bmax; while over, -1 to the row of
          smallest marginal loss 3 c_i 2^{-2 b_i} among b_i > bmin; ties go to the
          lower row index (the page says only "adjust widths to meet the budget").
  fit     for each row, f_k = 1/4 + k/20 (k = 0..15); Delta_k = f16(f_k R_i / n_i);
          squared error of rounding the row to {-n..n} Delta_k; the smallest error
          wins, ties to the larger f ("fit f over 16 values in [1/4, 1] by squared
          error per scale group").

Guards (the pages are silent): every b_i = bbar when all R_i = 0; c_i is kept in
[1e-300, 1e300] before logarithms (an infinite factor, s + r = 0, is the cap);
Delta_k = 0 stores level 0.
"""
from __future__ import annotations

import numpy as np

from .numerics import f16, rne
from .quantizers import fit_fraction, levels_n, one_bit_round, one_bit_step
from .recurrence import GAMMA_ERASURE, persistence_factor

C_FLOOR = 1e-300
C_CAP = 1e300


def proxy_cost(c, b):
    """Distortion proxy sum_i c_i 2^{-2 b_i}."""
    return float(np.sum(np.asarray(c, np.float64) * 2.0 ** (-2.0 * np.asarray(b, np.float64))))


def real_widths(c, bbar: float):
    """b*_i = bbar + 0.5 log2(c_i / GM(c))."""
    c = np.maximum(np.asarray(c, dtype=np.float64), C_FLOOR)
    gm = np.exp(np.mean(np.log(c)))
    return bbar + 0.5 * np.log2(c / gm)


def integer_widths(c, bstar, bbar: int, bmin: int, bmax: int):
    """Round, clip and greedily adjust to the budget sum b_i = bbar * len(c)."""
    c = np.maximum(np.asarray(c, dtype=np.float64), C_FLOOR)
    b = np.clip(rne(bstar), bmin, bmax).astype(np.int64)
    target = bbar * len(c)
    while b.sum() < target:
        gain = np.where(b < bmax, 0.75 * c * 2.0 ** (-2.0 * b), -np.inf)
        b[int(np.argmax(gain))] += 1
    while b.sum() > target:
        loss = np.where(b > bmin, 3.0 * c * 2.0 ** (-2.0 * b), np.inf)
        b[int(np.argmin(loss))] -= 1
    return b


def row_costs(Y, s_rows, r_rows, factor=GAMMA_ERASURE, C=1):
    """(R, R~, Gamma-hat, c) of one head from its stored values Y [dk][dv]; s_rows None
    means no decay estimate (Gamma = 1 for every row)."""
    Y = np.asarray(Y, dtype=np.float64)
    R = np.max(np.abs(Y), axis=1)
    rms = np.sqrt(np.mean(R ** 2))
    Rt = R / rms if rms > 0 else np.zeros_like(R)
    if s_rows is None:
        G = np.ones_like(R)
    else:
        with np.errstate(divide="ignore"):
            G = persistence_factor(s_rows, r_rows, factor, C)
    return R, Rt, G, np.minimum(G * Rt ** 2, C_CAP)


def fit_row(x, R: float, b: int):
    """Clipping-fit index k and the row's squared errors for all 16 candidates; a
    one-bit row has no fit (sign times mean |x|): every candidate carries its error and
    k = 15 is kept."""
    x = np.asarray(x, dtype=np.float64)
    if b == 1:
        d, _ = one_bit_step(x)
        return 15, np.full(16, float(np.sum((x - d * one_bit_round(x, d, "rtn").kappa) ** 2)))
    n = levels_n(b)
    errs = np.zeros(16)
    for k in range(16):
        d = float(f16(fit_fraction(k) * R / n))
        if d == 0.0:
            kap = np.zeros_like(x)
        else:
            kap = np.clip(rne(x / d), -n, n)
        errs[k] = np.sum((x - d * kap) ** 2)
    best = 15
    for k in range(14, -1, -1):        # ties go to the larger f
        if errs[k] < errs[best]:
            best = k
    return best, errs


def allocate_head(Y, s_rows, r_rows, bbar=4, bmin=2, bmax=8, factor=GAMMA_ERASURE, C=1):
    """Widths, fit indices and diagnostics for one head's stored values Y."""
    Y = np.asarray(Y, dtype=np.float64)
    dk = Y.shape[0]
    R, Rt, G, c = row_costs(Y, s_rows, r_rows, factor, C)
    if np.all(R == 0):
        bstar = np.full(dk, float(bbar))
        b = np.full(dk, bbar, dtype=np.int64)
    else:
        bstar = real_widths(c, bbar)
        b = integer_widths(c, bstar, bbar, bmin, bmax)
    fits = np.zeros(dk, dtype=np.int64)
    errs = np.zeros((dk, 16))
    for i in range(dk):
        fits[i], errs[i] = fit_row(Y[i], R[i], int(b[i]))
    return {"widths": b, "fit": fits, "bstar": bstar, "c": np.maximum(c, C_FLOOR),
            "R": R, "Rt": Rt, "Gamma": G, "fit_err": errs}


def allocate_layer(Ys, s_rows, r_rows, bbar=4, bmin=2, bmax=8, factor=GAMMA_ERASURE, C=1):
    """Widths and fit indices for the heads of one layer of one sequence under the
    layer-wise mean budget ([LBRS] "State bit allocation": "at layer-wise mean budget
    bbar"; "Range normalization": R~ within each output group, one head). Costs per
    head as in ``allocate_head``; the geometric mean, the rounding and the one-bit
    adjustments run over all rows of the layer (sum b = bbar * rows, ties to the
    lower (head, row)); every row keeps bbar only when the whole layer is zero.
    ``Ys`` [H][dk][dv]; ``s_rows`` / ``r_rows`` per head (None: no decay estimate).
    Returns one dict per head, as ``allocate_head``."""
    H = len(Ys)
    parts = [row_costs(Ys[h], None if s_rows is None else s_rows[h], None if r_rows is None else r_rows[h],
                       factor, C) for h in range(H)]
    dk = len(parts[0][0])
    c_all = np.concatenate([p[3] for p in parts])
    if all(np.all(p[0] == 0) for p in parts):
        bstar = np.full(H * dk, float(bbar))
        b = np.full(H * dk, bbar, dtype=np.int64)
    else:
        bstar = real_widths(c_all, bbar)
        b = integer_widths(c_all, bstar, bbar, bmin, bmax)
    out = []
    for h in range(H):
        R, Rt, G, c = parts[h]
        bh = b[h * dk:(h + 1) * dk]
        fits = np.zeros(dk, dtype=np.int64)
        errs = np.zeros((dk, 16))
        for i in range(dk):
            fits[i], errs[i] = fit_row(np.asarray(Ys[h][i], np.float64), R[i], int(bh[i]))
        out.append({"widths": bh.copy(), "fit": fits, "bstar": bstar[h * dk:(h + 1) * dk],
                    "c": np.maximum(c, C_FLOOR), "R": R, "Rt": Rt, "Gamma": G, "fit_err": errs})
    return out


def allocate_heads(Ys, s_rows, r_rows, bbar=4, bmin=2, bmax=8, factor=GAMMA_ERASURE, C=1, group=32):
    """One width per head for the heads of one sequence's layer ([LBRS] "Allocation
    units": per-head decay and normalisation give each head one width and block scales;
    R~ = 1, so decay alone sets the widths; "at layer-wise mean budget"). Reading: under
    one width the head's proxy cost is sum_i c_i 2^{-2b} with c_i = Gamma_i (R~ = 1), so
    the head's cost is c_h = sum_i Gamma_i (kept in [1e-300, 1e300]); widths by the same
    rule as rows (geometric mean, rounding, clip, one-bit adjustments over the heads, ties
    to the lower head). Then for each scale group (``group`` rows of one column): the
    clipping fit over the 16 fractions at the head's new width, Delta = f16(f R / n) and
    the nearest levels. Returns widths [H], and per head fit / delta [dk/group][dv] and
    kappa [dk][dv]."""
    H = len(Ys)
    c = np.zeros(H)
    for h in range(H):
        with np.errstate(divide="ignore"):
            G = persistence_factor(s_rows[h], r_rows[h], factor, C)
        c[h] = min(float(np.sum(G)), C_CAP)
    bstar = real_widths(c, bbar)
    b = integer_widths(c, bstar, bbar, bmin, bmax)
    fits, deltas, kappas, errs = [], [], [], []
    for h in range(H):
        Y = np.asarray(Ys[h], np.float64)
        dk, dv = Y.shape
        ng = dk // group
        n = levels_n(int(b[h]))
        fk = np.zeros((ng, dv), np.int64)
        dl = np.zeros((ng, dv))
        er = np.zeros((ng, dv, 16))
        for g in range(ng):
            for j in range(dv):
                x = Y[g * group:(g + 1) * group, j]
                R = float(np.max(np.abs(x)))
                fk[g, j], er[g, j] = fit_row(x, R, int(b[h]))
                dl[g, j] = float(f16(fit_fraction(int(fk[g, j])) * R / n))
        kap = np.zeros((dk, dv), np.int64)
        for g in range(ng):
            for j in range(dv):
                x = Y[g * group:(g + 1) * group, j]
                kap[g * group:(g + 1) * group, j] = (np.zeros(group, np.int64) if dl[g, j] == 0.0 else
                                                     np.clip(rne(x / dl[g, j]), -n, n).astype(np.int64))
        fits.append(fk)
        deltas.append(dl)
        kappas.append(kap)
        errs.append(er)
    return {"widths": b, "bstar": bstar, "c": np.maximum(c, C_FLOOR), "fit": fits, "delta": deltas,
            "kappa": kappas, "fit_err": errs}


def default_r(dk: int) -> float:
    """Closed form of r_i for the synthetic stream: beta ~ U(0,1) and unit keys of
    isotropic direction give E[beta (2 - beta)] = 2/3 and E[k_i^2] = 1/dk, so
    r_i = (1/2)(2/3)(1/dk) = 1/(3 dk)."""
    return 1.0 / (3.0 * dk)
