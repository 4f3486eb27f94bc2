"""Teacher-forced comparison of one GPU write-back step against the oracle.

Protocol (the tolerances are those fixed for the decode write-back step):
  1. The oracle starts from the GPU's stored bytes before the step (decoded by the
     oracle's own reader) and the GPU's residuals, and runs one float64 step on the same
     inputs.
  2. Metadata first: every float16 scale, zero point and row step must equal the
     oracle's, except that the adjacent float16 value is accepted where the oracle's
     float64 pre-rounding value lies within 1e-6 (relative) of the midpoint between the
     two. BITALLOC widths and fit indices must be unchanged by a decode step.
  3. Codes, given the GPU's accepted metadata: the oracle re-rounds its float64
     pre-rounding values on the GPU's grid. Codes must be bit-equal, except that at most
     a 1e-4 fraction of the elements may differ by exactly one step, and only where the
     oracle's pre-rounding value lies within 1e-5 of a step of the rounding boundary
     (for float16 rows the step is the float16 spacing at the value).
  4. Outputs: relative L2 error of o per head <= 1e-4.
Error-feedback residuals are compared where the codes agree, within the rounding of
the GPU's arithmetic (float32 storage of the residual; float32 values for the float32
layouts).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from oracle import layouts as L
from oracle.numerics import f16_value
from oracle.step import decode_step, write_back

WINDOW = 1e-5
MAX_FRAC = 1e-4
META_REL = 1e-6
O_REL = 1e-4


@dataclass
class Tally:
    elems: int = 0
    mismatch: int = 0
    bad: list = field(default_factory=list)
    meta_blocks: int = 0
    meta_adjacent: int = 0
    o_worst: float = 0.0
    o_num: float = 0.0
    o_den: float = 0.0
    e_worst: float = 0.0

    def ok(self):
        return (not self.bad and self.mismatch <= MAX_FRAC * max(self.elems, 1)
                and self.o_worst <= O_REL)

    def summary(self):
        return (f"elems={self.elems} mismatch={self.mismatch} ({self.mismatch / max(self.elems, 1):.2e}) "
                f"bad={len(self.bad)} meta_adjacent={self.meta_adjacent}/{self.meta_blocks} "
                f"o_worst={self.o_worst:.2e} e_worst={self.e_worst:.2e} first_bad={self.bad[:3]}")


def _adjacent_f16(a_bits, b_bits):
    a = np.asarray(a_bits, np.uint16).view(np.float16)
    b = np.asarray(b_bits, np.uint16).view(np.float16)
    return (np.nextafter(a, b) == b) | (a == b)


def _meta_ok(gpu_bits, orc_bits, pre, tally, what, meta_rel=META_REL):
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    orc_bits = np.asarray(orc_bits, np.uint16)
    tally.meta_blocks += gpu_bits.size
    diff = gpu_bits != orc_bits
    if not diff.any():
        return
    gv = f16_value(gpu_bits[diff])
    ov = f16_value(orc_bits[diff])
    mid = 0.5 * (gv + ov)
    pre_d = np.asarray(pre)[diff]
    adj = _adjacent_f16(gpu_bits[diff], orc_bits[diff])
    near = np.abs(pre_d - mid) <= meta_rel * np.maximum(np.abs(mid), 1e-300)
    good = adj & near
    tally.meta_adjacent += int(good.sum())
    if not good.all():
        idx = np.argwhere(diff)[~good][:3]
        tally.bad.append((what, "metadata", idx.tolist(), gv[~good][:3].tolist(), ov[~good][:3].tolist(),
                          pre_d[~good][:3].tolist()))


def check_head(lay: L.Layout, reg_in, reg_gpu, e_in, e_gpu, o_gpu, q, k, v, beta, s, t, b, h, perm,
               tally: Tally):
    """Compare one head's GPU step against the oracle; accumulate into ``tally``."""
    reg_in = np.asarray(reg_in, np.uint8)[: lay.region_size()]
    reg_gpu = np.asarray(reg_gpu, np.uint8)[: lay.region_size()]
    r = decode_step(lay, reg_in, e_in, q, k, v, beta, s, t, b, h, perm)
    o = np.asarray(o_gpu, np.float64)
    den = np.linalg.norm(r.o)
    rel = np.linalg.norm(o - r.o) / max(den, 1e-30)
    tally.o_worst = max(tally.o_worst, rel)
    tally.o_num += float(np.sum((o - r.o) ** 2))
    tally.o_den += float(den ** 2)
    compare_write_back(lay, reg_in, reg_gpu, r.wb, e_in, e_gpu, t, b, h, tally)
    return r


def compare_write_back(lay: L.Layout, reg_in, reg_gpu, wb, e_in, e_gpu, t, b, h, tally: Tally,
                       window=WINDOW, meta_rel=META_REL, fp32_rel=4 * 2.0 ** -24, abs_rel=None):
    """Compare a GPU-written region with the oracle's write-back record ``wb`` of the
    same pre-rounding values (metadata first, then codes on the GPU's grid).

    With ``abs_rel`` (GPU paths whose arithmetic error is bounded relative to the row's
    magnitude rather than to the value), a differing code is accepted when the GPU's
    stored value lies within half a step plus abs_rel * max|row| of the oracle's value;
    otherwise the boundary window (in steps) applies."""
    reg_in = np.asarray(reg_in, np.uint8)[: lay.region_size()]
    reg_gpu = np.asarray(reg_gpu, np.uint8)[: lay.region_size()]
    where = (b, h, t)
    cin = L.decode_region(lay, reg_in)
    g = L.decode_region(lay, reg_gpu)
    X = wb.X
    if lay.kind == L.FP32:
        err = np.abs(g.S32 - X)
        tol = fp32_rel * (np.abs(X) + np.max(np.abs(X)))
        tally.elems += X.size
        if np.any(err > tol):
            i = np.unravel_index(np.argmax(err - tol), err.shape)
            tally.bad.append((where, "fp32 value", i, g.S32[i], X[i]))
        return
    override = None
    owb = L.decode_region(lay, wb.region)
    if lay.kind in (L.HAD_INT8, L.MIXED):
        _meta_ok(g.scale_bits, owb.scale_bits, wb.meta_pre["scale"], tally, (where, "scale"), meta_rel)
        _meta_ok(g.zero_bits, owb.zero_bits, wb.meta_pre["zero"], tally, (where, "zero"), meta_rel)
        override = {"scale": g.scale, "zero": g.zero}
    elif lay.kind == L.BITALLOC:
        if not (np.array_equal(g.widths, cin.widths) and np.array_equal(g.fit, cin.fit)):
            tally.bad.append((where, "widths/fit changed by a decode step"))
        _meta_ok(g.delta_bits, owb.delta_bits, wb.meta_pre["delta"], tally, (where, "delta"), meta_rel)
        override = {"delta": g.delta}
    elif lay.kind == L.HEADALLOC:
        if not (g.width == cin.width and np.array_equal(g.fit, cin.fit)):
            tally.bad.append((where, "width/fit changed by a decode step"))
        _meta_ok(g.delta_bits, owb.delta_bits, wb.meta_pre["delta"], tally, (where, "delta"), meta_rel)
        override = {"delta": g.delta}
    wb2 = write_back(lay, X, e_in, t, b, h, prev=cin, meta_override=override)
    req = L.decode_region(lay, wb2.region)
    if lay.kind == L.UNIFORM:
        gc, oc = g.kappa, req.kappa
        step = np.full(X.shape, 2.0 ** (1 - lay.bits))
    elif lay.kind == L.BITALLOC:
        gc, oc = g.kappa, req.kappa
        step = np.repeat(g.delta[:, None], lay.dv, axis=1)
    elif lay.kind == L.HEADALLOC:
        gc, oc = g.kappa, req.kappa
        step = np.repeat(g.delta, L.HA_GROUP, axis=0)
    else:
        q0 = lay.dk - lay.int8_rows
        gc = np.zeros(X.shape, np.int64)
        oc = np.zeros(X.shape, np.int64)
        gc[q0:], oc[q0:] = g.codes, req.codes
        if lay.kind == L.MIXED:
            # float16 rows: codes are the bit patterns; adjacency by one float16 step
            gc[:q0], oc[:q0] = g.hi_bits.astype(np.int64), req.hi_bits.astype(np.int64)
        step = np.zeros(X.shape)
        step[q0:] = np.repeat(g.scale, lay.block, axis=1)
        if lay.kind == L.MIXED:
            step[:q0] = 1.0
    tally.elems += X.size
    diff = gc != oc
    if diff.any():
        d = np.abs(gc - oc)
        if lay.kind == L.MIXED:
            q0 = lay.dk - lay.int8_rows
            adj = np.zeros(X.shape, bool)
            adj[:q0] = _adjacent_f16(g.hi_bits, req.hi_bits)
            adj[q0:] = d[q0:] == 1
        else:
            adj = d == 1
        if abs_rel is None:
            near = wb2.boundary <= window
            ok = ~diff | (adj & near)
        else:
            gv = L.stored_values(lay, g)
            rowmax = np.max(np.abs(X), axis=1, keepdims=True)
            if lay.kind == L.MIXED:
                q0 = lay.dk - lay.int8_rows
                a = np.abs(X[:q0])
                r = a.astype(np.float16)
                lower = np.where(r.astype(np.float64) <= a, r.astype(np.float64),
                                 np.nextafter(r, np.float16(0)).astype(np.float64))
                upper = np.where(r.astype(np.float64) >= a, r.astype(np.float64),
                                 np.nextafter(r, np.float16(np.inf)).astype(np.float64))
                step = step.copy()
                step[:q0] = np.maximum(upper - lower, 2.0 ** -24)
            ok = ~diff | (np.abs(gv - X) <= 0.5 * step * (1 + 1e-9) + abs_rel * rowmax)
        tally.mismatch += int(diff.sum())
        if not ok.all():
            idx = np.argwhere(~ok)[:3]
            tally.bad.append((where, "codes", idx.tolist(), gc[~ok][:3].tolist(), oc[~ok][:3].tolist(),
                              wb2.boundary[~ok][:3].tolist(), wb2.tau[~ok][:3].tolist()))
    if lay.mode in ("dir", "resq"):
        # direction counters / k-bit residual values: exact, except where a decision
        # (level, vote band edge, residual level) is within the window
        eg = np.asarray(e_gpu, np.float64)
        eo = wb2.e_new
        near_any = wb2.boundary <= window
        off = (eg != eo) & ~near_any
        tally.e_worst = max(tally.e_worst, float(np.max(np.where(near_any, 0.0, np.abs(eg - eo)))))
        if off.any():
            i = np.unravel_index(np.argmax(off), off.shape)
            tally.bad.append((where, "memory state", i, eg[i], eo[i], wb2.boundary[i]))
    if lay.mode == "ef":
        eg = np.asarray(e_gpu, np.float64)
        eo = wb2.e_new
        same = ~diff
        if lay.kind == L.MIXED:
            same[: lay.dk - lay.int8_rows] = False
        if lay.kind in (L.HAD_INT8, L.MIXED):
            tol = 2.0 ** -22 * np.abs(eo) + 1e-9 * step
        else:
            # float32 update: x carries a few ulps of its largest term (bounded by the
            # row maximum), and the residual inherits that error
            rowmax = np.max(np.abs(X), axis=1, keepdims=True)
            tol = 1e-6 * (rowmax + np.abs(np.asarray(e_in))) + 1e-7 * step
        err = np.where(same, np.abs(eg - eo) - tol, -np.inf)
        tally.e_worst = max(tally.e_worst, float(np.max(np.where(same, np.abs(eg - eo), 0))))
        if np.any(err > 0):
            i = np.unravel_index(np.argmax(err), err.shape)
            tally.bad.append((where, "residual", i, eg[i], eo[i]))


def compare_alloc_write_back(lay: L.Layout, reg_gpu, reg_orc, alloc, X, tally: Tally, where,
                             window=WINDOW, meta_rel=META_REL, draws=None, layer=False):
    """Compare a write-back that allocated (BITALLOC) with the oracle's on the same
    updated state X. Widths: equal, or an allocation of the same budget whose proxy
    cost under the oracle's costs is within 1e-6 of the oracle's (the float32 state
    moves near-tied costs; ``layer``: the budget and the cost are the sequence's, which
    the caller checks with ``compare_layer_widths``). Rows of equal width: fit indices
    equal or of equal squared error within 1e-6; rows of equal width and fit: Delta
    equal or the adjacent float16 where the pre-rounding value is within ``meta_rel``
    of the midpoint; rows of equal width, fit and Delta: codes equal or one apart within
    ``window`` steps of a rounding boundary (``draws``: row -> 16-bit draws, for
    stochastic rounding, whose boundary is the draw). Returns the number of rows left
    out of the code comparison."""
    from oracle.quantizers import fit_fraction, levels_n, one_bit_round, sym_round
    g = L.decode_region(lay, np.asarray(reg_gpu, np.uint8)[: lay.region_size()])
    o = L.decode_region(lay, np.asarray(reg_orc, np.uint8)[: lay.region_size()])
    if ((not layer and g.widths.sum() != lay.bbar * lay.dk) or g.widths.min() < lay.bmin or
            g.widths.max() > lay.bmax):
        tally.bad.append((where, "width budget", int(g.widths.sum())))
        return lay.dk
    c = alloc["c"]
    same_w = g.widths == o.widths
    if not same_w.all() and not layer:
        cg = float(np.sum(c * 2.0 ** (-2.0 * g.widths)))
        co = float(np.sum(c * 2.0 ** (-2.0 * o.widths)))
        if cg > co * (1 + 1e-6) or (~same_w).sum() > 8:
            tally.bad.append((where, "widths", np.argwhere(~same_w).ravel()[:6].tolist(), cg, co))
    same_f = same_w & (g.fit == o.fit)
    for i in np.argwhere(same_w & ~same_f).ravel():
        e = alloc["fit_err"][i]
        if abs(e[g.fit[i]] - e[o.fit[i]]) > 1e-6 * max(e[o.fit[i]], 1e-300):
            tally.bad.append((where, "fit", int(i), int(g.fit[i]), int(o.fit[i])))
    rows = np.argwhere(same_f).ravel()
    pre = np.array([float(np.mean(np.abs(X[i]))) if o.widths[i] == 1 else
                    fit_fraction(int(o.fit[i])) * alloc["R"][i] / levels_n(int(o.widths[i])) for i in rows])
    _meta_ok(g.delta_bits[rows], o.delta_bits[rows], pre, tally, (where, "delta"), meta_rel)
    skipped = lay.dk - rows.size
    for i in rows:
        if g.delta_bits[i] != o.delta_bits[i]:
            skipped += 1
            continue
        n = levels_n(int(g.widths[i]))
        mode, r16 = ("rtn", None) if draws is None else ("sr", draws(i))
        rr = (one_bit_round(X[i], float(g.delta[i]), mode, r16=r16) if g.widths[i] == 1 else
              sym_round(X[i], float(g.delta[i]), n, mode, r16=r16))
        tally.elems += lay.dv
        diff = g.kappa[i] != rr.kappa
        if diff.any():
            tally.mismatch += int(diff.sum())
            ok = ~diff | ((np.abs(g.kappa[i] - rr.kappa) == 1) & (rr.boundary <= window))
            if not ok.all():
                j = np.argwhere(~ok).ravel()[:3]
                tally.bad.append((where, "codes", int(i), j.tolist(), g.kappa[i][j].tolist(), rr.kappa[j].tolist()))
    return skipped


def compare_layer_widths(lay: L.Layout, regs_gpu, allocs, tally: Tally, where):
    """The widths of one sequence's heads after a layer-budget allocation: the sum over
    the H heads is bbar H dk, and where they differ from the oracle's the allocation's
    proxy cost under the oracle's costs is within 1e-6 of the oracle's, on at most 8
    rows (the float32 state moves near-tied costs)."""
    gw = np.concatenate([L.decode_region(lay, np.asarray(r, np.uint8)[: lay.region_size()]).widths for r in regs_gpu])
    ow = np.concatenate([a["widths"] for a in allocs])
    c = np.concatenate([a["c"] for a in allocs])
    if gw.sum() != lay.bbar * lay.dk * len(allocs):
        tally.bad.append((where, "layer width budget", int(gw.sum())))
        return
    if not np.array_equal(gw, ow):
        cg = float(np.sum(c * 2.0 ** (-2.0 * gw)))
        co = float(np.sum(c * 2.0 ** (-2.0 * ow)))
        if cg > co * (1 + 1e-6) or int(np.sum(gw != ow)) > 8:
            tally.bad.append((where, "layer widths", np.argwhere(gw != ow).ravel()[:6].tolist(), cg, co))


def check_heads_chunk(args):
    """Worker of the full-layer comparison: check heads [lo, hi) of one teacher-forced
    step from arrays saved by the caller (numpy only, so that it runs in a spawned
    process). Returns the chunk's tally."""
    import os
    (d, lay_kw, lo, hi, t) = args
    lay = L.Layout(**lay_kw)
    ld = lambda n: np.load(os.path.join(d, n + ".npy"), mmap_mode="r")
    reg_in, reg_out, o = ld("reg_in"), ld("reg_out"), ld("o")
    q, k, v, beta, s = ld("q"), ld("k"), ld("v"), ld("beta"), ld("s")
    perm = ld("perm") if os.path.exists(os.path.join(d, "perm.npy")) else None
    # error-feedback residuals before and after the step, when the caller saved them
    e_in = ld("e_in") if os.path.exists(os.path.join(d, "e_in.npy")) else None
    e_out = ld("e_out") if os.path.exists(os.path.join(d, "e_out.npy")) else None
    H = lay.H
    tally = Tally()
    for idx in range(lo, hi):
        b, h = divmod(idx, H)
        check_head(lay, reg_in[idx], reg_out[idx], None if e_in is None else np.asarray(e_in[b, h]),
                   None if e_out is None else np.asarray(e_out[b, h]), o[b, h], q[b, h], k[b, h], v[b, h],
                   beta[b, h], s[b, h], t, b, h, None if perm is None else perm[h], tally)
    return tally
