"""One quantized write-back step of one head, and the calls built on it.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

The step follows the write-back operator in its stated order ([WB] "Post-training
write-back interventions and diagnostics": the stored q_{t-1} enters step t, the
recurrence computes h_t, write-back produces q_t for step t+1; [DAMP]
"Implementation": reconstruct, update, re-quantize, write back):

  1. decode the stored region and dequantize it (``layouts``);
  2. undo the storage transforms: Hadamard rows back to the original domain, rows
     back to logical order;
  3. one gated delta-rule step and the readout o_t before quantization
     (``recurrence.delta_step``);
  4. apply the storage transforms to h_t = S_t: rows to physical order, Hadamard
     rows rotated;
  5. compute the metadata from h_t (block min/max, row maxima) and round every
     element under the write-back rule (``quantizers``);
  6. encode the new region.

Cadence: decode writes back every token (C = 1); prefill writes back after every
C-th token of the call and after its last token, and outputs always come from the
unquantized running state ([LBRS] "Accumulated readout error"; [LBRS] "Protocol":
each write-back is quantized and dequantized before reuse).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import layouts as L
from .allocation import allocate_head, allocate_heads, allocate_layer
from .numerics import f16, f16_bits
from .philox import sr_draws
from .quantizers import (DIR, EF, RESQ, SR, affine_metadata, affine_round, levels_n, one_bit_round,
                         one_bit_step, row_step, sym_round, uniform_memory_round, uniform_round,
                         write_activity)
from .recurrence import delta_step


@dataclass
class WriteBack:
    region: np.ndarray             # new region bytes
    e_new: np.ndarray | None       # new residuals [dk][dv] (EF) or None
    X: np.ndarray                  # h_t in the stored domain, physical rows (float64)
    meta_pre: dict = field(default_factory=dict)   # metadata before float16 rounding
    meta: dict = field(default_factory=dict)       # metadata as stored
    tau: np.ndarray | None = None  # grid coordinate per element (rounding rows)
    boundary: np.ndarray | None = None
    activity: np.ndarray | None = None   # UNIFORM: the eight write-activity counts
    votes_new: np.ndarray | None = None  # UNIFORM: per-element vote state after the step


def _draws(lay, b, h, t, rows):
    r = np.zeros((len(rows), lay.dv))
    for n, row in enumerate(rows):
        r[n] = sr_draws(lay.seed, b, h, lay.H, t, int(row), lay.dv)
    return r


def write_back(lay: L.Layout, X: np.ndarray, e_in, t: int, b: int, h: int,
               prev: L.Content | None = None, meta_override: dict | None = None,
               votes_in=None) -> WriteBack:
    """Round stored-domain values X (physical rows) into a new region.

    ``prev`` supplies the BITALLOC widths and fit indices and the UNIFORM levels entering
    the step; ``meta_override`` (tests) replaces the computed metadata so that X can be
    re-rounded with another side's metadata. ``votes_in`` is the UNIFORM vote state of
    the previous step (zeros when absent) for the write-activity counts.
    """
    dk, dv = lay.dk, lay.dv
    X = np.asarray(X, dtype=np.float64)
    mode = lay.mode
    e = np.zeros((dk, dv)) if e_in is None else np.asarray(e_in, dtype=np.float64)
    wb = WriteBack(region=None, e_new=None, X=X)
    tau = np.full((dk, dv), np.nan)
    bnd = np.full((dk, dv), np.inf)
    e_new = e.copy()
    if lay.kind == L.FP32:
        c = L.Content(S32=X.astype(np.float32).astype(np.float64))
        wb.region = L.encode_region(lay, c)
        return wb
    if lay.kind == L.UNIFORM and mode in (DIR, RESQ):
        kp = prev.kappa if prev is not None else np.zeros((dk, dv), np.int64)
        mr = uniform_memory_round(X, lay.bits, mode, kp, e, lay.mem_bits)
        wb.region = L.encode_region(lay, L.Content(kappa=mr.kappa))
        tau, bnd, e_new = mr.tau, mr.boundary, mr.side_new
        wb.activity, wb.votes_new = write_activity(X, kp, mr.kappa, lay.bits, mr.triggers,
                                                   np.zeros((dk, dv)) if votes_in is None else votes_in)
    elif lay.kind == L.UNIFORM:
        r16 = _draws(lay, b, h, t, range(dk)) if mode == SR else None
        rr = uniform_round(X, lay.bits, mode, e, r16)
        wb.region = L.encode_region(lay, L.Content(kappa=rr.kappa))
        tau, bnd, e_new = rr.tau, rr.boundary, rr.e_new
        if prev is not None:
            wb.activity, wb.votes_new = write_activity(X, prev.kappa, rr.kappa, lay.bits, np.zeros((dk, dv), bool),
                                                       np.zeros((dk, dv)) if votes_in is None else votes_in)
    elif lay.kind in (L.HAD_INT8, L.MIXED):
        G = lay.block
        nb = dv // G
        q0 = lay.k_hi if lay.kind == L.MIXED else 0
        nq = dk - q0
        c = L.Content(codes=np.zeros((nq, dv), np.int64), scale_bits=np.zeros((nq, nb), np.uint16),
                      zero_bits=np.zeros((nq, nb), np.uint16))
        scale = np.zeros((nq, nb))
        zero = np.zeros((nq, nb))
        spre = np.zeros((nq, nb))
        zpre = np.zeros((nq, nb))
        for p in range(nq):
            for g in range(nb):
                blk = X[q0 + p, g * G:(g + 1) * G]
                scale[p, g], zero[p, g], spre[p, g], zpre[p, g] = affine_metadata(blk, lay.int_bits)
        if meta_override is not None:
            scale, zero = meta_override["scale"], meta_override["zero"]
        r16 = _draws(lay, b, h, t, range(q0, dk)) if mode == SR else None
        rr = affine_round(X[q0:], np.repeat(scale, G, axis=1), np.repeat(zero, G, axis=1),
                          mode, e[q0:], r16, lay.int_bits)
        c.codes = rr.kappa
        c.scale_bits = f16_bits(scale)
        c.zero_bits = f16_bits(zero)
        tau[q0:], bnd[q0:], e_new[q0:] = rr.tau, rr.boundary, rr.e_new
        if lay.kind == L.MIXED:
            hi = X[:q0]
            c.hi_bits = f16_bits(hi)
            # float16 rows round to nearest; one "step" is one float16 spacing, and
            # the boundary is the midpoint between the two float16 values around |x|
            a = np.abs(hi)
            r = a.astype(np.float16)
            rv = r.astype(np.float64)
            lower = np.where(rv <= a, rv, np.nextafter(r, np.float16(0)).astype(np.float64))
            upper = np.where(rv >= a, rv, np.nextafter(r, np.float16(np.inf)).astype(np.float64))
            span = upper - lower
            tau[:q0] = np.where(span > 0, hi / np.where(span > 0, span, 1.0), 0.0)
            bnd[:q0] = np.where(span > 0, np.abs(a - 0.5 * (lower + upper))
                                / np.where(span > 0, span, 1.0), np.inf)
        wb.meta_pre = {"scale": spre, "zero": zpre}
        wb.meta = {"scale": scale, "zero": zero}
        wb.region = L.encode_region(lay, c)
    elif lay.kind == L.BITALLOC:
        widths, fits = prev.widths, prev.fit
        R = np.max(np.abs(X), axis=1)
        delta = np.zeros(dk)
        dpre = np.zeros(dk)
        for i in range(dk):
            if widths[i] == 1:
                delta[i], dpre[i] = one_bit_step(X[i])
            else:
                delta[i], dpre[i] = row_step(R[i], int(widths[i]), int(fits[i]))
        if meta_override is not None:
            delta = meta_override["delta"]
        r16 = _draws(lay, b, h, t, range(dk)) if mode == SR else None
        kappa = np.zeros((dk, dv), np.int64)
        for i in range(dk):
            n = levels_n(int(widths[i]))
            ri = None if r16 is None else r16[i]
            rr = (one_bit_round(X[i], delta[i], mode, e[i], ri) if widths[i] == 1 else
                  sym_round(X[i], delta[i], n, mode, e[i], ri))
            kappa[i], tau[i], bnd[i], e_new[i] = rr.kappa, rr.tau, rr.boundary, rr.e_new
        c = L.Content(kappa=kappa, widths=widths, fit=fits, delta_bits=f16_bits(delta))
        wb.meta_pre = {"delta": dpre, "R": R}
        wb.meta = {"delta": delta}
        wb.region = L.encode_region(lay, c)
    elif lay.kind == L.HEADALLOC:
        # the head's width and each group's fit index stay; Delta of a group (32 rows
        # of one column) from its maximum
        bw, fits = int(prev.width), prev.fit
        G = L.HA_GROUP
        ng = dk // G
        n = levels_n(bw)
        Rg = np.max(np.abs(X.reshape(ng, G, dv)), axis=1)
        delta = np.zeros((ng, dv))
        dpre = np.zeros((ng, dv))
        for g in range(ng):
            for j in range(dv):
                delta[g, j], dpre[g, j] = row_step(Rg[g, j], bw, int(fits[g, j]))
        if meta_override is not None:
            delta = meta_override["delta"]
        r16 = _draws(lay, b, h, t, range(dk)) if mode == SR else None
        rr = sym_round(X, np.repeat(delta, G, axis=0), n, mode, e, r16)
        kappa, tau, bnd, e_new = rr.kappa, rr.tau, rr.boundary, rr.e_new
        c = L.Content(kappa=kappa, width=bw, fit=fits, delta_bits=f16_bits(delta))
        wb.meta_pre = {"delta": dpre, "R": Rg}
        wb.meta = {"delta": delta}
        wb.region = L.encode_region(lay, c)
    else:
        raise ValueError(lay.kind)
    wb.tau, wb.boundary = tau, bnd
    if mode in (EF, DIR, RESQ):
        if lay.kind == L.MIXED:
            e_new[: lay.k_hi] = e[: lay.k_hi]          # float16 rows carry no residual
        wb.e_new = e_new
    return wb


@dataclass
class StepResult:
    wb: WriteBack
    o: np.ndarray          # readout [dv]
    S_prev: np.ndarray     # dequantized input state, logical order
    S_new: np.ndarray      # h_t, logical order


def decode_step(lay: L.Layout, region, e_in, q, k, v, beta, s, t: int, b: int, h: int,
                perm=None, votes_in=None) -> StepResult:
    """One decode token for head (b, h), starting from the given stored region (and, for
    the UNIFORM write-activity counts, the previous step's vote state)."""
    content = L.decode_region(lay, region)
    Y = L.stored_values(lay, content)
    S = L.to_logical(lay, Y, perm)
    S_new, o = delta_step(S, q, k, v, beta, s)
    X = L.to_stored(lay, S_new, perm)
    wb = write_back(lay, X, e_in, t, b, h, prev=content, votes_in=votes_in)
    return StepResult(wb=wb, o=o, S_prev=S, S_new=S_new)


def export_state(lay: L.Layout, region, perm=None) -> np.ndarray:
    """Stored region -> state in the original domain and logical row order."""
    content = L.decode_region(lay, region)
    return L.to_logical(lay, L.stored_values(lay, content), perm)


def import_state(lay: L.Layout, S, region_prev, perm=None, b=0, h=0) -> np.ndarray:
    """One round-to-nearest write-back of a given state (BITALLOC keeps the widths
    and fit indices of ``region_prev``)."""
    rtn = L.Layout(**{**lay.__dict__, "mode": "rtn"})
    content = L.decode_region(lay, region_prev)
    X = L.to_stored(lay, S, perm)
    return write_back(rtn, X, None, 0, b, h, prev=content).region


def allocate_region(lay: L.Layout, region, s_rows, r_rows, factor="erasure", C=1):
    """The allocation pass on one BITALLOC head: new widths and fit indices from the
    stored state, then the stored values re-rounded (nearest) at the new widths."""
    content = L.decode_region(lay, region)
    Y = L.stored_values(lay, content)
    return _allocate_and_round(lay, Y, s_rows, r_rows, factor, C)


def allocate_layer_regions(lay: L.Layout, regions, s_rows, r_rows, factor="erasure", C=1):
    """The allocation pass over the H heads of one sequence under the layer-wise budget
    (``lay.budget == "layer"``): widths from the stored states of all heads, then each
    head's stored values re-rounded (nearest) at its new widths."""
    Ys = [L.stored_values(lay, L.decode_region(lay, reg)) for reg in regions]
    allocs = allocate_layer(Ys, s_rows, r_rows, lay.bbar, lay.bmin, lay.bmax, factor, C)
    return [_round_at(lay, Ys[h], allocs[h]) for h in range(len(regions))], allocs


def allocate_headalloc_regions(lay: L.Layout, regions, s_rows, r_rows, factor="erasure", C=1):
    """The allocation pass over the H heads of one sequence for the per-head unit
    (HEADALLOC): one width per head from decay alone, clipping fits per scale group at
    the new width, the stored values re-rounded (nearest)."""
    Ys = [L.stored_values(lay, L.decode_region(lay, reg)) for reg in regions]
    al = allocate_heads(Ys, s_rows, r_rows, lay.bbar, lay.bmin, lay.bmax, factor, C, L.HA_GROUP)
    out = []
    for h, Y in enumerate(Ys):
        c = L.Content(kappa=al["kappa"][h], width=int(al["widths"][h]), fit=al["fit"][h],
                      delta_bits=f16_bits(al["delta"][h]))
        out.append(L.encode_region(lay, c))
    return out, al


def decode_step_alloc(lay: L.Layout, region, q, k, v, beta, s, s_rows, r_rows, factor="erasure", C=1,
                      t: int = 0, b: int = 0, h: int = 0):
    """One decode token for a BITALLOC head whose write-back allocates ([LBRS] "State
    bit allocation": widths are chosen at each write-back): the step from the stored
    state, then widths, fits and Delta chosen for the updated state itself and the
    state rounded once onto that grid, by the layout's rule (RTN; SR with the draws of
    token t of head (b, h)). ``s_rows`` / ``r_rows`` feed the allocation (None: no
    decay estimate). Returns (region, alloc, o, S_new)."""
    content = L.decode_region(lay, region)
    Y = L.stored_values(lay, content)
    S_new, o = delta_step(Y, q, k, v, beta, s)
    alloc = allocate_head(S_new, s_rows, r_rows, lay.bbar, lay.bmin, lay.bmax, factor, C)
    return _round_at(lay, S_new, alloc, lay.mode, t, b, h), alloc, o, S_new


def decode_step_alloc_layer(lay: L.Layout, regions, q, k, v, beta, s, s_rows, r_rows, factor="erasure", C=1,
                            t: int = 0, b: int = 0):
    """One decode token for the H heads of one sequence under the layer-wise budget
    ([LBRS] "State bit allocation": widths at each write-back, "at layer-wise mean
    budget bbar"): each head's step from its stored state, then the widths over every
    row of the H updated states (``allocate_layer``), and each head rounded once at its
    widths by the layout's rule. Per-head inputs are indexed [h]; ``s_rows`` /
    ``r_rows`` [H][dk] or None. Returns (regions, allocs, outputs, updated states)."""
    Ss, outs = [], []
    for h, reg in enumerate(regions):
        Y = L.stored_values(lay, L.decode_region(lay, reg))
        S_new, o = delta_step(Y, q[h], k[h], v[h], beta[h], s[h])
        Ss.append(S_new)
        outs.append(o)
    allocs = allocate_layer(Ss, s_rows, r_rows, lay.bbar, lay.bmin, lay.bmax, factor, C)
    regs = [_round_at(lay, Ss[h], allocs[h], lay.mode, t, b, h) for h in range(len(regions))]
    return regs, allocs, outs, Ss


def _allocate_and_round(lay: L.Layout, Y, s_rows, r_rows, factor, C):
    alloc = allocate_head(Y, s_rows, r_rows, lay.bbar, lay.bmin, lay.bmax, factor, C)
    return _round_at(lay, Y, alloc), alloc


def _round_at(lay: L.Layout, Y, alloc, mode: str = "rtn", t: int = 0, b: int = 0, h: int = 0):
    """Round Y at the allocation's widths and fits by ``mode`` (SR: the draws of token
    t, head (b, h)). The allocation pass alone re-rounds to nearest; a decode write-back
    that allocates uses the layout's rule."""
    widths, fits = alloc["widths"], alloc["fit"]
    delta = np.zeros(lay.dk)
    kappa = np.zeros((lay.dk, lay.dv), np.int64)
    for i in range(lay.dk):
        r16 = _draws(lay, b, h, t, [i])[0] if mode == "sr" else None
        if widths[i] == 1:
            delta[i], _ = one_bit_step(Y[i])
            kappa[i] = one_bit_round(Y[i], delta[i], mode, r16=r16).kappa
            continue
        delta[i], _ = row_step(alloc["R"][i], int(widths[i]), int(fits[i]))
        n = levels_n(int(widths[i]))
        rr = sym_round(Y[i], delta[i], n, mode, r16=r16)
        kappa[i] = rr.kappa
    c = L.Content(kappa=kappa, widths=widths, fit=fits, delta_bits=f16_bits(delta))
    return L.encode_region(lay, c)


def prefill(lay: L.Layout, region, e_in, q, k, v, beta, s, t0: int, C: int, b: int, h: int,
            perm=None, return_last=False, records=None):
    """Token-by-token prefill of one head with write-back after every C-th token of
    the call and after the last one. q, k, v, beta, s are per-token arrays for this
    head ([T][d], [T], [T][dk] or [T]). Returns (region, e, outputs [T][dv]) and, with
    ``return_last``, the record of the last write-back (its pre-rounding values);
    ``records`` (a list) receives (token index, record) of every write-back."""
    T = len(beta)
    content = L.decode_region(lay, region)
    S = L.to_logical(lay, L.stored_values(lay, content), perm)
    e = e_in
    outs = np.zeros((T, lay.dv))
    wb = None
    for i in range(T):
        S, outs[i] = delta_step(S, q[i], k[i], v[i], beta[i], s[i])
        if (i + 1) % C == 0 or i == T - 1:
            X = L.to_stored(lay, S, perm)
            wb = write_back(lay, X, e, t0 + i, b, h, prev=content)
            if records is not None:
                records.append((i, wb))
            region = wb.region
            e = wb.e_new
            content = L.decode_region(lay, region)
            S = L.to_logical(lay, L.stored_values(lay, content), perm)
    if return_last:
        return region, e, outs, wb
    return region, e, outs
