"""Byte layouts of one stored head state, encoded and decoded in plain numpy.

TEST INFRASTRUCTURE (see ``oracle/__init__``). This is the oracle's own reader and
writer of the storage format; it shares no code with the C++/HIP side.

One head state (dk x dv, row i = key channel i) occupies one *region*; regions are
stored for (b, h) in order b*H + h, each padded to a multiple of 256 bytes. All
multi-byte fields are little-endian.

FP32      identity write-back: float32 [dk][dv], logical row order.
UNIFORM   B-bit two's-complement level index kappa of element (i, j) at bit offset
          B*(i*dv + j), least-significant bit first; value kappa * 2^(1-B)
          ([WB-zh] "Core method": Delta_4 = 0.125 on [-1, 1]).
HAD_INT8  every row Hadamard-rotated along the value axis ([DAMP] "Quantization &
          calibration details"): u8 codes [dk][dv], then for each row and each
          block of G consecutive values one (f16 scale, f16 zero) pair [dk][dv/G][2].
MIXED     static mixed precision ([DAMP] "Risk scoring and selection",
          "Implementation"; [LBRS] "Related work" counts 9.875 bits): physical row p
          holds logical row perm[p]; physical rows 0..k_hi-1 are float16 values
          [k_hi][dv] (unrotated); the remaining rows are Hadamard INT8 as above:
          u8 codes [dk-k_hi][dv], then (f16 scale, f16 zero) [dk-k_hi][dv/G][2].
          With the INT4 tier (int_bits = 4; [DAMP] "Quantization & calibration details"
          gives b = 4 beside b = 8) the codes are 4 bits, two a byte, low nibble first,
          and the affine grid has 15 steps.
BITALLOC  decay-aware per-row widths ([LBRS] "State bit allocation", "Levels and
          storage": prefix sums of widths give row offsets): row i's codes start at
          byte (dv/8) * sum_{i'<i} b_i', element j at bits [j b_i, (j+1) b_i),
          stored as kappa + n_i; the code area holds dk*dv*b_cap/8 bytes, b_cap = bbar
          when the budget is per head (the area is exactly full) and b_cap = bmax when
          the budget is per layer (a head's widths may sum to anything up to bmax*dk;
          the bytes after its last row are zero); then f16 Delta [dk]; then u8 meta
          [dk] = (b_i - 1) | (k_i << 4), k_i the clipping-fit index.
HEADALLOC per-head widths with block scales ([LBRS] "Allocation units": for per-head
          decay and normalisation one width per head and a scale per block of 32 key
          channels; "Levels and storage"): element (i, j) at bits [(i dv + j) b, +b)
          as kappa + n, n = 2^(b-1) - 1, in a code area of dk*dv*bmax/8 bytes (zero after
          the last element); then f16 Delta [dk/32][dv] (one per 32 rows of a column);
          then u8 clipping-fit index [dk/32][dv]; then u8 (b - 1) and 15 zero bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .hadamard import sylvester
from .numerics import f16_bits, f16_value, pack_fields, unpack_fields

FP32, UNIFORM, HAD_INT8, MIXED, BITALLOC, HEADALLOC = "fp32", "uniform", "had_int8", "mixed", "bitalloc", "headalloc"
KINDS = (FP32, UNIFORM, HAD_INT8, MIXED, BITALLOC, HEADALLOC)
HA_GROUP = 32              # HEADALLOC: key channels (rows) per scale group


@dataclass
class Layout:
    kind: str
    B: int
    H: int
    dk: int
    dv: int
    per_row_decay: bool = True
    bits: int = 4          # UNIFORM level width
    block: int = 32        # affine block length G along the value axis
    k_hi: int = 16         # MIXED: protected float16 rows per head
    bbar: int = 4          # BITALLOC mean width
    bmin: int = 2
    bmax: int = 8
    mode: str = "rtn"
    seed: int = 0
    mem_bits: int = 0      # k of the temporal-memory rules (direction / residual memory)
    budget: str = "head"   # BITALLOC width budget: "head" or "layer" (all heads of a sequence)
    int_bits: int = 8      # HAD_INT8 / MIXED integer tier: 8 (INT8) or 4 (INT4, two codes a byte)
    extra: dict = field(default_factory=dict)

    @property
    def int8_rows(self) -> int:
        return self.dk - self.k_hi if self.kind == MIXED else self.dk

    @property
    def code_capacity(self) -> int:
        """BITALLOC / HEADALLOC code-area bytes of one head."""
        if self.kind == HEADALLOC:
            return self.dk * self.dv * self.bmax // 8
        return self.dk * self.dv * (self.bmax if self.budget == "layer" else self.bbar) // 8

    def region_size(self) -> int:
        dk, dv = self.dk, self.dv
        if self.kind == FP32:
            return 4 * dk * dv
        if self.kind == UNIFORM:
            return dk * dv * self.bits // 8
        if self.kind == HAD_INT8:
            return dk * dv * self.int_bits // 8 + dk * (dv // self.block) * 4
        if self.kind == MIXED:
            q = dk - self.k_hi
            return self.k_hi * dv * 2 + q * dv * self.int_bits // 8 + q * (dv // self.block) * 4
        if self.kind == BITALLOC:
            return self.code_capacity + 2 * dk + dk
        if self.kind == HEADALLOC:
            ng = dk // HA_GROUP
            return self.code_capacity + 3 * ng * dv + 16
        raise ValueError(self.kind)

    def region_stride(self) -> int:
        return (self.region_size() + 255) // 256 * 256

    def side_elems(self) -> int:
        """Auxiliary write-back values per head: the error-feedback residual (EF on a
        rounding layout), the k-bit residual (residual memory) or the direction counter
        (direction memory), one per element; 0 otherwise."""
        if self.mode not in ("ef", "dir", "resq") or self.kind == FP32:
            return 0
        return self.dk * self.dv


# ---------------------------------------------------------------------------
# Decoded content of one region

@dataclass
class Content:
    S32: np.ndarray | None = None        # FP32 values
    kappa: np.ndarray | None = None      # UNIFORM / BITALLOC signed levels [rows][dv]
    codes: np.ndarray | None = None      # affine u8 codes [int8 rows][dv]
    scale: np.ndarray | None = None      # affine f16 scale values [rows][nb]
    zero: np.ndarray | None = None       # affine f16 zero values [rows][nb]
    scale_bits: np.ndarray | None = None
    zero_bits: np.ndarray | None = None
    hi_bits: np.ndarray | None = None    # MIXED float16 rows, bit patterns [k_hi][dv]
    widths: np.ndarray | None = None     # BITALLOC b_i
    fit: np.ndarray | None = None        # BITALLOC k_i
    delta: np.ndarray | None = None      # BITALLOC f16 Delta values
    width: int | None = None             # HEADALLOC b of the head
    delta_bits: np.ndarray | None = None


def decode_region(lay: Layout, region: np.ndarray) -> Content:
    r = np.asarray(region, dtype=np.uint8)
    dk, dv = lay.dk, lay.dv
    if lay.kind == FP32:
        return Content(S32=r[: 4 * dk * dv].view(np.float32).reshape(dk, dv).astype(np.float64))
    if lay.kind == UNIFORM:
        B = lay.bits
        u = unpack_fields(r, B, dk * dv).reshape(dk, dv)
        kappa = np.where(u >= 2 ** (B - 1), u - 2 ** B, u)
        return Content(kappa=kappa)
    if lay.kind in (HAD_INT8, MIXED):
        off = 0
        c = Content()
        nq = lay.int8_rows
        nb = dv // lay.block
        if lay.kind == MIXED:
            c.hi_bits = r[: lay.k_hi * dv * 2].view(np.uint16).reshape(lay.k_hi, dv).copy()
            off = lay.k_hi * dv * 2
        cb = nq * dv * lay.int_bits // 8
        if lay.int_bits == 8:
            c.codes = r[off: off + cb].reshape(nq, dv).astype(np.int64)
        else:
            c.codes = unpack_fields(r[off: off + cb], lay.int_bits, nq * dv).reshape(nq, dv)
        off += cb
        pairs = r[off: off + nq * nb * 4].view(np.uint16).reshape(nq, nb, 2)
        c.scale_bits = pairs[:, :, 0].copy()
        c.zero_bits = pairs[:, :, 1].copy()
        c.scale = f16_value(c.scale_bits)
        c.zero = f16_value(c.zero_bits)
        return c
    if lay.kind == BITALLOC:
        cbytes = lay.code_capacity
        dbits = r[cbytes: cbytes + 2 * dk].view(np.uint16).copy()
        meta = r[cbytes + 2 * dk: cbytes + 3 * dk].astype(np.int64)
        widths = (meta & 7) + 1
        fit = meta >> 4
        kappa = np.zeros((dk, dv), dtype=np.int64)
        off = 0
        for i in range(dk):
            b = int(widths[i])
            nbytes = dv * b // 8
            u = unpack_fields(r[off: off + nbytes], b, dv)
            # b = 1: the field is kappa' in {0, 1} for the levels -Delta, +Delta
            kappa[i] = 2 * u - 1 if b == 1 else u - (2 ** (b - 1) - 1)
            off += nbytes
        return Content(kappa=kappa, widths=widths, fit=fit, delta=f16_value(dbits),
                       delta_bits=dbits)
    if lay.kind == HEADALLOC:
        ng = dk // HA_GROUP
        cap = lay.code_capacity
        dbits = r[cap: cap + 2 * ng * dv].view(np.uint16).reshape(ng, dv).copy()
        fit = r[cap + 2 * ng * dv: cap + 3 * ng * dv].astype(np.int64).reshape(ng, dv)
        b = int(r[cap + 3 * ng * dv]) + 1
        u = unpack_fields(r[: dk * dv * b // 8], b, dk * dv).reshape(dk, dv)
        return Content(kappa=u - (2 ** (b - 1) - 1), width=b, fit=fit, delta=f16_value(dbits), delta_bits=dbits)
    raise ValueError(lay.kind)


def encode_region(lay: Layout, c: Content) -> np.ndarray:
    dk, dv = lay.dk, lay.dv
    out = np.zeros(lay.region_size(), dtype=np.uint8)
    if lay.kind == FP32:
        out[:] = np.asarray(c.S32, dtype=np.float32).reshape(-1).view(np.uint8)
        return out
    if lay.kind == UNIFORM:
        B = lay.bits
        u = np.asarray(c.kappa, dtype=np.int64) % (2 ** B)
        data = pack_fields(u.reshape(-1), B)
        out[: data.size] = data
        return out
    if lay.kind in (HAD_INT8, MIXED):
        off = 0
        if lay.kind == MIXED:
            hb = np.asarray(c.hi_bits, dtype=np.uint16).reshape(-1).view(np.uint8)
            out[: hb.size] = hb
            off = hb.size
        if lay.int_bits == 8:
            cd = np.asarray(c.codes, dtype=np.uint8).reshape(-1)
        else:
            cd = pack_fields(np.asarray(c.codes, dtype=np.int64).reshape(-1), lay.int_bits)
        out[off: off + cd.size] = cd
        off += cd.size
        pairs = np.stack([np.asarray(c.scale_bits, np.uint16), np.asarray(c.zero_bits, np.uint16)],
                         axis=-1).reshape(-1).view(np.uint8)
        out[off: off + pairs.size] = pairs
        return out
    if lay.kind == BITALLOC:
        off = 0
        for i in range(dk):
            b = int(c.widths[i])
            n = 2 ** (b - 1) - 1
            k = np.asarray(c.kappa[i], dtype=np.int64)
            data = pack_fields((k + 1) // 2 if b == 1 else k + n, b)
            out[off: off + data.size] = data
            off += data.size
        cbytes = lay.code_capacity
        if lay.budget == "layer":
            assert off <= cbytes, "widths exceed the head's code capacity"
        else:
            assert off == cbytes, "widths do not meet the head budget"
        out[cbytes: cbytes + 2 * dk] = np.asarray(c.delta_bits, np.uint16).view(np.uint8)
        meta = (np.asarray(c.widths, np.int64) - 1) | (np.asarray(c.fit, np.int64) << 4)
        out[cbytes + 2 * dk: cbytes + 3 * dk] = meta.astype(np.uint8)
        return out
    if lay.kind == HEADALLOC:
        ng = dk // HA_GROUP
        cap = lay.code_capacity
        b = int(c.width)
        data = pack_fields(np.asarray(c.kappa, dtype=np.int64).reshape(-1) + (2 ** (b - 1) - 1), b)
        assert data.size <= cap
        out[: data.size] = data
        out[cap: cap + 2 * ng * dv] = np.asarray(c.delta_bits, np.uint16).reshape(-1).view(np.uint8)
        out[cap + 2 * ng * dv: cap + 3 * ng * dv] = np.asarray(c.fit, np.int64).reshape(-1).astype(np.uint8)
        out[cap + 3 * ng * dv] = b - 1
        return out
    raise ValueError(lay.kind)


# ---------------------------------------------------------------------------
# Values held by a region

def stored_values(lay: Layout, c: Content) -> np.ndarray:
    """Dequantized values in the stored domain, physical row order, float64.

    Hadamard INT8 rows stay rotated here; float16 rows are in the original domain.
    """
    dk, dv = lay.dk, lay.dv
    if lay.kind == FP32:
        return np.array(c.S32, dtype=np.float64)
    if lay.kind == UNIFORM:
        return c.kappa.astype(np.float64) * 2.0 ** (1 - lay.bits)
    if lay.kind in (HAD_INT8, MIXED):
        G = lay.block
        sc = np.repeat(c.scale, G, axis=1)
        ze = np.repeat(c.zero, G, axis=1)
        y = ze + c.codes.astype(np.float64) * sc
        if lay.kind == HAD_INT8:
            return y
        return np.concatenate([f16_value(c.hi_bits), y], axis=0)
    if lay.kind == BITALLOC:
        return c.kappa.astype(np.float64) * c.delta[:, None]
    if lay.kind == HEADALLOC:
        return c.kappa.astype(np.float64) * np.repeat(c.delta, HA_GROUP, axis=0)
    raise ValueError(lay.kind)


def rotated_rows(lay: Layout) -> np.ndarray:
    """Boolean mask over physical rows: True where the row is stored rotated."""
    m = np.zeros(lay.dk, dtype=bool)
    if lay.kind == HAD_INT8:
        m[:] = True
    elif lay.kind == MIXED:
        m[lay.k_hi:] = True
    return m


def to_logical(lay: Layout, Y: np.ndarray, perm=None) -> np.ndarray:
    """Stored-domain physical rows -> state S in the original domain, logical order."""
    Y = np.asarray(Y, dtype=np.float64)
    X = Y.copy()
    rot = rotated_rows(lay)
    if rot.any():
        Hm = sylvester(lay.dv)
        X[rot] = Y[rot] @ Hm.T          # H^-1 = H: x_i = H y_i
    if lay.kind == MIXED:
        S = np.zeros_like(X)
        S[np.asarray(perm)] = X          # physical row p holds logical row perm[p]
        return S
    return X


def to_stored(lay: Layout, S: np.ndarray, perm=None) -> np.ndarray:
    """State S (logical order) -> physical rows in the stored domain."""
    S = np.asarray(S, dtype=np.float64)
    X = S[np.asarray(perm)] if lay.kind == MIXED else S.copy()
    rot = rotated_rows(lay)
    if rot.any():
        Hm = sylvester(lay.dv)
        X[rot] = X[rot] @ Hm.T           # y_i = H x_i
    return X


def bits_per_value_stored(lay: Layout) -> float:
    """Stored bits per state element, counting every metadata byte of the region."""
    return lay.region_size() * 8.0 / (lay.dk * lay.dv)


def initial_region(lay: Layout) -> np.ndarray:
    """Region of the zero state S_0 = 0 (auxiliary state reset, [WB-zh]
    "Reproduction assessment"): BITALLOC rows start at the mean width with the
    widest clipping fraction (k = 15, f = 1) and Delta = 0."""
    dk, dv = lay.dk, lay.dv
    if lay.kind == BITALLOC:
        c = Content(kappa=np.zeros((dk, dv), np.int64), widths=np.full(dk, lay.bbar),
                    fit=np.full(dk, 15), delta_bits=np.zeros(dk, np.uint16))
        return encode_region(lay, c)
    if lay.kind == HEADALLOC:
        ng = dk // HA_GROUP
        c = Content(kappa=np.zeros((dk, dv), np.int64), width=lay.bbar, fit=np.full((ng, dv), 15),
                    delta_bits=np.zeros((ng, dv), np.uint16))
        return encode_region(lay, c)
    return np.zeros(lay.region_size(), dtype=np.uint8)


__all__ = ["Layout", "Content", "decode_region", "encode_region", "stored_values", "HEADALLOC", "HA_GROUP",
           "to_logical", "to_stored", "rotated_rows", "initial_region", "f16_bits",
           "KINDS", "FP32", "UNIFORM", "HAD_INT8", "MIXED", "BITALLOC",
           "bits_per_value_stored"]
