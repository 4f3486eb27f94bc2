"""Hand-built pins of the oracle's conventions: tie rules, the DAMP ranking and the
byte packing.

Every expected value below is worked out by hand from the stated convention (the
arithmetic is written next to it), not taken from the oracle:
  * clipping fit ([LBRS] "Levels and storage": f over 16 values in [1/4, 1] by squared
    error): ties go to the larger f;
  * width integerisation ([LBRS] "State bit allocation": adjust widths to the budget):
    one-bit moves on the proxy's marginal cost, ties to the lower row;
  * DAMP selection ([DAMP] "Risk scoring and selection"): the k_hi highest C_u, ties to
    the lower row; permutation = selected rows ascending, then the rest ascending;
    P_u = 1 / max(1 - a^2, tau);
  * packing: UNIFORM two's-complement nibbles and BITALLOC b-bit fields LSB first at
    byte (dv/8) * sum of the previous widths, then f16 Delta and (b - 1) | (k << 4).
A plausible slip (ties to the other side, a sign, an off-by-one row offset, a swapped
nibble) fails one of them.
"""
import math

import numpy as np

from oracle import layouts as L
from oracle.allocation import fit_row, integer_widths, real_widths
from oracle.damp import risk_scores, select_permutation


# ---------------------------------------------------------------------------
# clipping fit


def test_fit_all_zero_row_takes_the_widest_fraction():
    # R = 0: every candidate step f16(f * 0 / n) is 0, every level 0, every error 0 --
    # a 16-way tie, which the convention resolves to k = 15 (f = 1)
    k, errs = fit_row(np.zeros(128), 0.0, 4)
    assert k == 15
    assert np.all(errs == 0.0)


def test_fit_exact_tie_goes_to_the_larger_fraction():
    # Width 2 (n = 1), R = 1. Candidates 12 and 13: f = 0.85 and 0.9, whose float16
    # steps are 1.7001953125 / 2 = 0.85009765625 (0.7 * 1024 = 716.8 -> 717) and
    # 1.7998046875 / 2 = 0.89990234375 (0.8 * 1024 = 819.2 -> 819); they sum to 1.75.
    # Row = [1, 0.75, 0, ...]: both values round to level 1 under either step, so
    #   err12 = (1 - 0.85009765625)^2 + (0.75 - 0.85009765625)^2
    #         = 0.14990234375^2 + 0.10009765625^2
    #   err13 = (1 - 0.89990234375)^2 + (0.75 - 0.89990234375)^2
    #         = 0.10009765625^2 + 0.14990234375^2          (the same two squares)
    # and every other candidate lies farther from the parabola's centre 0.875.
    x = np.zeros(128)
    x[0], x[1] = 1.0, 0.75
    k, errs = fit_row(x, 1.0, 2)
    a, b = 0.14990234375 ** 2, 0.10009765625 ** 2
    assert errs[12] == a + b and errs[13] == b + a
    assert np.all(np.delete(errs, [12, 13]) > errs[12])
    assert k == 13


# ---------------------------------------------------------------------------
# width integerisation


def _widths(c, bmin=2, bmax=8, bbar=4):
    c = np.asarray(c, np.float64)
    return list(integer_widths(c, real_widths(c, bbar), bbar, bmin, bmax))


def test_widths_removal_tie_moves_the_lower_row():
    # c = (4, 1, 1): GM = 4^(1/3), b* = 4 + (1/2) log2(c / GM) = (4 2/3, 3 2/3, 3 2/3)
    # -> rounded (5, 4, 4), one bit over. Losses 3 c 2^(-2b): 3*4/1024 = 3*1/256 =
    # 12/1024 for all three rows -> the lowest row gives the bit: (4, 4, 4)
    # (ties to the highest row would give (5, 4, 3)).
    assert _widths([4.0, 1.0, 1.0]) == [4, 4, 4]


def test_widths_addition_tie_moves_the_lower_row():
    # c = (1/4, 1, 1): b* = (3 1/3, 4 1/3, 4 1/3) -> (3, 4, 4), one bit short. Gains
    # (3/4) c 2^(-2b): (3/4)(1/4)/64 = (3/4)/256 = 3/1024 for all three -> row 0
    # takes it: (4, 4, 4).
    assert _widths([0.25, 1.0, 1.0]) == [4, 4, 4]


def test_widths_tie_between_equal_rows_behind_a_capped_row():
    # c = (16, 1, 1), b_max = 5: b* = (5 1/3, 3 1/3, 3 1/3) -> (5, 3, 3), one short;
    # row 0 sits at b_max, rows 1 and 2 tie at (3/4)/64 -> row 1: (5, 4, 3).
    assert _widths([16.0, 1.0, 1.0], bmax=5) == [5, 4, 3]
    # c = (1, 1, 64), b_max = 5: b* = (3, 3, 6) -> clipped (3, 3, 5), one short; rows 0
    # and 1 tie at (3/4)/64 -> row 0: (4, 3, 5).
    assert _widths([1.0, 1.0, 64.0], bmax=5) == [4, 3, 5]


# ---------------------------------------------------------------------------
# DAMP ranking


def test_damp_selection_ties_and_order():
    # C = (5, 3, 3, 1), keep 2: row 0, then the tie 1 / 2 goes to row 1.
    assert list(select_permutation([5.0, 3.0, 3.0, 1.0], 2)) == [0, 1, 2, 3]
    # C = (1, 3, 5, 3), keep 2: rows 2 and 1 (tie with row 3 to the lower), listed
    # ascending, then rows 0 and 3.
    assert list(select_permutation([1.0, 3.0, 5.0, 3.0], 2)) == [1, 2, 0, 3]
    # all equal over 128 rows: the first 16 rows are kept, the order is the identity
    assert list(select_permutation(np.ones(128), 16)) == list(range(128))


def test_damp_risk_score_hand_values():
    # One sample of a 3 x 128 head: row 0 = e_0, rows 1 and 2 zero. H e_0 is the
    # constant 1/sqrt(128) = 0.0883883476...; each 32-value block has max = min, so
    # scale = 0 and the block is stored as zero = f16(1/sqrt(128)) = 1.4140625 * 2^-4
    # (0.41421356 * 1024 = 424.15 -> 424) = 0.08837890625; the rotation back keeps the
    # energy, so E_0 = 128 (1/sqrt(128) - 0.08837890625)^2 and E_1 = E_2 = 0.
    X = np.zeros((1, 3, 128))
    X[0, 0, 0] = 1.0
    s = np.array([1e-3, 0.5, 1.0])
    E, P, C = risk_scores(X, s, 0.01, 32)
    e0 = 128 * (1 / math.sqrt(128) - 0.08837890625) ** 2
    # (the oracle rotates in float64: 1 - x^_0 loses ~11 digits to cancellation)
    assert abs(E[0] - e0) <= 1e-9 * e0 and E[1] == 0.0 and E[2] == 0.0
    # P_u = 1 / max(1 - e^{-2 s}, 0.01): 1 - e^{-0.002} = 0.0019980 < 0.01 -> 100;
    # 1 / (1 - e^{-1}) = 1.58197670686932...; 1 / (1 - e^{-2}) = 1.15651764274966...
    assert P[0] == 100.0
    assert abs(P[1] - 1.5819767068693265) < 1e-14
    assert abs(P[2] - 1.1565176427496657) < 1e-14
    assert abs(C[0] - 100.0 * e0) <= 1e-9 * C[0] and C[1] == 0.0


# ---------------------------------------------------------------------------
# byte packing


def test_uniform_nibble_packing_by_hand():
    lay = L.Layout(kind=L.UNIFORM, B=1, H=1, dk=16, dv=16, bits=4)
    kappa = np.zeros((16, 16), np.int64)
    kappa[0, :4] = [-1, 2, -8, 7]          # two's complement: F, 2, 8, 7
    kappa[1, 0] = 3                        # element 16 -> byte 8, low nibble
    reg = L.encode_region(lay, L.Content(kappa=kappa))
    # element n at bits [4n, 4n + 4), least significant first
    assert reg[0] == 0x2F and reg[1] == 0x78 and reg[8] == 0x03
    assert np.count_nonzero(reg) == 3
    assert np.array_equal(L.decode_region(lay, reg).kappa, kappa)


def test_bitalloc_field_packing_by_hand():
    lay = L.Layout(kind=L.BITALLOC, B=1, H=1, dk=128, dv=128)
    widths = np.full(128, 4)
    widths[0], widths[1] = 3, 5            # sum stays 512
    fit = np.full(128, 15)
    fit[0] = 7
    kappa = np.zeros((128, 128), np.int64)
    kappa[0, :] = 2                        # width 3: n = 3, field 5 = 0b101
    kappa[1, 0], kappa[1, 1] = 2, -15      # width 5: n = 15, fields 17 = 0b10001 and 0
    kappa[2, 0] = -7                       # width 4: n = 7, field 0; starts at byte 48 + 80
    kappa[2, 1] = 1                        # field 8 = 0b1000 -> high nibble of byte 128
    dbits = np.zeros(128, np.uint16)
    dbits[0], dbits[127] = 0x3C00, 0x1234
    reg = L.encode_region(lay, L.Content(kappa=kappa, widths=widths, fit=fit, delta_bits=dbits))
    # row 0, fields 101 at bits 3j: bits 0..7 = 1,0,1,1,0,1,1,0 -> 0x6D;
    # bits 8..15 = 1,1,0,1,1,0,1,1 -> 0xDB; bits 16..23 = 0,1,1,0,1,1,0,1 -> 0xB6
    assert list(reg[:3]) == [0x6D, 0xDB, 0xB6] and list(reg[3:6]) == [0x6D, 0xDB, 0xB6]
    # row 1 starts at byte 16 * 3 = 48: fields 10001 and 00000 -> bits 0..7 =
    # 1,0,0,0,1,0,0,0 -> 0x11; row 1's other fields are 15 = 01111
    assert reg[48] == 0x11
    # row 2 starts at byte 48 + 16 * 5 = 128: fields 0 and 8 -> 0x80
    assert reg[128] == 0x80
    # after the 8192 code bytes: f16 Delta little-endian, then (b - 1) | (k << 4)
    assert reg[8192] == 0x00 and reg[8193] == 0x3C and reg[8192 + 254] == 0x34 and reg[8192 + 255] == 0x12
    assert reg[8192 + 256] == (2 | (7 << 4)) and reg[8192 + 257] == (4 | (15 << 4))
    assert reg[8192 + 258] == (3 | (15 << 4))
    dec = L.decode_region(lay, reg)
    assert np.array_equal(dec.kappa, kappa) and np.array_equal(dec.widths, widths)
