"""Bit-exact GPU cases of round to nearest: exact half-step ties and values beyond the
rails, with no boundary window.

[WB-zh] "Reproduction assessment" fixes the rounding of the deterministic write-back:
half-step ties go to the even index and values beyond the grid are clipped to the rail.
A stored state of zero, no decay (s = 0), beta = 1 and a one-hot key k = e_i make one
decode step write row i := v exactly (u = k^T S = 0, w = v, S' = e_i v^T); the values
of v are multiples of 1/16, exact in float32, chosen on half steps and beyond the rails
of a grid whose step is 1/8. The expected levels are worked out here from the rule
(round half to even, then clip), not from the oracle, and compared code for code. The
same values go through the import (one round-to-nearest write-back of a given state).
The Hadamard-rotated INT8 rows cannot carry exact ties from float32 inputs (the rotation
rounds), so they are not in these cases; the float16 rows of the mixed layout are
(float16 midpoints, ties to the even significand).
"""
import numpy as np
import pytest

from oracle import layouts as L

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

STEP = 0.125


def _half_steps_and_rails(dv=128):
    """Values for one row: every half step (m + 1/2)/8 for m = -10..9 (signed ties on
    both sides of zero, and the ties just past the rails), levels themselves, zero, and
    values well beyond the rails; multiples of 1/16, exact in float32."""
    v = [(m + 0.5) * STEP for m in range(-10, 10)]
    v += [m * STEP for m in range(-9, 9)]
    v += [0.0, -0.0, 1.0, -1.0, 1.5, -1.5, 3.0, -3.0, 0.9375, -0.9375, 2.5, -2.5]
    v += [(m + 0.5) * STEP for m in range(-3, 3)] * 4
    rng = np.random.default_rng(5)
    while len(v) < dv:
        v.append(float(rng.integers(-40, 40)) / 16.0)
    return np.array(v[:dv], dtype=np.float32)


def _rne_clip(x, lo, hi):
    # round half to even, then clip to the rails
    return np.clip(np.rint(np.asarray(x, np.float64)), lo, hi).astype(np.int64)


def _one_hot_step(st, B, H, dk, dv, rows, vrow, per_row=True):
    """One decode step with S = 0 stored, s = 0, beta = 1, k = e_rows[h], v = vrow."""
    q = np.zeros((B, H, dk), np.float32)
    k = np.zeros((B, H, dk), np.float32)
    for b in range(B):
        for h in range(H):
            k[b, h, rows[h]] = 1.0
            q[b, h, rows[h]] = 0.5
    v = np.broadcast_to(vrow, (B, H, dv)).astype(np.float32).copy()
    beta = np.ones((B, H), np.float32)
    s = np.zeros((B, H, dk) if per_row else (B, H), np.float32)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q, k, v, beta, s)]
    o = torch.zeros((B, H, dv), dtype=torch.float32, device="cuda")
    st.step_decode(*dev, o, 0)
    torch.cuda.synchronize()
    # o = S'^T q = q_i v, read before quantization
    assert np.array_equal(o.cpu().numpy(), 0.5 * v), "readout"


def _regions(st, lay):
    return st.regions().cpu().numpy()[:, : lay.region_size()]


@pytest.mark.parametrize("path", ["decode", "import"])
def test_uniform4_ties_and_rails_exact(path):
    import linear_attn_decode_amd as wb
    print(f"\n[case] exact uniform-4 {path}", flush=True)
    B, H, d = 1, 2, 128
    lay = L.Layout(kind=L.UNIFORM, B=B, H=H, dk=d, dv=d, bits=4)
    st = wb.WriteBackState("uniform", "rtn", B, H, d, d, True, bits=4)
    vrow = _half_steps_and_rails(d)
    rows = [5, 77]
    if path == "decode":
        _one_hot_step(st, B, H, d, d, rows, vrow)
    else:
        S = np.zeros((B, H, d, d), np.float32)
        for h in range(H):
            S[0, h, rows[h]] = vrow
        st.quantize(torch.from_numpy(S).cuda())
        torch.cuda.synchronize()
    regs = _regions(st, lay)
    want = _rne_clip(vrow / STEP, -8, 7)
    for h in range(H):
        kappa = L.decode_region(lay, regs[h]).kappa
        exp = np.zeros((d, d), np.int64)
        exp[rows[h]] = want
        assert np.array_equal(kappa, exp), (h, np.argwhere(kappa != exp)[:5])


@pytest.mark.parametrize("fit,R", [(15, 0.875), (0, 3.5)], ids=["f1-ties", "f025-rails"])
@pytest.mark.parametrize("path", ["decode", "import"])
def test_bitalloc_ties_and_rails_exact(path, fit, R):
    """Width 4 (n = 7). With fit k the step is f16(f R / 7): f = 1, R = 0.875 and
    f = 1/4, R = 3.5 both give 0.125; in the second case values up to 28 steps are
    clipped to +-7."""
    import linear_attn_decode_amd as wb
    print(f"\n[case] exact bitalloc {path} fit={fit} R={R}", flush=True)
    B, H, d = 1, 2, 128
    lay = L.Layout(kind=L.BITALLOC, B=B, H=H, dk=d, dv=d)
    st = wb.WriteBackState("bitalloc", "rtn", B, H, d, d, True)
    vrow = _half_steps_and_rails(d)
    vrow = np.clip(vrow, -R, R).astype(np.float32)
    vrow[0] = R                                       # the row maximum sets the step
    rows = [9, 100]
    code_bytes = d * d * lay.bbar // 8
    regs_dev = st.regions()
    for h in range(H):
        regs_dev[h, code_bytes + 2 * d + rows[h]] = (lay.bbar - 1) | (fit << 4)
    torch.cuda.synchronize()
    if path == "decode":
        _one_hot_step(st, B, H, d, d, rows, vrow)
    else:
        S = np.zeros((B, H, d, d), np.float32)
        for h in range(H):
            S[0, h, rows[h]] = vrow
        st.quantize(torch.from_numpy(S).cuda())
        torch.cuda.synchronize()
    regs = _regions(st, lay)
    want = _rne_clip(vrow / STEP, -7, 7)
    for h in range(H):
        c = L.decode_region(lay, regs[h])
        exp = np.zeros((d, d), np.int64)
        exp[rows[h]] = want
        assert np.array_equal(c.kappa, exp), (h, np.argwhere(c.kappa != exp)[:5])
        dexp = np.zeros(d, np.uint16)
        dexp[rows[h]] = 0x3000                        # float16 0.125
        assert np.array_equal(c.delta_bits, dexp), h
        assert np.all(c.widths == lay.bbar) and c.fit[rows[h]] == fit


@pytest.mark.parametrize("path", ["decode", "import"])
def test_headalloc_ties_and_rails_exact(path):
    """One width (4, n = 7) and a step per 32 key rows of a column. Import: in group 0
    row 0 holds 0.875 (f = 1: step 0.125) and rows 1..31 the half steps; in group 1 the
    fit index is set to 0 (f = 1/4) and row 32 holds 3.5 (step 0.125), the other rows
    values up to 28 steps, clipped to +-7. Decode: one written row per head; with f = 1
    every value is its column's maximum (level +-7), with f = 1/4 it is four times past
    the rail."""
    import linear_attn_decode_amd as wb
    print(f"\n[case] exact headalloc {path}", flush=True)
    B, H, d = 1, 2, 128
    lay = L.Layout(kind=L.HEADALLOC, B=B, H=H, dk=d, dv=d, per_row_decay=False)
    st = wb.WriteBackState("headalloc", "rtn", B, H, d, d, False)
    cap = lay.code_capacity
    ng = d // L.HA_GROUP
    regs_dev = st.regions()
    for h in range(H):
        # fit index 0 (f = 1/4) for every column of group 1
        regs_dev[h, cap + 2 * ng * d + d: cap + 2 * ng * d + 2 * d] = 0
    torch.cuda.synchronize()
    vcol = _half_steps_and_rails(32)                  # 32 values down a column
    if path == "import":
        S = np.zeros((B, H, d, d), np.float32)
        g0 = np.clip(vcol, -0.875, 0.875)
        g0[0] = 0.875
        g1 = np.clip(vcol * 4, -3.5, 3.5)
        g1[0] = 3.5
        for h in range(H):
            S[0, h, 0:32, :] = g0[:, None]
            S[0, h, 32:64, :] = g1[:, None]
        st.quantize(torch.from_numpy(S).cuda())
        torch.cuda.synchronize()
        regs = _regions(st, lay)
        for h in range(H):
            c = L.decode_region(lay, regs[h])
            exp = np.zeros((d, d), np.int64)
            exp[0:32] = _rne_clip(g0 / STEP, -7, 7)[:, None]
            exp[32:64] = _rne_clip(g1 / STEP, -7, 7)[:, None]
            assert np.array_equal(c.kappa, exp), (h, np.argwhere(c.kappa != exp)[:5])
            assert np.all(c.delta_bits[:2] == 0x3000) and np.all(c.delta_bits[2:] == 0)
    else:
        vrow = _half_steps_and_rails(d)
        vrow[vrow == 0] = 0.25                        # a zero column has a zero step
        rows = [3, 40]                                # group 0 (f = 1) and group 1 (f = 1/4)
        _one_hot_step(st, B, H, d, d, rows, vrow, per_row=False)
        regs = _regions(st, lay)
        for h in range(H):
            c = L.decode_region(lay, regs[h])
            exp = np.zeros((d, d), np.int64)
            exp[rows[h]] = np.where(vrow > 0, 7, -7)
            assert np.array_equal(c.kappa, exp), (h, np.argwhere(c.kappa != exp)[:5])


@pytest.mark.parametrize("path", ["decode", "import"])
def test_mixed_float16_rows_ties_exact(path):
    """float16 rows of the mixed layout: values on float16 midpoints round to the even
    significand (1 + 2^-11 -> 1, 1 + 3 * 2^-11 -> 1 + 2^-9, their negatives, and
    midpoints at other exponents); a value below half the smallest subnormal goes to 0."""
    import linear_attn_decode_amd as wb
    print(f"\n[case] exact mixed float16 rows {path}", flush=True)
    B, H, d = 1, 2, 128
    lay = L.Layout(kind=L.MIXED, B=B, H=H, dk=d, dv=d, block=32, k_hi=16)
    rng = np.random.default_rng(8)
    perm = np.stack([rng.permutation(d) for _ in range(H)])
    st = wb.WriteBackState("mixed", "rtn", B, H, d, d, True, block=32, k_hi=16, perm=perm)
    e = []
    want = []
    for sgn in (1.0, -1.0):
        for ex in (-3, 0, 4):
            for m in range(0, 8):
                # midpoint between the float16 values (1024 + m) and (1024 + m + 1) * 2^(ex - 10)
                e.append(sgn * (1024 + m + 0.5) * 2.0 ** (ex - 10))
                want.append(sgn * (1024 + m + (m % 2)) * 2.0 ** (ex - 10))
    e.append(2.0 ** -26)                              # below half the smallest subnormal 2^-24
    want.append(0.0)
    e.append(3 * 2.0 ** -25)                          # 1.5 subnormal steps: tie to 2 * 2^-24
    want.append(2 * 2.0 ** -24)
    vrow = np.zeros(d, np.float32)
    vrow[: len(e)] = e
    wrow = np.zeros(d)
    wrow[: len(want)] = want
    assert np.array_equal(vrow.astype(np.float64), np.array(list(e) + [0.0] * (d - len(e))))
    phys = 5                                          # a float16 row
    rows = [int(perm[h][phys]) for h in range(H)]     # its logical row
    if path == "decode":
        _one_hot_step(st, B, H, d, d, rows, vrow)
    else:
        S = np.zeros((B, H, d, d), np.float32)
        for h in range(H):
            S[0, h, rows[h]] = vrow
        st.quantize(torch.from_numpy(S).cuda())
        torch.cuda.synchronize()
    regs = _regions(st, lay)
    for h in range(H):
        c = L.decode_region(lay, regs[h])
        got = c.hi_bits.view(np.float16).astype(np.float64)
        exp = np.zeros((lay.k_hi, d))
        exp[phys] = wrow
        assert np.array_equal(got, exp), (h, np.argwhere(got != exp)[:5])
