"""GPU parity of the fused decode write-back step (every layout x write-back rule),
import/export, the allocation pass and DAMP selection, against the CPU oracle.

Each test prints the case it runs before launching GPU work."""
import numpy as np
import pytest

from oracle import layouts as L
from oracle.allocation import allocate_head
from oracle.damp import risk_scores, select_permutation
from oracle.numerics import f16_value
from oracle.step import allocate_region, decode_step, export_state, import_state, write_back
from synth import decode_inputs
from tests.parity import Tally, check_head

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _wb():
    import linear_attn_decode_amd as wb
    return wb


def _layout(kind, mode, B, H, dk, per_row=True, **kw):
    args = dict(kind=kind, B=B, H=H, dk=dk, dv=dk, mode=mode, per_row_decay=per_row, seed=0x5EED_1234_ABCD)
    if kind == L.HAD_INT8:
        args["block"] = 128
    args.update(kw)
    return L.Layout(**args)


def _state(lay, perm=None):
    wb = _wb()
    return wb.WriteBackState(lay.kind, lay.mode, lay.B, lay.H, lay.dk, lay.dv, lay.per_row_decay,
                             bits=lay.bits, block=lay.block, k_hi=lay.k_hi, bbar=lay.bbar, bmin=lay.bmin,
                             bmax=lay.bmax, seed=lay.seed, perm=perm, mem_bits=lay.mem_bits, budget=lay.budget,
                             int_bits=0 if lay.int_bits == 8 else lay.int_bits)


def _warm_state(rng, B, H, dk, dv):
    """A realistic stored state: rows of very different ranges."""
    scale = np.exp(rng.uniform(-3.0, 0.5, (B, H, dk, 1)))
    return (rng.standard_normal((B, H, dk, dv)) * scale).astype(np.float32)


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_decode(lay, T, heads=None, warm=True, seed=1, perm=None, steps_checked=None, alloc_every=None,
               edit=None, state=None):
    """Teacher-forced decode steps against the oracle (``state``: continue an existing
    state instead of a fresh one)."""
    print(f"\n[case] kind={lay.kind} mode={lay.mode} B={lay.B} H={lay.H} dk={lay.dk} T={T}", flush=True)
    B, H, dk, dv = lay.B, lay.H, lay.dk, lay.dv
    rng = np.random.default_rng(seed)
    if lay.kind == L.MIXED and perm is None:
        perm = np.stack([rng.permutation(dk) for _ in range(H)])
    st = _state(lay, perm) if state is None else state
    inp = decode_inputs(seed, B, H, dk, dv, T, lay.per_row_decay)
    if edit is not None:
        edit(inp)
    dev = {k: _to_dev(v) for k, v in inp.items()}
    o = torch.zeros((B, H, dv), dtype=torch.float32, device="cuda")
    if warm:
        st.quantize(_to_dev(_warm_state(rng, B, H, dk, dv)))
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    tally = Tally()
    s_all = inp["s"]
    for t in range(T):
        check = steps_checked is None or t in steps_checked
        if alloc_every and t % alloc_every == 0 and t > 0:
            st.allocate_bits(dev["s"] if s_all.ndim == 3 else None)
        if check:
            regs = st.regions()
            reg_in = {bh: regs[bh[0] * H + bh[1]].cpu().numpy() for bh in heads}
            res = st.residuals()
            e_in = {bh: res[bh[0], bh[1]].cpu().numpy() for bh in heads} if res is not None else None
        st.step_decode(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], dev["s"], o, t)
        if not check:
            continue
        torch.cuda.synchronize()
        regs = st.regions()
        res = st.residuals()
        o_np = o.cpu().numpy()
        for (b, h) in heads:
            check_head(lay, reg_in[(b, h)], regs[b * H + h].cpu().numpy(),
                       None if e_in is None else e_in[(b, h)],
                       None if res is None else res[b, h].cpu().numpy(), o_np[b, h],
                       inp["q"][t, b, h], inp["k"][t, b, h], inp["v"][t, b, h], inp["beta"][t, b, h],
                       s_all[b, h], t, b, h, None if perm is None else perm[h], tally)
    print("[tally]", tally.summary(), flush=True)
    assert tally.ok(), tally.summary()
    return tally


def test_tiny_uniform_4bit_rtn_every_step():
    lay = _layout(L.UNIFORM, "rtn", 1, 1, 16, bits=4)
    run_decode(lay, 256, warm=False, seed=0)


def test_tiny_uniform_4bit_error_feedback_every_step():
    lay = _layout(L.UNIFORM, "ef", 1, 1, 16, bits=4)
    run_decode(lay, 256, warm=False, seed=0)


@pytest.mark.parametrize("mode,k", [("dir", 2), ("dir", 3), ("resq", 2), ("resq", 4)])
def test_tiny_uniform_4bit_temporal_memory_every_step(mode, k):
    lay = _layout(L.UNIFORM, mode, 1, 1, 16, bits=4, mem_bits=k)
    run_decode(lay, 256, warm=False, seed=0)


@pytest.mark.parametrize("mode,k,bits", [("dir", 2, 4), ("dir", 4, 2), ("resq", 3, 4), ("resq", 2, 8)])
def test_uniform_temporal_memory_128(mode, k, bits):
    lay = _layout(L.UNIFORM, mode, 2, 2, 128, bits=bits, mem_bits=k)
    run_decode(lay, 6, warm=True, seed=14)


@pytest.mark.parametrize("mode,k", [("rtn", 0), ("ef", 0), ("dir", 2), ("resq", 3)])
def test_uniform_write_activity_counters(mode, k):
    """Per-head write activity (all eight counts) summed over the steps, and the vote
    state after every step, against the oracle on the same stored states (each step
    starts from the GPU's region, side state and vote state); an element may differ only
    where one of its decisions (write margin 1, vote band edges, level rounding) is
    within the comparison window."""
    print(f"\n[case] write activity UNIFORM-4 mode={mode} k={k}", flush=True)
    from tests.parity import WINDOW
    B, H, dk, T = 2, 2, 128, 6
    lay = _layout(L.UNIFORM, mode, B, H, dk, bits=4, mem_bits=k)
    rng = np.random.default_rng(15)
    st = _state(lay)
    inp = decode_inputs(15, B, H, dk, dk, T, True)
    dev = {key: _to_dev(val) for key, val in inp.items()}
    st.quantize(_to_dev((_warm_state(rng, B, H, dk, dk) * 0.3).astype(np.float32)))
    ctr = torch.zeros((B, H, 8), dtype=torch.int32, device="cuda")
    votes = torch.zeros((B, H, dk, dk), dtype=torch.uint8, device="cuda")
    st.set_activity(ctr, votes)
    o = torch.zeros((B, H, dk), dtype=torch.float32, device="cuda")
    expect = np.zeros((B, H, 8), np.int64)
    slack = np.zeros((B, H), np.int64)
    vote_bad = 0
    step = 2.0 ** -3
    for t in range(T):
        torch.cuda.synchronize()
        regs = st.regions().cpu().numpy()
        res = st.residuals()
        e_in = res.cpu().numpy() if res is not None else None
        v_in = votes.cpu().numpy()
        st.step_decode(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], dev["s"], o, t)
        torch.cuda.synchronize()
        v_out = votes.cpu().numpy()
        for b in range(B):
            for h in range(H):
                reg_in = regs[b * H + h][: lay.region_size()]
                r = decode_step(lay, reg_in, None if e_in is None else e_in[b, h], inp["q"][t, b, h],
                                inp["k"][t, b, h], inp["v"][t, b, h], inp["beta"][t, b, h], inp["s"][b, h],
                                t, b, h, votes_in=v_in[b, h])
                expect[b, h] += r.wb.activity
                kp = L.decode_region(lay, reg_in).kappa
                ad = np.abs(r.wb.X - kp * step) / step
                near = (np.abs(ad - 0.5) <= WINDOW) | (np.abs(ad - 0.125) <= WINDOW) | (r.wb.boundary <= WINDOW)
                slack[b, h] += int(near.sum())
                vote_bad += int(((v_out[b, h] != r.wb.votes_new) & ~near).sum())
    st.set_activity(None)
    torch.cuda.synchronize()
    got = ctr.cpu().numpy().astype(np.int64)
    print("[activity] gpu", got.sum(axis=(0, 1)).tolist(), "oracle", expect.sum(axis=(0, 1)).tolist(),
          "near-boundary elements", int(slack.sum()), "vote-state mismatches", vote_bad, flush=True)
    assert vote_bad == 0
    assert np.all(np.abs(got - expect) <= slack[..., None]), (got, expect, slack)
    assert expect[..., 0].sum() > 0 and expect[..., 2].sum() > 0
    assert expect[..., 5].sum() > 0 and expect[..., 6].sum() > 0 and 0 < expect[..., 7].sum() < expect[..., 2].sum()
    if mode == "dir":
        assert expect[..., 3].sum() > 0 and expect[..., 4].sum() > 0
    else:
        assert got[..., 3].sum() == 0


def test_tiny_fp32_identity():
    lay = _layout(L.FP32, "rtn", 1, 1, 16)
    run_decode(lay, 64, warm=False, seed=0)


CASES = [
    (L.FP32, {}), (L.UNIFORM, {"bits": 4}), (L.UNIFORM, {"bits": 2}), (L.UNIFORM, {"bits": 8}),
    (L.HAD_INT8, {"block": 128}), (L.HAD_INT8, {"block": 32}), (L.MIXED, {"block": 32, "k_hi": 16}),
    (L.BITALLOC, {}), (L.BITALLOC, {"budget": "layer"}), (L.HEADALLOC, {}),
    (L.HAD_INT8, {"block": 32, "int_bits": 4}), (L.HAD_INT8, {"block": 128, "int_bits": 4}),
    (L.MIXED, {"block": 32, "k_hi": 16, "int_bits": 4}),
]


@pytest.mark.parametrize("kind,kw", CASES, ids=[f"{k}-{'-'.join(map(str, v.values()))}" for k, v in CASES])
@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_decode_matrix(kind, kw, mode):
    if kind == L.FP32 and mode != "rtn":
        pytest.skip("identity write-back has no rounding rule")
    lay = _layout(kind, mode, 2, 3, 128, **kw)
    run_decode(lay, 4, warm=True, seed=11)


def test_decode_per_head_decay_had_int8():
    lay = _layout(L.HAD_INT8, "rtn", 2, 2, 128, per_row=False, block=128)
    run_decode(lay, 3, warm=True, seed=12)


def test_bitalloc_after_allocation_rtn_and_sr():
    for mode in ("rtn", "sr"):
        lay = _layout(L.BITALLOC, mode, 2, 2, 128)
        run_decode(lay, 7, warm=True, seed=13, alloc_every=3)


@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_bitalloc_one_bit_rows_decode_after_allocation(mode):
    """Decode steps with rows one bit wide (bmin = 1, mean width 3: the allocation
    passes leave slow rows wide and fast rows at sign times mean |x|)."""
    print(f"\n[case] one-bit rows BITALLOC decode {mode}", flush=True)
    lay = _layout(L.BITALLOC, mode, 2, 2, 128, bbar=3, bmin=1)
    run_decode(lay, 7, warm=True, seed=19, alloc_every=3)


def _width_patterns(rng, lay, n):
    """Row-width patterns for `n` heads that put every width the layout allows next to
    every other inside the groups of rows a wavefront handles together: all rows at the
    narrowest and (layer budget) the widest width, rows in random order, widths falling
    with the row index, and alternating extremes; under the per-head budget each pattern
    is brought to the budget's total by moving single bits between random rows."""
    dk, lo, hi = lay.dk, lay.bmin, lay.bmax
    pats = [np.full(dk, lo), np.full(dk, hi) if lay.budget == "layer" else rng.integers(lo, hi + 1, dk),
            rng.integers(lo, hi + 1, dk), np.sort(rng.integers(lo, hi + 1, dk))[::-1],
            np.where(np.arange(dk) % 2 == 0, lo, hi)]
    out = []
    for i in range(n):
        w = np.array(pats[i % len(pats)] if i < len(pats) else rng.integers(lo, hi + 1, dk), np.int64)
        if lay.budget != "layer":
            total = lay.bbar * dk
            while w.sum() != total:
                j = int(rng.integers(dk))
                if w.sum() > total and w[j] > lo:
                    w[j] -= 1
                elif w.sum() < total and w[j] < hi:
                    w[j] += 1
        out.append(w)
    return out


@pytest.mark.parametrize("budget,bmin", [("head", 2), ("head", 1), ("layer", 2), ("layer", 1)])
@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_bitalloc_decode_arbitrary_widths(budget, bmin, mode):
    """Decode steps from regions written by the oracle's encoder with arbitrary row widths
    (every width next to every other, heads at the narrowest and widest totals under the
    layer budget, one-bit rows among them), random levels, fit indices and steps."""
    print(f"\n[case] arbitrary widths BITALLOC budget={budget} bmin={bmin} {mode}", flush=True)
    B, H, dk = 2, 4, 128
    lay = _layout(L.BITALLOC, mode, B, H, dk, bbar=3 if bmin == 1 else 4, bmin=bmin, budget=budget)
    rng = np.random.default_rng(61 + bmin)
    st = _state(lay)
    regs = st.regions()
    size = lay.region_size()
    for i, w in enumerate(_width_patterns(rng, lay, B * H)):
        n = 2 ** (w - 1) - 1
        kappa = np.where((w == 1)[:, None], 2 * rng.integers(0, 2, (dk, dk)) - 1,
                         rng.integers(-n[:, None], n[:, None] + 1, (dk, dk)))
        delta = (10.0 ** rng.uniform(-3, -1, dk)).astype(np.float16)
        c = L.Content(kappa=kappa, widths=w, fit=rng.integers(0, 16, dk), delta_bits=delta.view(np.uint16))
        regs[i, :size].copy_(torch.from_numpy(L.encode_region(lay, c)))
    torch.cuda.synchronize()
    run_decode(lay, 3, warm=False, seed=62, state=st)


@pytest.mark.parametrize("per_row", [False, True])
@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_headalloc_decode_arbitrary_widths(mode, per_row):
    """Decode steps of the per-head unit from regions written by the oracle's encoder:
    every width from 2 to 8 among the heads, random levels, fit indices and group steps
    (some steps zero)."""
    print(f"\n[case] arbitrary widths HEADALLOC {mode} per_row={per_row}", flush=True)
    B, H, dk = 2, 4, 128
    lay = _layout(L.HEADALLOC, mode, B, H, dk, per_row=per_row)
    rng = np.random.default_rng(71)
    st = _state(lay)
    regs = st.regions()
    size = lay.region_size()
    ng = dk // L.HA_GROUP
    for i in range(B * H):
        w = [2, 3, 4, 5, 6, 7, 8, int(rng.integers(2, 9))][i]
        n = 2 ** (w - 1) - 1
        delta = (10.0 ** rng.uniform(-3, -1, (ng, dk))).astype(np.float16)
        delta[rng.random((ng, dk)) < 0.02] = 0
        c = L.Content(kappa=rng.integers(-n, n + 1, (dk, dk)), width=w, fit=rng.integers(0, 16, (ng, dk)),
                      delta_bits=delta.view(np.uint16))
        regs[i, :size].copy_(torch.from_numpy(L.encode_region(lay, c)))
    torch.cuda.synchronize()
    run_decode(lay, 3, warm=False, seed=72, state=st)


@pytest.mark.parametrize("case", ["warm", "spread"])
def test_allocate_bits_one_bit_rows_matches_oracle(case):
    """The allocation pass with a one-bit floor (bmin = 1, mean width 3) on two passes,
    the second from the widths the first left (one-bit rows read as -Delta, +Delta)."""
    print(f"\n[case] allocate_bits one-bit floor {case}", flush=True)
    B, H, dk = 2, 4, 128
    lay = _layout(L.BITALLOC, "rtn", B, H, dk, bbar=3, bmin=1)
    rng = np.random.default_rng(47)
    st = _state(lay)
    S, s = _alloc_case(case, rng, B, H, dk)
    st.quantize(_to_dev(S))
    r = np.full((B, H, dk), 1.0 / (3 * dk), dtype=np.float32)
    ones = 0
    for pas, s_pass in enumerate((s, np.ascontiguousarray(s[..., ::-1]))):
        torch.cuda.synchronize()
        before = st.regions().cpu().numpy()
        st.allocate_bits(_to_dev(s_pass), _to_dev(r))
        torch.cuda.synchronize()
        after = st.regions().cpu().numpy()
        for b in range(B):
            for h in range(H):
                reg_in = before[b * H + h][: lay.region_size()]
                reg_orc, alloc = allocate_region(lay, reg_in, s_pass[b, h].astype(np.float64),
                                                 r[b, h].astype(np.float64))
                ones += int((alloc["widths"] == 1).sum())
                _check_alloc_head(lay, after[b * H + h][: lay.region_size()], reg_orc, alloc, (pas, b, h), reg_in)
    print(f"[alloc-1bit] one-bit rows chosen over both passes: {ones}", flush=True)
    assert ones > 0


@pytest.mark.parametrize("mode", ["rtn", "ef"])
def test_bitalloc_layer_budget_decode_after_allocation(mode):
    """Decode steps on heads whose widths differ under the layer-wise budget (each
    head's codes end at its own length inside the code area)."""
    print(f"\n[case] layer-budget BITALLOC decode {mode}", flush=True)
    lay = _layout(L.BITALLOC, mode, 2, 4, 128, budget="layer")
    run_decode(lay, 7, warm=True, seed=17, alloc_every=3)


# ---------------------------------------------------------------------------- import / export


@pytest.mark.parametrize("kind,kw", CASES, ids=[f"{k}-{'-'.join(map(str, v.values()))}" for k, v in CASES])
def test_import_export(kind, kw):
    print(f"\n[case] import/export kind={kind} {kw}", flush=True)
    B, H, dk = 2, 2, 128
    lay = _layout(kind, "rtn", B, H, dk, **kw)
    rng = np.random.default_rng(21)
    perm = np.stack([rng.permutation(dk) for _ in range(H)]) if kind == L.MIXED else None
    st = _state(lay, perm)
    S = _warm_state(rng, B, H, dk, dk)
    st.quantize(_to_dev(S))
    out = torch.zeros((B, H, dk, dk), dtype=torch.float32, device="cuda")
    st.dequant(out)
    torch.cuda.synchronize()
    regs = st.regions().cpu().numpy()
    S_gpu = out.cpu().numpy()
    init = L.initial_region(lay)
    tally = Tally()
    for b in range(B):
        for h in range(H):
            p = None if perm is None else perm[h]
            reg = regs[b * H + h][: lay.region_size()]
            # export: the oracle's decoder on the GPU bytes, to float32
            ref = export_state(lay, reg, p)
            assert np.allclose(S_gpu[b, h], ref, rtol=2 ** -23, atol=1e-7 * np.abs(ref).max())
            # import: one nearest write-back of S from the zero state's metadata
            X = L.to_stored(lay, S[b, h].astype(np.float64), p)
            cin = L.decode_region(lay, init)
            orc = write_back(lay, X, None, 0, b, h, prev=cin)
            g = L.decode_region(lay, reg)
            o_reg = orc.region
            if kind == L.FP32:
                assert np.array_equal(reg, o_reg)
                continue
            if kind in (L.HAD_INT8, L.MIXED):
                oc = L.decode_region(lay, o_reg)
                from tests.parity import _meta_ok
                _meta_ok(g.scale_bits, oc.scale_bits, orc.meta_pre["scale"], tally, ("scale", b, h))
                _meta_ok(g.zero_bits, oc.zero_bits, orc.meta_pre["zero"], tally, ("zero", b, h))
                override = {"scale": g.scale, "zero": g.zero}
            elif kind in (L.BITALLOC, L.HEADALLOC):
                from tests.parity import _meta_ok
                oc = L.decode_region(lay, o_reg)
                _meta_ok(g.delta_bits, oc.delta_bits, orc.meta_pre["delta"], tally, ("delta", b, h))
                override = {"delta": g.delta}
            else:
                override = None
            req = write_back(lay, X, None, 0, b, h, prev=cin, meta_override=override)
            diff = req.region != reg
            if diff.any():
                # element-level check through the decoded codes
                rc = L.decode_region(lay, req.region)
                if kind == L.UNIFORM or kind == L.BITALLOC:
                    d = rc.kappa != g.kappa
                    assert np.all(req.boundary[d] <= 1e-5), (kind, np.argwhere(d)[:3])
                    tally.mismatch += int(d.sum())
                else:
                    q0 = dk - lay.int8_rows
                    d = rc.codes != g.codes
                    assert np.all(req.boundary[q0:][d] <= 1e-5)
                    tally.mismatch += int(d.sum())
                    if kind == L.MIXED:
                        dh = rc.hi_bits != g.hi_bits
                        assert np.all(req.boundary[:q0][dh] <= 1e-5)
                        tally.mismatch += int(dh.sum())
            tally.elems += dk * dk
    print("[tally]", tally.summary(), flush=True)
    assert not tally.bad and tally.mismatch <= 1e-4 * tally.elems, tally.summary()


# ---------------------------------------------------------------------------- degenerate inputs

def _zero_keys(inp):
    inp["k"][:] = 0.0


def _no_write(inp):
    inp["beta"][:] = 0.0


def _no_decay(inp):
    inp["s"][:] = 0.0


def _one_hot_overwrite(inp):
    # unit keys e_i with beta = 1: the delta rule replaces row i by v ([LBRS] recurrence)
    T, B, H, dk = inp["k"].shape
    inp["k"][:] = 0.0
    for t in range(T):
        inp["k"][t, :, :, (7 * t + 3) % dk] = 1.0
    inp["beta"][:] = 1.0


DEGENERATE = [
    ("zero-state-zero-keys", _zero_keys, False),   # every stored value stays 0: Delta = 0, zero-range blocks
    ("pure-decay", _no_write, True),
    ("no-decay", _no_decay, True),
    ("one-hot-overwrite", _one_hot_overwrite, True),
]


@pytest.mark.parametrize("case,edit,warm", DEGENERATE, ids=[c[0] for c in DEGENERATE])
@pytest.mark.parametrize("kind,kw,mode", [
    (L.UNIFORM, dict(bits=4), "rtn"), (L.HAD_INT8, dict(block=128), "rtn"), (L.MIXED, dict(block=32, k_hi=16), "rtn"),
    (L.BITALLOC, {}, "rtn"), (L.MIXED, dict(block=32, k_hi=16), "ef"), (L.BITALLOC, {}, "sr"),
], ids=["uniform4-rtn", "had128-rtn", "mixed-rtn", "bitalloc-rtn", "mixed-ef", "bitalloc-sr"])
def test_decode_degenerate_inputs(case, edit, warm, kind, kw, mode):
    lay = _layout(kind, mode, 2, 2, 128, **kw)
    run_decode(lay, 3, warm=warm, edit=edit, seed=11)


# ---------------------------------------------------------------------------- allocation pass


def _alloc_case(case, rng, B, H, dk):
    """(state, s) for an allocation case. "warm": rows of very different ranges;
    "groups": three groups of identical rows (magnitudes 1, 1e-2, 1e-5) with one decay,
    so that clipping forces over a hundred one-bit moves per head that end inside a group of
    exactly tied rows; "spread": row magnitudes and decays both spread over several
    decades (many rows clipped at both ends)."""
    if case == "warm":
        S = _warm_state(rng, B, H, dk, dk)
        s = np.exp(rng.uniform(np.log(1e-3), 0.0, (B, H, dk))).astype(np.float32)
    elif case == "groups":
        base = rng.standard_normal((B, H, 1, dk)).astype(np.float32)
        mag = np.array([1.0, 1e-2, 1e-5], np.float32)[np.arange(dk) % 3]
        S = np.ascontiguousarray(np.broadcast_to(base, (B, H, dk, dk)) * mag[None, None, :, None])
        s = np.full((B, H, dk), 0.05, np.float32)
    else:
        S = (rng.standard_normal((B, H, dk, dk)) * np.exp(rng.uniform(-8.0, 2.0, (B, H, dk, 1)))).astype(np.float32)
        s = np.exp(rng.uniform(np.log(1e-4), np.log(2.0), (B, H, dk))).astype(np.float32)
    return S, s


def _check_alloc_head(lay, reg_gpu, reg_orc, alloc, tag, reg_in):
    """Widths equal except near-ties of the real widths (b* within 1e-5 of a .5 boundary,
    the budget kept); fit indices equal except near-equal fit errors; then, for every row
    and whatever the widths and fits agreed on, the GPU's Delta against the oracle's step
    for the GPU's width and fit (equal, or the adjacent float16 within 1e-6 of a
    midpoint), and the GPU's codes against the oracle's rounding of the stored values Y
    on the GPU's grid (equal, or one step apart within 1e-5 of a step of a boundary).
    When every choice agrees the repacked bytes must also be equal."""
    from oracle.numerics import f16_bits
    from oracle.quantizers import levels_n, one_bit_round, one_bit_step, row_step, sym_round
    from tests.parity import _meta_ok
    g = L.decode_region(lay, reg_gpu)
    o = L.decode_region(lay, reg_orc)
    assert g.widths.sum() == lay.bbar * lay.dk, tag
    bad_w = np.argwhere(g.widths != o.widths).ravel()
    if bad_w.size:
        frac = np.abs(alloc["bstar"][bad_w] - np.floor(alloc["bstar"][bad_w]) - 0.5)
        assert np.all(frac < 1e-5), (tag, bad_w, alloc["bstar"][bad_w])
    same_w = g.widths == o.widths
    for i in np.argwhere(same_w & (g.fit != o.fit)).ravel():
        e = alloc["fit_err"][i]
        assert abs(e[g.fit[i]] - e[o.fit[i]]) <= 1e-6 * max(e[o.fit[i]], 1e-300), (tag, i)
    if bad_w.size == 0 and np.array_equal(g.fit, o.fit):
        assert np.array_equal(reg_gpu, reg_orc), tag
        return
    # re-round every row of the stored values with the GPU's widths and fits
    Y = L.stored_values(lay, L.decode_region(lay, reg_in))
    tally = Tally()
    for i in range(lay.dk):
        b = int(g.widths[i])
        if b == 1:
            d, pre = one_bit_step(Y[i])
        else:
            d, pre = row_step(float(alloc["R"][i]), b, int(g.fit[i]))
        _meta_ok(g.delta_bits[i:i + 1], f16_bits(np.array([d])), np.array([pre]), tally, (tag, "delta", i))
        if g.delta_bits[i] != f16_bits(np.array([d]))[0]:
            continue
        rr = one_bit_round(Y[i], d, "rtn") if b == 1 else sym_round(Y[i], d, levels_n(b), "rtn")
        diff = g.kappa[i] != rr.kappa
        tally.elems += lay.dv
        if diff.any():
            tally.mismatch += int(diff.sum())
            ok = ~diff | ((np.abs(g.kappa[i] - rr.kappa) == 1) & (rr.boundary <= 1e-5))
            if not ok.all():
                tally.bad.append((tag, "codes", i, np.argwhere(~ok).ravel()[:3].tolist()))
    assert tally.ok(), (tag, tally.summary())


@pytest.mark.parametrize("case", ["warm", "groups", "spread"])
def test_allocate_bits_matches_oracle(case):
    """Two allocation passes per head: the first from the imported state (every row at
    the mean width), the second, with the decays reversed across rows, from the mixed
    widths the first one left (rows stored with 2 to 8 bits)."""
    print(f"\n[case] allocate_bits {case} B=2 H=4", flush=True)
    B, H, dk = 2, 4, 128
    lay = _layout(L.BITALLOC, "rtn", B, H, dk)
    rng = np.random.default_rng(31)
    st = _state(lay)
    S, s = _alloc_case(case, rng, B, H, dk)
    st.quantize(_to_dev(S))
    r = np.full((B, H, dk), 1.0 / (3 * dk), dtype=np.float32)
    moved = 0
    wide_rows = 0
    for pas, s_pass in enumerate((s, np.ascontiguousarray(s[..., ::-1]))):
        torch.cuda.synchronize()
        before = st.regions().cpu().numpy()
        st.allocate_bits(_to_dev(s_pass), _to_dev(r))
        torch.cuda.synchronize()
        after = st.regions().cpu().numpy()
        for b in range(B):
            for h in range(H):
                reg_in = before[b * H + h][: lay.region_size()]
                reg_gpu = after[b * H + h][: lay.region_size()]
                reg_orc, alloc = allocate_region(lay, reg_in, s_pass[b, h].astype(np.float64),
                                                 r[b, h].astype(np.float64))
                if pas == 1:
                    wide_rows += int((L.decode_region(lay, reg_in).widths >= 6).sum())
                moved += int(np.abs(np.clip(np.rint(alloc["bstar"]), lay.bmin, lay.bmax)
                                    - L.decode_region(lay, reg_orc).widths).sum())
                _check_alloc_head(lay, reg_gpu, reg_orc, alloc, (pas, b, h), reg_in)
    print(f"[alloc] one-bit moves over the heads: {moved}; rows stored with 6+ bits before the second pass: "
          f"{wide_rows}", flush=True)
    if case != "warm":
        assert moved >= 50 * B * H
    assert wide_rows > 0


@pytest.mark.parametrize("mode,per_row", [("rtn", True), ("sr", True), ("rtn", False)])
def test_online_estimators_and_allocation_from_them(mode, per_row):
    """Span-64 estimators folded in by every decode step (a decay stream that varies per
    token) against the oracle's recursion; then allocation passes that take s and r
    from them under each persistence factor, against the oracle fed the GPU's
    estimator values; a head whose estimators saw no token allocates by range alone."""
    from oracle.estimators import ema_estimates, ema_fold, ema_init
    print(f"\n[case] online estimators BITALLOC {mode} per_row={per_row}", flush=True)
    B, H, dk, T = 2, 3, 128, 40
    lay = _layout(L.BITALLOC, mode, B, H, dk, per_row=per_row)
    rng = np.random.default_rng(52)
    st = _state(lay)
    inp = decode_inputs(52, B, H, dk, dk, T, per_row)
    dev = {key: _to_dev(val) for key, val in inp.items()}
    st.quantize(_to_dev(_warm_state(rng, B, H, dk, dk)))
    o = torch.zeros((B, H, dk), dtype=torch.float32, device="cuda")
    # the state never saw a token: every row gets the same factor
    est = torch.zeros((B, H, 2 * dk + 4), dtype=torch.float32, device="cuda")
    st.set_estimators(est)
    before = st.regions().cpu().numpy()
    st.allocate_bits(None)
    torch.cuda.synchronize()
    after = st.regions().cpu().numpy()
    for b in range(B):
        for h in range(H):
            reg_in = before[b * H + h][: lay.region_size()]
            reg_orc, alloc = allocate_region(lay, reg_in, None, None)
            _check_alloc_head(lay, after[b * H + h][: lay.region_size()], reg_orc, alloc, ("flat", b, h), reg_in)
    jit = np.exp(0.4 * rng.standard_normal((T,) + inp["s"].shape)).astype(np.float32)
    s_t = (inp["s"][None] * jit).astype(np.float32)
    orc = {(b, h): ema_init(dk) for b in range(B) for h in range(H)}
    for t in range(T):
        st.step_decode(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], _to_dev(s_t[t]), o, t)
        for b in range(B):
            for h in range(H):
                srow = s_t[t, b, h] if per_row else np.full(dk, s_t[t, b, h])
                orc[(b, h)] = ema_fold(orc[(b, h)], srow.astype(np.float64), float(inp["beta"][t, b, h]),
                                       inp["k"][t, b, h].astype(np.float64))
    torch.cuda.synchronize()
    e = est.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ob = orc[(b, h)]
            for got, want in ((e[b, h, :dk], ob.Na), (e[b, h, dk:2 * dk], ob.Nr), (e[b, h, 2 * dk], ob.W)):
                err = np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30))
                worst = max(worst, float(err))
    print(f"[est] worst relative error of the estimators after {T} tokens: {worst:.2e}", flush=True)
    assert worst < 2e-5
    st.set_estimators(None)
    st.set_estimators(est)
    for factor, C in (("erasure", 1), ("w1", 1), ("hC", 64), ("hC", 4)):
        torch.cuda.synchronize()
        before = st.regions().cpu().numpy()
        st.allocate_bits(None, factor=factor, C=C)
        torch.cuda.synchronize()
        after = st.regions().cpu().numpy()
        for b in range(B):
            for h in range(H):
                sh, r = ema_estimates(e[b, h, :dk], e[b, h, dk:2 * dk], float(e[b, h, 2 * dk]))
                reg_in = before[b * H + h][: lay.region_size()]
                reg_orc, alloc = allocate_region(lay, reg_in, sh, r, factor, C)
                _check_alloc_head(lay, after[b * H + h][: lay.region_size()], reg_orc, alloc, (factor, C, b, h), reg_in)
    # explicit decays with the alternative factors
    s_np = inp["s"] if per_row else np.repeat(inp["s"][..., None], dk, axis=-1).astype(np.float32)
    for factor, C in (("w1", 1), ("hC", 16)):
        torch.cuda.synchronize()
        before = st.regions().cpu().numpy()
        st.allocate_bits(_to_dev(np.ascontiguousarray(s_np[..., ::-1])), factor=factor, C=C)
        torch.cuda.synchronize()
        after = st.regions().cpu().numpy()
        for b in range(B):
            for h in range(H):
                reg_in = before[b * H + h][: lay.region_size()]
                reg_orc, alloc = allocate_region(lay, reg_in, s_np[b, h, ::-1].astype(np.float64),
                                                 np.full(dk, 1.0 / (3 * dk)), factor, C)
                _check_alloc_head(lay, after[b * H + h][: lay.region_size()], reg_orc, alloc, (factor, C, b, h), reg_in)


@pytest.mark.parametrize("case", ["est-erasure", "est-hC64", "decays-w1", "per-head-est", "one-bit-floor"])
def test_decode_step_with_allocation(case):
    """Decode tokens whose write-back allocates (teacher-forced: each token starts from
    the GPU's stored region and estimators) against the oracle's plain step, allocation
    on the updated state and single rounding; readout within 1e-4 relative."""
    from oracle.estimators import EmaState, ema_estimates, ema_fold
    from oracle.step import decode_step_alloc
    from tests.parity import O_REL, Tally, compare_alloc_write_back
    print(f"\n[case] decode step with allocation {case}", flush=True)
    B, H, dk, T = 2, 3, 128, 5
    per_row = case != "per-head-est"
    use_est = case != "decays-w1"
    factor, C = {"est-erasure": ("erasure", 1), "est-hC64": ("hC", 64), "decays-w1": ("w1", 1),
                 "per-head-est": ("erasure", 1), "one-bit-floor": ("erasure", 1)}[case]
    kw = dict(bbar=3, bmin=1) if case == "one-bit-floor" else {}
    lay = _layout(L.BITALLOC, "rtn", B, H, dk, per_row=per_row, **kw)
    rng = np.random.default_rng(61)
    st = _state(lay)
    inp = decode_inputs(61, B, H, dk, dk, T, per_row)
    dev = {key: _to_dev(val) for key, val in inp.items()}
    st.quantize(_to_dev(_warm_state(rng, B, H, dk, dk)))
    o = torch.zeros((B, H, dk), dtype=torch.float32, device="cuda")
    est = None
    if use_est:
        est = torch.zeros((B, H, 2 * dk + 4), dtype=torch.float32, device="cuda")
        # a few ordinary tokens first, so that the estimators hold a history
        st.set_estimators(est)
        for t in range(3):
            st.step_decode(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], dev["s"], o, t)
    tally = Tally()
    skipped = 0
    for t in range(T):
        torch.cuda.synchronize()
        regs_in = st.regions().cpu().numpy()
        e_in = est.cpu().numpy().astype(np.float64) if use_est else None
        st.step_decode_alloc(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], dev["s"], o, t, factor, C)
        torch.cuda.synchronize()
        regs = st.regions().cpu().numpy()
        o_np = o.cpu().numpy()
        e_out = est.cpu().numpy().astype(np.float64) if use_est else None
        for b in range(B):
            for h in range(H):
                s_bh = inp["s"][b, h].astype(np.float64)
                s_rows = s_bh if per_row else np.full(dk, float(s_bh))
                beta = float(inp["beta"][t, b, h])
                if use_est:
                    es = EmaState(Na=e_in[b, h, :dk], Nr=e_in[b, h, dk:2 * dk], W=float(e_in[b, h, 2 * dk]))
                    es = ema_fold(es, s_rows, beta, inp["k"][t, b, h].astype(np.float64))
                    for got, want in ((e_out[b, h, :dk], es.Na), (e_out[b, h, dk:2 * dk], es.Nr)):
                        assert np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30)) < 1e-5
                    sa, ra = ema_estimates(es.Na, es.Nr, es.W)
                else:
                    sa, ra = s_rows, np.full(dk, 1.0 / (3 * dk))
                reg_orc, alloc, o_orc, X = decode_step_alloc(
                    lay, regs_in[b * H + h], inp["q"][t, b, h], inp["k"][t, b, h], inp["v"][t, b, h], beta,
                    s_bh, sa, ra, factor, C)
                skipped += compare_alloc_write_back(lay, regs[b * H + h], reg_orc, alloc, X, tally, (t, b, h))
                err = np.linalg.norm(o_np[b, h] - o_orc) / max(np.linalg.norm(o_orc), 1e-30)
                tally.o_worst = max(tally.o_worst, float(err))
    print("[tally]", tally.summary(), "rows left out of the code comparison:", skipped, flush=True)
    assert tally.ok(), tally.summary()
    assert skipped <= 0.01 * T * B * H * dk


@pytest.mark.parametrize("case", ["layer-rtn", "layer-sr", "head-sr", "layer-sr-one-bit", "layer-rtn-decays-hC"])
def test_decode_step_with_allocation_layer_budget_and_sr(case):
    """Allocating decode tokens at the layer-wise budget and/or with stochastic rounding
    (teacher-forced from the GPU's stored regions and estimators) against the oracle:
    each head's plain step, the widths over the sequence's H updated states (layer) or
    the head's own (head), and one rounding by the layout's rule with the draws of the
    token. Readout within 1e-4 relative; widths per sequence within the proxy-cost
    tolerance; codes to the decode bound."""
    from oracle.estimators import EmaState, ema_estimates, ema_fold
    from oracle.step import decode_step_alloc, decode_step_alloc_layer
    from oracle.philox import sr_draws
    from tests.parity import Tally, compare_alloc_write_back, compare_layer_widths
    print(f"\n[case] decode step with allocation {case}", flush=True)
    B, H, dk, T = 2, 4, 128, 4
    layer = case.startswith("layer")
    mode = "sr" if "-sr" in case else "rtn"
    use_est = "decays" not in case
    factor, C = ("hC", 64) if "hC" in case else ("erasure", 1)
    kw = dict(bbar=3, bmin=1) if "one-bit" in case else {}
    lay = _layout(L.BITALLOC, mode, B, H, dk, budget="layer" if layer else "head", **kw)
    rng = np.random.default_rng(67)
    st = _state(lay)
    inp = decode_inputs(67, B, H, dk, dk, T + 2, True)
    dev = {key: _to_dev(val) for key, val in inp.items()}
    S0 = _warm_state(rng, B, H, dk, dk) * np.exp(rng.uniform(-1.5, 1.5, (B, H, 1, 1))).astype(np.float32)
    st.quantize(_to_dev(S0))
    o = torch.zeros((B, H, dk), dtype=torch.float32, device="cuda")
    est = None
    if use_est:
        est = torch.zeros((B, H, 2 * dk + 4), dtype=torch.float32, device="cuda")
        st.set_estimators(est)
        for t in range(2):
            st.step_decode(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], dev["s"], o, t)
    tally = Tally()
    skipped = 0
    for t in range(2, T + 2):
        torch.cuda.synchronize()
        regs_in = st.regions().cpu().numpy()
        e_in = est.cpu().numpy().astype(np.float64) if use_est else None
        st.step_decode_alloc(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], dev["s"], o, t, factor, C)
        torch.cuda.synchronize()
        regs = st.regions().cpu().numpy()
        o_np = o.cpu().numpy()
        for b in range(B):
            sa_h, ra_h = [], []
            for h in range(H):
                s_rows = inp["s"][b, h].astype(np.float64)
                if use_est:
                    es = EmaState(Na=e_in[b, h, :dk], Nr=e_in[b, h, dk:2 * dk], W=float(e_in[b, h, 2 * dk]))
                    es = ema_fold(es, s_rows, float(inp["beta"][t, b, h]), inp["k"][t, b, h].astype(np.float64))
                    sa, ra = ema_estimates(es.Na, es.Nr, es.W)
                else:
                    sa, ra = s_rows, np.full(dk, 1.0 / (3 * dk))
                sa_h.append(sa)
                ra_h.append(ra)
            args = [[inp[n][t, b, h] for h in range(H)] for n in ("q", "k", "v")]
            betas = [float(inp["beta"][t, b, h]) for h in range(H)]
            ss = [inp["s"][b, h].astype(np.float64) for h in range(H)]
            rin = [regs_in[b * H + h] for h in range(H)]
            if layer:
                regs_o, allocs, outs, Xs = decode_step_alloc_layer(lay, rin, *args, betas, ss, sa_h, ra_h, factor,
                                                                   C, t, b)
                compare_layer_widths(lay, [regs[b * H + h] for h in range(H)], allocs, tally, (t, b))
            else:
                res = [decode_step_alloc(lay, rin[h], args[0][h], args[1][h], args[2][h], betas[h], ss[h],
                                         sa_h[h], ra_h[h], factor, C, t, b, h) for h in range(H)]
                regs_o, allocs, outs, Xs = (list(x) for x in zip(*res))
            for h in range(H):
                draws = None
                if mode == "sr":
                    draws = (lambda bb, hh: (lambda i: np.asarray(sr_draws(lay.seed, bb, hh, H, t, int(i), dk),
                                                                  np.float64)))(b, h)
                skipped += compare_alloc_write_back(lay, regs[b * H + h], regs_o[h], allocs[h], Xs[h], tally,
                                                    (t, b, h), draws=draws, layer=layer)
                err = np.linalg.norm(o_np[b, h] - outs[h]) / max(np.linalg.norm(outs[h]), 1e-30)
                tally.o_worst = max(tally.o_worst, float(err))
    print("[tally]", tally.summary(), "rows left out of the code comparison:", skipped, flush=True)
    assert tally.ok(), tally.summary()
    assert skipped <= 0.01 * T * B * H * dk


@pytest.mark.parametrize("case", ["warm", "spread"])
def test_allocate_bits_layer_budget_matches_oracle(case):
    """The layer-wise allocation (costs per head, widths over every row of a sequence,
    fits and repack per head) against the oracle on two passes, the second with the
    decays reversed across rows and the states of half the heads scaled down, from the
    widths the first pass left; whole regions compared (the code area is zero after
    each head's last row)."""
    from oracle.step import allocate_layer_regions
    print(f"\n[case] allocate_bits layer budget {case} B=2 H=8", flush=True)
    B, H, dk = 2, 8, 128
    lay = _layout(L.BITALLOC, "rtn", B, H, dk, budget="layer")
    rng = np.random.default_rng(37)
    st = _state(lay)
    S, s = _alloc_case(case, rng, B, H, dk)
    # heads of a sequence differ: decays shifted per head
    s = (s * np.exp(rng.uniform(-2.0, 1.0, (B, H, 1)))).astype(np.float32)
    st.quantize(_to_dev(S))
    r = np.full((B, H, dk), 1.0 / (3 * dk), dtype=np.float32)
    spread = 0
    for pas, s_pass in enumerate((s, np.ascontiguousarray(s[..., ::-1]))):
        if pas == 1:
            torch.cuda.synchronize()
            out = torch.zeros((B, H, dk, dk), dtype=torch.float32, device="cuda")
            st.dequant(out)
            out[:, ::2] *= 0.01
            st.quantize(out.contiguous())
        torch.cuda.synchronize()
        before = st.regions().cpu().numpy()
        st.allocate_bits(_to_dev(s_pass), _to_dev(r))
        torch.cuda.synchronize()
        after = st.regions().cpu().numpy()
        for b in range(B):
            regs_in = [before[b * H + h][: lay.region_size()] for h in range(H)]
            orc, allocs = allocate_layer_regions(lay, regs_in, [s_pass[b, h].astype(np.float64) for h in range(H)],
                                                 [r[b, h].astype(np.float64) for h in range(H)])
            g_w = [L.decode_region(lay, after[b * H + h][: lay.region_size()]).widths for h in range(H)]
            assert sum(int(w.sum()) for w in g_w) == lay.bbar * H * dk
            sums = [int(w.sum()) for w in g_w]
            spread = max(spread, max(sums) - min(sums))
            for h in range(H):
                reg_gpu = after[b * H + h][: lay.region_size()]
                o_w = allocs[h]["widths"]
                if not np.array_equal(g_w[h], o_w):
                    bad = np.argwhere(g_w[h] != o_w).ravel()
                    frac = np.abs(allocs[h]["bstar"][bad] - np.floor(allocs[h]["bstar"][bad]) - 0.5)
                    assert np.all(frac < 1e-5), (pas, b, h, bad, allocs[h]["bstar"][bad])
                    continue
                g = L.decode_region(lay, reg_gpu)
                o = L.decode_region(lay, orc[h])
                if not np.array_equal(g.fit, o.fit):
                    for i in np.argwhere(g.fit != o.fit).ravel():
                        e = allocs[h]["fit_err"][i]
                        assert abs(e[g.fit[i]] - e[o.fit[i]]) <= 1e-6 * max(e[o.fit[i]], 1e-300), (pas, b, h, i)
                    continue
                assert np.array_equal(reg_gpu, orc[h]), (pas, b, h)
    print(f"[alloc-layer] largest difference of head bit totals within a sequence: {spread}", flush=True)
    assert spread > 0


@pytest.mark.parametrize("per_row", [False, True])
def test_headalloc_allocation_matches_oracle_and_decode_after(per_row):
    """The per-head unit: widths over the heads of each sequence from the summed row
    factors, group fits and repack against the oracle on two passes (the second with the
    decays permuted across heads), whole regions compared; then decode steps on the
    heads of different widths."""
    from oracle.step import allocate_headalloc_regions
    print(f"\n[case] headalloc allocation per_row={per_row} B=2 H=8", flush=True)
    B, H, dk = 2, 8, 128
    lay = _layout(L.HEADALLOC, "rtn", B, H, dk, per_row=per_row)
    rng = np.random.default_rng(43)
    st = _state(lay)
    st.quantize(_to_dev(_warm_state(rng, B, H, dk, dk)))
    s_head = np.exp(rng.uniform(np.log(1e-3), 0.0, (B, H)))
    s = np.repeat(s_head[..., None], dk, axis=-1)
    if per_row:
        s = s * np.exp(rng.uniform(-1.0, 1.0, (B, H, dk)))
    s = s.astype(np.float32)
    r = np.full((B, H, dk), 1.0 / (3 * dk), dtype=np.float32)
    spread = 0
    for pas, s_pass in enumerate((s, np.ascontiguousarray(s[:, ::-1]))):
        torch.cuda.synchronize()
        before = st.regions().cpu().numpy()
        st.allocate_bits(_to_dev(s_pass), _to_dev(r))
        torch.cuda.synchronize()
        after = st.regions().cpu().numpy()
        for b in range(B):
            regs_in = [before[b * H + h][: lay.region_size()] for h in range(H)]
            orc, al = allocate_headalloc_regions(lay, regs_in, [s_pass[b, h].astype(np.float64) for h in range(H)],
                                                 [r[b, h].astype(np.float64) for h in range(H)])
            gw = np.array([L.decode_region(lay, after[b * H + h][: lay.region_size()]).width for h in range(H)])
            assert gw.sum() == lay.bbar * H
            spread = max(spread, int(gw.max() - gw.min()))
            if not np.array_equal(gw, al["widths"]):
                bad = np.argwhere(gw != al["widths"]).ravel()
                frac = np.abs(al["bstar"][bad] - np.floor(al["bstar"][bad]) - 0.5)
                assert np.all(frac < 1e-5), (pas, b, bad, al["bstar"][bad])
                continue
            for h in range(H):
                reg_gpu = after[b * H + h][: lay.region_size()]
                g = L.decode_region(lay, reg_gpu)
                if not np.array_equal(g.fit, al["fit"][h]):
                    for gi in np.argwhere(g.fit != al["fit"][h]):
                        e = al["fit_err"][h][gi[0], gi[1]]
                        gf, of = g.fit[gi[0], gi[1]], al["fit"][h][gi[0], gi[1]]
                        assert abs(e[gf] - e[of]) <= 1e-6 * max(e[of], 1e-300), (pas, b, h, gi)
                    continue
                assert np.array_equal(reg_gpu, orc[h]), (pas, b, h)
    print(f"[headalloc] largest width difference between heads of a sequence: {spread}", flush=True)
    assert spread >= 2
    run_decode(lay, 4, warm=False, seed=44, state=st)


@pytest.mark.parametrize("unit", ["layer", "headalloc"])
def test_allocation_from_estimators_layer_and_head_units(unit):
    """The layer-budget and per-head allocations taking s and r from the online
    estimators (folded in by the decode steps, here through the generic kernel), against
    the oracle fed the GPU's estimator values."""
    from oracle.estimators import ema_estimates
    from oracle.step import allocate_headalloc_regions, allocate_layer_regions
    print(f"\n[case] allocation from estimators: {unit}", flush=True)
    B, H, dk, T = 2, 4, 128, 12
    kind, kw = (L.BITALLOC, dict(budget="layer")) if unit == "layer" else (L.HEADALLOC, {})
    lay = _layout(kind, "rtn", B, H, dk, **kw)
    rng = np.random.default_rng(71)
    st = _state(lay)
    inp = decode_inputs(71, B, H, dk, dk, T, True)
    dev = {key: _to_dev(val) for key, val in inp.items()}
    st.quantize(_to_dev(_warm_state(rng, B, H, dk, dk)))
    est = torch.zeros((B, H, 2 * dk + 4), dtype=torch.float32, device="cuda")
    st.set_estimators(est)
    o = torch.zeros((B, H, dk), dtype=torch.float32, device="cuda")
    # per-head decay shifts so that heads differ
    s_t = (inp["s"] * np.exp(rng.uniform(-1.5, 1.5, (B, H, 1)))).astype(np.float32)
    for t in range(T):
        st.step_decode(dev["q"][t], dev["k"][t], dev["v"][t], dev["beta"][t], _to_dev(s_t), o, t)
    torch.cuda.synchronize()
    e = est.cpu().numpy().astype(np.float64)
    before = st.regions().cpu().numpy()
    st.allocate_bits(None, factor="hC", C=16)
    torch.cuda.synchronize()
    after = st.regions().cpu().numpy()
    for b in range(B):
        sr = [ema_estimates(e[b, h, :dk], e[b, h, dk:2 * dk], float(e[b, h, 2 * dk])) for h in range(H)]
        regs_in = [before[b * H + h][: lay.region_size()] for h in range(H)]
        if unit == "layer":
            orc, al = allocate_layer_regions(lay, regs_in, [x[0] for x in sr], [x[1] for x in sr], "hC", 16)
            widths_o = [a["widths"] for a in al]
            bstar = np.concatenate([a["bstar"] for a in al])
            gw = [L.decode_region(lay, after[b * H + h][: lay.region_size()]).widths for h in range(H)]
        else:
            orc, al = allocate_headalloc_regions(lay, regs_in, [x[0] for x in sr], [x[1] for x in sr], "hC", 16)
            widths_o = [np.array([w]) for w in al["widths"]]
            bstar = al["bstar"]
            gw = [np.array([L.decode_region(lay, after[b * H + h][: lay.region_size()]).width]) for h in range(H)]
        go, oo = np.concatenate(gw), np.concatenate(widths_o)
        if not np.array_equal(go, oo):
            bad = np.argwhere(go != oo).ravel()
            assert np.all(np.abs(bstar[bad] - np.floor(bstar[bad]) - 0.5) < 1e-5), (b, bad)
            continue
        for h in range(H):
            reg_gpu = after[b * H + h][: lay.region_size()]
            g = L.decode_region(lay, reg_gpu)
            o_fit = al[h]["fit"] if unit == "layer" else al["fit"][h]
            if not np.array_equal(g.fit, o_fit):
                # only fits whose squared errors tie within 1e-6 may differ
                for idx in np.argwhere(g.fit != o_fit):
                    idx = tuple(idx)
                    e = al[h]["fit_err"][idx] if unit == "layer" else al["fit_err"][h][idx]
                    assert abs(e[g.fit[idx]] - e[o_fit[idx]]) <= 1e-6 * max(e[o_fit[idx]], 1e-300), (b, h, idx)
                continue
            assert np.array_equal(reg_gpu, orc[h]), (b, h)


def test_allocation_then_decode_full_budget_zero_state():
    # a zero state keeps every row at the mean width
    lay = _layout(L.BITALLOC, "rtn", 1, 2, 128)
    st = _state(lay)
    s = _to_dev(np.full((1, 2, 128), 0.01, np.float32))
    st.allocate_bits(s)
    torch.cuda.synchronize()
    regs = st.regions().cpu().numpy()
    for h in range(2):
        c = L.decode_region(lay, regs[h][: lay.region_size()])
        assert np.all(c.widths == 4) and np.all(c.kappa == 0)


# ---------------------------------------------------------------------------- DAMP selection


def test_damp_select_matches_oracle():
    print("\n[case] damp_select N=6 H=3", flush=True)
    wb = _wb()
    rng = np.random.default_rng(41)
    N, H, dk = 6, 3, 128
    samples = (rng.standard_normal((N, H, dk, dk)) * np.exp(rng.uniform(-3, 1, (1, H, dk, 1)))).astype(np.float32)
    s = np.exp(rng.uniform(np.log(1e-3), 0, (H, dk))).astype(np.float32)
    perm, cost = wb.damp_select(_to_dev(samples), _to_dev(s), k_hi=16, block=32, tau=0.01)
    torch.cuda.synchronize()
    perm = perm.cpu().numpy()
    cost = cost.cpu().numpy()
    for h in range(H):
        E, P, C = risk_scores(samples[:, h].astype(np.float64), s[h].astype(np.float64), 0.01, 32)
        assert np.allclose(cost[h], C, rtol=1e-5)
        ref = select_permutation(C, 16)
        if not np.array_equal(perm[h], ref):
            # only rows whose costs tie to 1e-6 at the selection boundary may swap
            thr = np.sort(C)[::-1][15]
            diff = set(perm[h][:16]) ^ set(ref[:16])
            assert all(abs(C[u] - thr) <= 1e-6 * thr for u in diff), h
        assert sorted(perm[h]) == list(range(dk))


# ---------------------------------------------------------------------------- full-size shapes


FULL = [
    ("gdn-had-int8", dict(kind=L.HAD_INT8, B=64, H=16, per_row=False, block=128), ["rtn"]),
    ("gdn-had-int4", dict(kind=L.HAD_INT8, B=64, H=16, per_row=False, block=128, int_bits=4), ["rtn"]),
    ("kda-mixed", dict(kind=L.MIXED, B=256, H=32, per_row=True, block=32, k_hi=16), ["rtn"]),
    ("kda-bitalloc", dict(kind=L.BITALLOC, B=256, H=32, per_row=True), ["rtn", "sr"]),
    ("kda-bitalloc-layer", dict(kind=L.BITALLOC, B=256, H=32, per_row=True, budget="layer"), ["rtn"]),
    ("kda-bitalloc-1bit", dict(kind=L.BITALLOC, B=256, H=32, per_row=True, bmin=1), ["rtn"]),
    ("gdn-headalloc", dict(kind=L.HEADALLOC, B=64, H=16, per_row=False), ["rtn"]),
]


@pytest.mark.parametrize("name,cfg,modes", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled_heads(name, cfg, modes):
    """The benchmark's launch configuration (all heads of a full layer per launch),
    checked on sampled heads over a few teacher-forced steps; BITALLOC after an
    allocation pass."""
    rng = np.random.default_rng(51)
    for mode in modes:
        c = dict(cfg)
        kind, B, H, per_row = c.pop("kind"), c.pop("B"), c.pop("H"), c.pop("per_row")
        lay = _layout(kind, mode, B, H, 128, per_row=per_row, **c)
        picks = sorted({(int(rng.integers(B)), int(rng.integers(H))) for _ in range(12)})
        run_decode(lay, 4, heads=picks, warm=True, seed=52, steps_checked={1, 3},
                   alloc_every=1 if kind == L.BITALLOC else None)
