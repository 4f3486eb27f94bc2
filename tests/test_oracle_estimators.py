"""Pins of the online decay / erasure estimators and of the persistence factors
([LBRS] "State bit allocation", "Approximate erasure rate", "Choice of persistence
factor")."""
import numpy as np

from oracle.allocation import allocate_head
from oracle.estimators import SPAN, ema_alpha, ema_estimates, ema_fold, ema_init
from oracle.recurrence import GAMMA_ERASURE, GAMMA_HC, GAMMA_W1, persistence_factor


def _stream(rng, n, dk, per_row=True):
    s = np.exp(rng.uniform(np.log(1e-3), 0.0, size=(n, dk if per_row else 1))) * np.ones((n, dk))
    beta = rng.uniform(0.0, 1.0, size=n)
    k = rng.standard_normal((n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    return s, beta, k


def _run(s, beta, k):
    st = ema_init(s.shape[1])
    for t in range(len(beta)):
        st = ema_fold(st, s[t], beta[t], k[t])
    return st


def test_constant_stream_is_reproduced_from_the_first_token():
    rng = np.random.default_rng(1)
    dk = 16
    s0 = np.exp(rng.uniform(np.log(1e-3), 0.0, size=dk))
    k0 = rng.standard_normal(dk)
    for n in (1, 5, 300):
        st = _run(np.tile(s0, (n, 1)), np.full(n, 0.3), np.tile(k0, (n, 1)))
        sh, r = ema_estimates(st.Na, st.Nr, st.W)
        assert np.allclose(sh, s0, rtol=1e-11, atol=0)
        assert np.allclose(r, 0.5 * 0.3 * 1.7 * k0 ** 2, rtol=1e-12, atol=0)


def test_recursion_equals_the_weighted_average_definition():
    """The estimate after n tokens is the average of e^{2g} (not its complement) with
    weights (1 - alpha)^(n - t), normalised by their sum, then -1/2 log."""
    rng = np.random.default_rng(2)
    n, dk = 120, 8
    s, beta, k = _stream(rng, n, dk)
    st = _run(s, beta, k)
    sh, r = ema_estimates(st.Na, st.Nr, st.W)
    w = (1.0 - 2.0 / 65.0) ** (n - 1 - np.arange(n))
    ea = (w[:, None] * np.exp(-2.0 * s)).sum(0) / w.sum()
    er = (w[:, None] * (beta * (2 - beta))[:, None] * k ** 2).sum(0) / w.sum()
    assert np.allclose(sh, -0.5 * np.log(ea), rtol=1e-9)
    assert np.allclose(r, 0.5 * er, rtol=1e-12)
    assert st.n == n and np.isclose(st.W, w.sum() * 2.0 / 65.0, rtol=1e-13)


def test_span_convention():
    # span S: centre of mass of the weights (S - 1) / 2 tokens back
    a = ema_alpha(SPAN)
    ages = np.arange(20000)
    w = a * (1.0 - a) ** ages
    assert np.isclose((w * ages).sum() / w.sum(), (SPAN - 1) / 2.0, rtol=1e-9)


def test_no_token_means_no_estimate():
    st = ema_init(4)
    assert ema_estimates(st.Na, st.Nr, st.W) == (None, None)


def test_persistence_factor_identities():
    s = np.exp(np.linspace(np.log(1e-3), 0.0, 9))
    w1 = persistence_factor(s, None, GAMMA_W1)
    # w1 = (erasure rate without r) * e^{2s};  h^{(1)} = w1
    assert np.allclose(w1, persistence_factor(s, 0.0, GAMMA_ERASURE) * np.exp(2 * s), rtol=1e-10)
    assert np.allclose(persistence_factor(s, None, GAMMA_HC, 1), w1, rtol=1e-12)
    # h^{(C)}: the geometric series over write-backs sum_{l>=0} e^{-2 C s l}
    for C in (4, 64):
        L = np.arange(0, 200000)
        brute = np.array([np.exp(-2.0 * C * si * L).sum() for si in s])
        assert np.allclose(persistence_factor(s, None, GAMMA_HC, C), brute, rtol=1e-9)
    # erasure rate scales as 1/C
    assert np.allclose(persistence_factor(s, 0.01, GAMMA_ERASURE, 8) * 8, persistence_factor(s, 0.01), rtol=1e-14)


def _head(rng, dk=32, dv=16):
    R = np.exp(rng.uniform(-3, 0.5, size=dk))
    return rng.standard_normal((dk, dv)) * R[:, None]


def test_allocation_invariances_under_the_factor():
    rng = np.random.default_rng(5)
    Y = _head(rng)
    s_eq = np.full(32, 0.05)
    flat = allocate_head(Y, None, None)["widths"]
    for kind, C in ((GAMMA_ERASURE, 1), (GAMMA_ERASURE, 64), (GAMMA_W1, 1), (GAMMA_HC, 16)):
        # a factor that is the same for every row leaves range alone to decide
        assert np.array_equal(allocate_head(Y, s_eq, 0.01, factor=kind, C=C)["widths"], flat)
    s = np.exp(rng.uniform(np.log(1e-3), 0.0, size=32))
    # the erasure rate's 1/C cancels in c / GM(c)
    assert np.array_equal(allocate_head(Y, s, 0.01, C=1)["widths"], allocate_head(Y, s, 0.01, C=64)["widths"])
    # equal ranges: the cost is the factor, which never grows with s, and a row of larger
    # cost never gets fewer bits (rows of exactly equal cost -- h^{(64)} is 1.0 in
    # float64 for every s above about 0.3 -- are ordered by row index instead)
    Yeq = np.tile(np.linspace(-1, 1, 16), (32, 1))
    order = np.argsort(s)
    for kind, C in ((GAMMA_ERASURE, 1), (GAMMA_W1, 1), (GAMMA_HC, 64)):
        a = allocate_head(Yeq, s, 0.0 if kind != GAMMA_ERASURE else 0.01, factor=kind, C=C)
        b, c = a["widths"], a["c"]
        assert np.all(np.diff(c[order]) <= 0), kind
        assert all(b[i] >= b[j] for i in range(32) for j in range(32) if c[i] > c[j]), kind
        assert b.sum() == 4 * 32 and b.max() > b.min()


def test_infinite_factor_is_capped():
    rng = np.random.default_rng(6)
    Y = _head(rng)
    s = np.full(32, 0.1)
    s[3] = 0.0
    a = allocate_head(Y, s, 0.0)               # s + r = 0 on row 3: factor infinite
    assert np.all(np.isfinite(a["bstar"])) and a["widths"][3] == 8 and a["widths"].sum() == 128


def test_step_with_allocation_reduces_to_its_parts():
    """A token that changes nothing (beta = 0, s = 0) makes the allocating write-back the
    allocation pass; any token's readout is the plain step's; the grid and codes are
    the rounding of the updated state at the widths the allocation chose for it."""
    from oracle import layouts as L
    from oracle.quantizers import levels_n, sym_round
    from oracle.step import allocate_region, decode_step, decode_step_alloc, import_state
    rng = np.random.default_rng(8)
    dk = dv = 32
    lay = L.Layout(kind=L.BITALLOC, B=1, H=1, dk=dk, dv=dv, mode="rtn", per_row_decay=True, bbar=4, bmin=2, bmax=8)
    S = rng.standard_normal((dk, dv)) * np.exp(rng.uniform(-3, 0.5, (dk, 1)))
    s_rows = np.exp(rng.uniform(np.log(1e-3), 0.0, dk))
    # a stored state with mixed widths: the zero state at the mean width, S imported
    # into it, then one allocation pass
    start = L.encode_region(lay, L.Content(kappa=np.zeros((dk, dv), np.int64), widths=np.full(dk, 4),
                                           fit=np.zeros(dk, np.int64), delta_bits=np.zeros(dk, np.uint16)))
    reg0, _ = allocate_region(lay, import_state(lay, S, start), s_rows, 0.01)
    assert L.decode_region(lay, reg0).widths.max() > 4
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    q = rng.standard_normal(dk)
    q /= np.linalg.norm(q)
    v = rng.standard_normal(dv)
    reg_a, alloc_a, o_a, _ = decode_step_alloc(lay, reg0, q, k, v, 0.0, np.zeros(dk), s_rows, 0.01, "w1")
    reg_p, _ = allocate_region(lay, reg0, s_rows, 0.01, "w1")
    assert np.array_equal(reg_a, reg_p)
    reg_b, alloc_b, o_b, S_new = decode_step_alloc(lay, reg0, q, k, v, 0.7, s_rows, s_rows, 0.01)
    ref = decode_step(lay, reg0, None, q, k, v, 0.7, s_rows, 0, 0, 0)
    assert np.allclose(o_b, ref.o, rtol=1e-13, atol=1e-15) and np.allclose(S_new, ref.S_new, rtol=0, atol=0)
    c = L.decode_region(lay, reg_b)
    assert c.widths.sum() == 4 * dk and np.array_equal(c.widths, alloc_b["widths"])
    for i in range(dk):
        n = levels_n(int(c.widths[i]))
        assert np.array_equal(c.kappa[i], sym_round(S_new[i], float(c.delta[i]), n, "rtn").kappa)


def _alloc_case(rng, dk, dv, H, **kw):
    from oracle import layouts as L
    from oracle.step import allocate_layer_regions, import_state
    args = dict(kind=L.BITALLOC, B=1, H=H, dk=dk, dv=dv, per_row_decay=True, bbar=4, bmin=2, bmax=8,
                budget="layer")
    lay = L.Layout(**{**args, **kw})
    start = L.encode_region(lay, L.Content(kappa=np.zeros((dk, dv), np.int64), widths=np.full(dk, 4),
                                           fit=np.zeros(dk, np.int64), delta_bits=np.zeros(dk, np.uint16)))
    regs = [import_state(lay, rng.standard_normal((dk, dv)) * np.exp(rng.uniform(-3, 0.5, (dk, 1))) * 3.0 ** h,
                         start) for h in range(H)]
    s_rows = [np.exp(rng.uniform(np.log(1e-3), 0.0, dk)) for _ in range(H)]
    regs, _ = allocate_layer_regions(lay, regs, s_rows, [0.01] * H)
    unit = lambda x: x / np.linalg.norm(x)
    tok = dict(q=[unit(rng.standard_normal(dk)) for _ in range(H)], k=[unit(rng.standard_normal(dk)) for _ in range(H)],
               v=[rng.standard_normal(dv) for _ in range(H)], beta=[0.6] * H,
               s=[np.exp(rng.uniform(np.log(1e-3), 0.0, dk)) for _ in range(H)])
    return lay, regs, s_rows, tok


def test_layer_step_with_allocation_reduces_to_its_parts():
    """The allocating token under the layer-wise budget: each head's readout and updated
    state are the plain step's; the widths of the H updated states are the layer
    allocation of those states (sum = bbar H dk) and every head is rounded to nearest
    on its new grid; with one head it is the per-head allocating token, byte for byte."""
    from oracle import layouts as L
    from oracle.allocation import allocate_layer
    from oracle.quantizers import levels_n, one_bit_round, sym_round
    from oracle.step import decode_step, decode_step_alloc, decode_step_alloc_layer
    rng = np.random.default_rng(81)
    dk, dv, H = 32, 8, 3
    lay, regs, s_rows, tok = _alloc_case(rng, dk, dv, H, bmin=1)
    new, allocs, outs, Ss = decode_step_alloc_layer(lay, regs, tok["q"], tok["k"], tok["v"], tok["beta"], tok["s"],
                                                    s_rows, [0.01] * H)
    ref_w = allocate_layer(Ss, s_rows, [0.01] * H, 4, 1, 8)
    total = 0
    for h in range(H):
        ref = decode_step(lay, regs[h], None, tok["q"][h], tok["k"][h], tok["v"][h], 0.6, tok["s"][h], 0, 0, h)
        assert np.array_equal(Ss[h], ref.S_new) and np.allclose(outs[h], ref.o, rtol=1e-13, atol=1e-15)
        c = L.decode_region(lay, new[h])
        assert np.array_equal(c.widths, ref_w[h]["widths"]) and np.array_equal(c.fit, ref_w[h]["fit"])
        total += int(c.widths.sum())
        for i in range(dk):
            if c.widths[i] == 1:
                want = one_bit_round(Ss[h][i], float(c.delta[i]), "rtn").kappa
            else:
                want = sym_round(Ss[h][i], float(c.delta[i]), levels_n(int(c.widths[i])), "rtn").kappa
            assert np.array_equal(c.kappa[i], want)
    assert total == 4 * H * dk
    one, *_ = decode_step_alloc_layer(lay, regs[:1], tok["q"][:1], tok["k"][:1], tok["v"][:1], [0.6], tok["s"][:1],
                                      s_rows[:1], [0.01])
    head, *_ = decode_step_alloc(lay, regs[0], tok["q"][0], tok["k"][0], tok["v"][0], 0.6, tok["s"][0],
                                 s_rows[0], 0.01)
    assert np.array_equal(one[0], head)


def test_allocating_write_back_stochastic_rounding():
    """SR on the allocated grid: each level is the floor or the ceiling of x / Delta
    (clipped; one-bit rows: of (x + Delta) / (2 Delta)), the draws depend on the token
    (two tokens give different codes) and, away from the rails, the levels average to
    the value over many tokens (E[xhat] = x) within 5 sigma of the mean of N draws
    (sigma <= Delta / 2 per draw)."""
    from oracle import layouts as L
    from oracle.step import _round_at, decode_step_alloc_layer
    rng = np.random.default_rng(82)
    dk, dv, H, N = 32, 8, 2, 256
    lay, regs, s_rows, tok = _alloc_case(rng, dk, dv, H, bmin=1, mode="sr", seed=0x5EED)
    new, allocs, outs, Ss = decode_step_alloc_layer(lay, regs, tok["q"], tok["k"], tok["v"], tok["beta"], tok["s"],
                                                    s_rows, [0.01] * H, t=7, b=0)
    for h in range(H):
        c = L.decode_region(lay, new[h])
        assert np.any(c.widths == 1)
        d = c.delta.astype(np.float64)[:, None]
        one = (c.widths == 1)[:, None]
        n = np.where(c.widths == 1, 1, (1 << (c.widths - 1)) - 1)[:, None].astype(np.float64)
        tau = np.where(one, (Ss[h] + d) / (2 * d), Ss[h] / np.where(d == 0, 1, d))
        lev = np.where(one, (c.kappa + 1) // 2, c.kappa)
        lo = np.where(one, 0, np.maximum(np.floor(tau), -n))
        hi = np.where(one, 1, np.minimum(np.ceil(tau), n))
        lo = np.where(one, np.clip(np.floor(tau), 0, 1), lo)
        hi = np.where(one, np.clip(np.ceil(tau), 0, 1), hi)
        assert np.all((lev >= lo) & (lev <= hi))
        acc = np.zeros((dk, dv))
        for t in range(N):
            reg = _round_at(lay, Ss[h], allocs[h], "sr", t, 0, h)
            acc += L.stored_values(lay, L.decode_region(lay, reg))
            if t == 1:
                assert not np.array_equal(reg, _round_at(lay, Ss[h], allocs[h], "sr", 0, 0, h))
        inside = np.where(one, np.abs(Ss[h]) <= d, np.abs(Ss[h]) <= n * d) & (d > 0)
        err = np.abs(acc / N - Ss[h])
        bound = 5 * np.broadcast_to(np.where(one, 2 * d, d), err.shape) / (2 * np.sqrt(N))
        assert inside.sum() > 0.75 * dk * dv
        assert np.all(err[inside] <= bound[inside])


# ---------------------------------------------------------------- layer-wise budget

def _heads(rng, H, dk=16, dv=8):
    return [rng.standard_normal((dk, dv)) * np.exp(rng.uniform(-3, 0.5, (dk, 1))) for _ in range(H)]


def test_layer_budget_with_one_head_is_the_head_budget():
    from oracle.allocation import allocate_layer
    rng = np.random.default_rng(21)
    Y = _heads(rng, 1)
    s = np.exp(rng.uniform(np.log(1e-3), 0.0, 16))
    a = allocate_layer(Y, [s], [0.01])[0]
    b = allocate_head(Y[0], s, 0.01)
    assert np.array_equal(a["widths"], b["widths"]) and np.array_equal(a["fit"], b["fit"])


def test_layer_budget_identical_heads_and_decay_across_heads():
    from oracle.allocation import allocate_layer
    rng = np.random.default_rng(22)
    Y = _heads(rng, 1)[0]
    s = np.exp(rng.uniform(np.log(1e-3), 0.0, 16))
    per_head = allocate_head(Y, s, 0.01)["widths"]
    for a in allocate_layer([Y, Y, Y], [s, s, s], [0.01] * 3):
        assert np.array_equal(a["widths"], per_head)
    # equal ranges, head 1 decays faster on every row: head 0 takes bits from head 1
    a0, a1 = allocate_layer([Y, Y], [s, s + 1.0], [0.01, 0.01])
    assert a0["widths"].sum() > 4 * 16 > a1["widths"].sum()
    assert a0["widths"].sum() + a1["widths"].sum() == 2 * 4 * 16


def test_layer_budget_is_the_brute_force_optimum_on_tiny_layers():
    import itertools
    from oracle.allocation import allocate_layer, proxy_cost
    rng = np.random.default_rng(23)
    for _ in range(20):
        Y = _heads(rng, 2, dk=2, dv=4)
        s = [np.exp(rng.uniform(np.log(1e-3), 0.0, 2)) for _ in range(2)]
        al = allocate_layer(Y, s, [0.01, 0.01], bbar=4, bmin=2, bmax=8)
        b = np.concatenate([a["widths"] for a in al])
        c = np.concatenate([a["c"] for a in al])
        best = min(proxy_cost(c, np.array(w)) for w in itertools.product(range(2, 9), repeat=4) if sum(w) == 16)
        assert b.sum() == 16 and np.isclose(proxy_cost(c, b), best, rtol=1e-12)


def test_layer_budget_zero_heads():
    from oracle.allocation import allocate_layer
    rng = np.random.default_rng(24)
    Z = np.zeros((16, 8))
    s = np.full(16, 0.05)
    for a in allocate_layer([Z, Z], [s, s], [0.01, 0.01]):
        assert np.all(a["widths"] == 4)
    Y = _heads(rng, 1)[0]
    a0, a1 = allocate_layer([Y, Z], [s, s], [0.01, 0.01])
    assert np.all(a1["widths"] == 2) and a0["widths"].sum() == 2 * 4 * 16 - 2 * 16


def test_layer_capacity_region_round_trip():
    from oracle import layouts as L
    from oracle.allocation import allocate_layer
    from oracle.step import allocate_layer_regions
    rng = np.random.default_rng(25)
    dk, dv, H = 16, 16, 3
    lay = L.Layout(kind=L.BITALLOC, B=1, H=H, dk=dk, dv=dv, bbar=4, bmin=2, bmax=8, budget="layer")
    assert lay.region_size() == dk * dv + 3 * dk
    s = [np.exp(rng.uniform(np.log(1e-3), 0.0, dk)) for _ in range(H)]
    s[2] = s[2] + 1.0
    start = [L.initial_region(lay) for _ in range(H)]
    Ys = _heads(rng, H, dk, dv)
    from oracle.step import import_state
    regs = [import_state(lay, Ys[h], start[h]) for h in range(H)]
    new, allocs = allocate_layer_regions(lay, regs, s, [0.01] * H)
    used = []
    for h in range(H):
        c = L.decode_region(lay, new[h])
        assert np.array_equal(c.widths, allocs[h]["widths"])
        u = int(c.widths.sum()) * dv // 8
        used.append(u)
        assert np.all(new[h][u: lay.code_capacity] == 0)
        assert np.array_equal(L.encode_region(lay, c), new[h])
    assert sum(used) == H * dk * dv * 4 // 8 and used[2] < used[0]
