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
