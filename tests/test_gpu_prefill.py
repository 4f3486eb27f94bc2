"""GPU parity of chunked prefill with deferred write-back against the token-by-token
oracle (same bfloat16 inputs, float64 recurrence, write-back after every C-th token and
after the last token; [LBRS] "Accumulated readout error", "Protocol").

Protocol for a call with several write-backs. The oracle runs its own trajectory from
the GPU's stored bytes at the start of the call and records, at each of its write-backs,
how close any decision came to flipping: the smallest distance of a pre-rounding value
to its rounding boundary (in steps; for float16 rows in float16 spacings) and of a
float16 scale / zero / step to its rounding midpoint (relative). The GPU runs the state
path in float64, so its values differ from the oracle's by ~1e-13 of a step; a decision
within GATE_CODE of a step (GATE_META relative) is one the two sides may take
differently, after which their trajectories may part legitimately. So, per head:
  * outputs of every token up to the first such write-back (all tokens if there is
    none) within O_REL relative L2 of the oracle's;
  * when the call has no such write-back, the stored region after the call held to the
    decode bound: metadata equal or the adjacent float16 within 1e-6 of a midpoint,
    codes equal except at most 1e-4 of them, one step apart and within 1e-5 of a step of
    the boundary.
The first gated write-back (if any) is reported. Calls of one write-back each are
teacher-forced from the GPU's bytes.
"""
import numpy as np
import pytest

from oracle import layouts as L
from oracle.step import prefill as oracle_prefill
from synth import bf16_to_f32, prefill_inputs
from tests.parity import Tally, compare_write_back

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

O_REL = 1e-4
GATE_CODE = 1e-9      # steps
GATE_META = 1e-12     # relative distance of a float16 pre-rounding value to its midpoint


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _f16_mid_dist(pre):
    """Relative distance of float64 values to the float16 rounding midpoint nearest them."""
    pre = np.asarray(pre, np.float64).ravel()
    if pre.size == 0:
        return np.array([np.inf])
    r = pre.astype(np.float16)
    rv = r.astype(np.float64)
    nb = np.where(rv <= pre, np.nextafter(r, np.float16(np.inf)), np.nextafter(r, np.float16(-np.inf)))
    mid = 0.5 * (rv + nb.astype(np.float64))
    ok = np.isfinite(mid)
    d = np.full(pre.shape, np.inf)
    d[ok] = np.abs(pre[ok] - mid[ok]) / np.maximum(np.abs(mid[ok]), 1e-300)
    return d


def _closest(wb):
    """(closest code decision in steps, closest metadata decision, relative) of one
    oracle write-back record."""
    code = float(np.min(wb.boundary)) if wb.boundary is not None else np.inf
    meta = np.inf
    if getattr(wb, "meta_pre", None):
        for v in wb.meta_pre.values():
            if v is not None and np.size(v):
                meta = min(meta, float(np.min(_f16_mid_dist(v))))
    return code, meta


def run_prefill(kind, T, C, calls=1, B=2, H=2, seed=3, per_row=True, chunk=64, **kw):
    import linear_attn_decode_amd as wb
    print(f"\n[case] prefill kind={kind} T={T} C={C} chunk={chunk} calls={calls} B={B} H={H} per_row={per_row}",
          flush=True)
    args = dict(kind=kind, B=B, H=H, dk=128, dv=128, mode="rtn", per_row_decay=per_row, block=32, k_hi=16)
    args.update(kw)
    lay = L.Layout(**args)
    rng = np.random.default_rng(seed)
    perm = np.stack([rng.permutation(128) for _ in range(H)]) if kind == L.MIXED else None
    st = wb.WriteBackState(kind, "rtn", B, H, 128, 128, per_row, bits=lay.bits, block=lay.block,
                           k_hi=lay.k_hi, perm=perm)
    S0 = (rng.standard_normal((B, H, 128, 128)) * np.exp(rng.uniform(-3, 0.5, (B, H, 128, 1)))).astype(np.float32)
    st.quantize(_dev(S0))
    inp = prefill_inputs(seed, B, H, 128, 128, T * calls, per_row)
    tally = Tally()
    o_worst = 0.0
    gated = []
    region_checked = 0
    for c in range(calls):
        sl = slice(c * T, (c + 1) * T)
        q, k, v = (_dev(inp[n][:, sl]) for n in ("q", "k", "v"))
        beta, s = _dev(inp["beta"][:, sl]), _dev(inp["s"][:, sl])
        o = torch.zeros((B, T, H, 128), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        reg_in = st.regions().cpu().numpy()
        st.prefill(q.view(torch.int16), k.view(torch.int16), v.view(torch.int16), beta, s, o, T, chunk, C, c * T)
        torch.cuda.synchronize()
        reg_out = st.regions().cpu().numpy()
        o_np = o.cpu().numpy()
        for bb in range(B):
            for hh in range(H):
                f = lambda n: bf16_to_f32(inp[n][bb, sl, hh]).astype(np.float64)
                recs = []
                reg, _, outs, last = oracle_prefill(lay, reg_in[bb * H + hh][: lay.region_size()], None, f("q"),
                                                    f("k"), f("v"), inp["beta"][bb, sl, hh], inp["s"][bb, sl, hh],
                                                    c * T, C, bb, hh, None if perm is None else perm[hh],
                                                    return_last=True, records=recs)
                # tokens up to and including the first write-back with a close decision
                upto = T
                for i, rec in recs:
                    cd, md = _closest(rec)
                    if cd <= GATE_CODE or md <= GATE_META:
                        upto = i + 1
                        gated.append((c, bb, hh, i, cd, md))
                        break
                got = o_np[bb, :upto, hh]
                ref = outs[:upto]
                rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
                o_worst = max(o_worst, rel)
                if upto == T:
                    region_checked += 1
                    compare_write_back(lay, reg_in[bb * H + hh], reg_out[bb * H + hh], last, None, None,
                                       c * T + T - 1, bb, hh, tally)
    tally.o_worst = o_worst
    print(f"[tally] {tally.summary()} regions_checked={region_checked}/{calls * B * H} "
          f"gated={gated[:4]}", flush=True)
    assert o_worst <= O_REL, o_worst
    assert tally.ok(), tally.summary()
    assert region_checked >= (calls * B * H) // 2, gated
    return tally


@pytest.mark.parametrize("kind", [L.FP32, L.UNIFORM, L.HAD_INT8, L.MIXED])
def test_prefill_one_write_back_per_call(kind):
    # T = C: one write-back per call, so every call is teacher-forced from the GPU bytes
    run_prefill(kind, 8, 8, calls=3)


def test_prefill_short_segments_and_ragged_tail():
    # C = 3 cuts segments at 3, 6, ...; T = 10 leaves a ragged last segment
    run_prefill(L.MIXED, 3, 3, calls=2)
    run_prefill(L.MIXED, 10, 10, calls=1)
    run_prefill(L.MIXED, 21, 8, calls=1)


def test_prefill_cadence_one():
    run_prefill(L.MIXED, 1, 1, calls=4)
    run_prefill(L.UNIFORM, 6, 1, calls=1)


@pytest.mark.parametrize("kind,per_row", [(L.MIXED, True), (L.HAD_INT8, False), (L.HAD_INT8, True)])
def test_prefill_long_call_every_eight_tokens(kind, per_row):
    # the workload's cadence: 512 tokens, write-back every 8 (64 in-call write-backs)
    run_prefill(kind, 512, 8, calls=1, per_row=per_row)


def test_prefill_long_call_uniform_and_fp32():
    run_prefill(L.UNIFORM, 128, 8, calls=1)
    run_prefill(L.FP32, 128, 8, calls=1)


@pytest.mark.parametrize("chunk", [1, 3, 8, 64])
def test_prefill_chunk_length_is_not_semantic(chunk):
    # segments are at most min(chunk, 8) tokens; the stored result is the same for every
    # chunk length (the recurrence is exact between write-backs)
    run_prefill(L.MIXED, 40, 16, calls=1, chunk=chunk)
