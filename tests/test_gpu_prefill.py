"""GPU parity of chunked prefill with deferred write-back against the token-by-token
oracle (same bfloat16 inputs, float64 recurrence, write-back after every C-th token and
after the last token).

Tolerance reading for prefill (the decode tolerances assume one float64 step; the
prefill contractions run in float32 on MFMA as the workload prescribes): the state at a
write-back carries the float32 rounding of 128-term contractions, an absolute error of a
few float32 ulps of the row's magnitude. So a stored value must lie within half a step
(plus PF_ABS_REL * max|row|) of the oracle's float64 value -- for float16 rows near zero
the float16 spacing is smaller than that error --, at most PF_MAX_FRAC of the codes may
differ at all, float16 metadata may take the adjacent value within PF_META_REL of a
midpoint, and outputs agree to PF_O_REL relative L2 per head per call when the call has
one write-back (teacher-forced from the GPU's bytes). With several write-backs in a call
the oracle rounds on its own trajectory: one legitimate flip moves one state element by
one step (about 1/255 of its row's range), which moves later outputs of that column by
~1e-3 relative, so such calls are held to PF_O_REL_TRAJ.
"""
import numpy as np
import pytest

from oracle import layouts as L
from oracle.step import prefill as oracle_prefill
from synth import bf16_to_f32, prefill_inputs
from tests.parity import Tally, compare_write_back

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

PF_ABS_REL = 2e-6      # ~32 float32 ulps of the row maximum
PF_MAX_FRAC = 2e-3
PF_META_REL = 2e-5
PF_O_REL = 1e-5
PF_O_REL_TRAJ = 2e-3


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_prefill(kind, T, C, calls=1, B=2, H=2, seed=3, per_row=True, check_regions=True, **kw):
    import linear_attn_decode_amd as wb
    print(f"\n[case] prefill kind={kind} T={T} C={C} calls={calls} B={B} H={H}", flush=True)
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
    for c in range(calls):
        sl = slice(c * T, (c + 1) * T)
        q, k, v = (_dev(inp[n][:, sl]) for n in ("q", "k", "v"))
        beta, s = _dev(inp["beta"][:, sl]), _dev(inp["s"][:, sl])
        o = torch.zeros((B, T, H, 128), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        reg_in = st.regions().cpu().numpy()
        st.prefill(q.view(torch.int16), k.view(torch.int16), v.view(torch.int16), beta, s, o, T, 64, C, c * T)
        torch.cuda.synchronize()
        reg_out = st.regions().cpu().numpy()
        o_np = o.cpu().numpy()
        for bb in range(B):
            for hh in range(H):
                f = lambda n: bf16_to_f32(inp[n][bb, sl, hh]).astype(np.float64)
                s_h = inp["s"][bb, sl, hh]
                reg, _, outs, last = oracle_prefill(lay, reg_in[bb * H + hh][: lay.region_size()], None, f("q"),
                                                    f("k"), f("v"), inp["beta"][bb, sl, hh], s_h, c * T, C, bb, hh,
                                                    None if perm is None else perm[hh], return_last=True)
                got = o_np[bb, :, hh]
                rel = np.linalg.norm(got - outs) / max(np.linalg.norm(outs), 1e-30)
                o_worst = max(o_worst, rel)
                if check_regions:
                    compare_write_back(lay, reg_in[bb * H + hh], reg_out[bb * H + hh], last, None, None,
                                       c * T + T - 1, bb, hh, tally, meta_rel=PF_META_REL, fp32_rel=2e-5,
                                       abs_rel=PF_ABS_REL)
    tally.o_worst = o_worst
    print("[tally]", tally.summary(), flush=True)
    n_wb = -(-T // C) if T % C else T // C
    assert o_worst <= (PF_O_REL if n_wb == 1 else PF_O_REL_TRAJ), o_worst
    if check_regions:
        assert not tally.bad and tally.mismatch <= PF_MAX_FRAC * max(tally.elems, 1), tally.summary()
    return tally


@pytest.mark.parametrize("kind", [L.FP32, L.UNIFORM, L.HAD_INT8, L.MIXED])
def test_prefill_one_write_back_per_call(kind):
    # T = C: one write-back per call, so every call is teacher-forced from the GPU bytes
    run_prefill(kind, 8, 8, calls=3)


def test_prefill_short_segments_and_ragged_tail():
    # C = 3 cuts segments at 3, 6, ...; T = 10 leaves a ragged last segment
    run_prefill(L.MIXED, 3, 3, calls=2)
    run_prefill(L.MIXED, 10, 10, calls=1)


def test_prefill_cadence_one():
    run_prefill(L.MIXED, 1, 1, calls=4)


def test_prefill_long_call_outputs():
    # 64 tokens, write-back every 8: the oracle re-rounds on its own trajectory, so
    # only the outputs are compared (they are read before every write-back)
    run_prefill(L.MIXED, 64, 8, calls=1, check_regions=False)
    run_prefill(L.HAD_INT8, 64, 8, calls=1, check_regions=False, per_row=False)
