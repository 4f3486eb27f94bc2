"""Every head of a full layer, one teacher-forced decode step, against the oracle.

The mixed layout at B = 256, H = 32 (round to nearest, stochastic rounding and error
feedback, its residuals compared too), the decay-aware per-row widths
at the same shape (round to nearest, Philox stochastic rounding and error feedback, after
an allocation pass; under the layer-wise budget; with one-bit rows allowed), the Hadamard INT8 layout
(all three rules) and its INT4 tier at B = 64, H = 16 with per-head decay and the per-head allocation unit
at that shape (all three rules), in the launch configurations
the benchmark times: every head state of the layer is compared, not a
sample, so that the parity bound (codes bit-equal except at most 1e-4 of the elements,
each one step apart and within 1e-5 of a step of the boundary; outputs within 1e-4
relative L2 per head) is checked at scale. The oracle runs in 16 spawned processes over
arrays saved to a temporary directory.
"""
import multiprocessing as mp
import os
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

from oracle import layouts as L
from synth import decode_inputs
from tests.parity import MAX_FRAC, Tally, check_heads_chunk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

WORKERS = 16


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


CASES = {
    "mixed-rtn": dict(kind=L.MIXED, mode="rtn", B=256, H=32, per_row=True, kw=dict(block=32, k_hi=16)),
    "bitalloc-rtn": dict(kind=L.BITALLOC, mode="rtn", B=256, H=32, per_row=True, kw={}),
    "bitalloc-sr": dict(kind=L.BITALLOC, mode="sr", B=256, H=32, per_row=True, kw={}),
    "bitalloc-layer-rtn": dict(kind=L.BITALLOC, mode="rtn", B=256, H=32, per_row=True, kw=dict(budget="layer")),
    "had-int8-rtn-gdn": dict(kind=L.HAD_INT8, mode="rtn", B=64, H=16, per_row=False, kw=dict(block=128)),
    "headalloc-rtn-gdn": dict(kind=L.HEADALLOC, mode="rtn", B=64, H=16, per_row=False, kw={}),
    "had-int4-rtn-gdn": dict(kind=L.HAD_INT8, mode="rtn", B=64, H=16, per_row=False, kw=dict(block=128, int_bits=4)),
    "bitalloc-1bit-rtn": dict(kind=L.BITALLOC, mode="rtn", B=256, H=32, per_row=True, kw=dict(bmin=1)),
    "headalloc-sr-gdn": dict(kind=L.HEADALLOC, mode="sr", B=64, H=16, per_row=False, kw={}),
    "mixed-sr": dict(kind=L.MIXED, mode="sr", B=256, H=32, per_row=True, kw=dict(block=32, k_hi=16)),
    "had-int8-sr-gdn": dict(kind=L.HAD_INT8, mode="sr", B=64, H=16, per_row=False, kw=dict(block=128)),
    "bitalloc-ef": dict(kind=L.BITALLOC, mode="ef", B=256, H=32, per_row=True, kw={}),
    "headalloc-ef-gdn": dict(kind=L.HEADALLOC, mode="ef", B=64, H=16, per_row=False, kw={}),
    "mixed-ef": dict(kind=L.MIXED, mode="ef", B=256, H=32, per_row=True, kw=dict(block=32, k_hi=16)),
    "had-int8-ef-gdn": dict(kind=L.HAD_INT8, mode="ef", B=64, H=16, per_row=False, kw=dict(block=128)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_full_layer_every_head(case):
    import linear_attn_decode_amd as wb
    c = CASES[case]
    kind, mode, B, H, per_row, kw = c["kind"], c["mode"], c["B"], c["H"], c["per_row"], c["kw"]
    d = 128
    lay_kw = dict(kind=kind, B=B, H=H, dk=d, dv=d, mode=mode, per_row_decay=per_row, seed=0x5EED_1234_ABCD, **kw)
    print(f"\n[case] full layer {case} B={B} H={H}", flush=True)
    rng = np.random.default_rng(61)
    perm = np.stack([rng.permutation(d) for _ in range(H)]) if kind == L.MIXED else None
    st = wb.WriteBackState(kind, mode, B, H, d, d, per_row, seed=lay_kw["seed"], perm=perm, **kw)
    scale = np.exp(rng.uniform(-3.0, 0.5, (B, H, d, 1)))
    S0 = (rng.standard_normal((B, H, d, d)) * scale).astype(np.float32)
    st.quantize(_dev(S0))
    del S0
    inp = decode_inputs(62, B, H, d, d, 2, per_row)
    dev = {n: _dev(a) for n, a in inp.items()}
    o = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
    if kind in (L.BITALLOC, L.HEADALLOC):
        s_rows = dev["s"] if per_row else dev["s"][:, :, None].expand(B, H, d).contiguous()
        st.allocate_bits(s_rows)
    # one untimed step, so that the compared step starts from a state the kernel wrote
    st.step_decode(dev["q"][0], dev["k"][0], dev["v"][0], dev["beta"][0], dev["s"], o, 0)
    torch.cuda.synchronize()
    reg_in = st.regions().cpu().numpy()[:, : L.Layout(**lay_kw).region_size()]
    e_in = st.residuals().cpu().numpy() if mode == "ef" else None
    st.step_decode(dev["q"][1], dev["k"][1], dev["v"][1], dev["beta"][1], dev["s"], o, 1)
    torch.cuda.synchronize()
    reg_out = st.regions().cpu().numpy()[:, : reg_in.shape[1]]
    with tempfile.TemporaryDirectory(dir="/tmp") as tmp:
        arrays = dict(reg_in=reg_in, reg_out=reg_out, o=o.cpu().numpy(), q=inp["q"][1], k=inp["k"][1],
                      v=inp["v"][1], beta=inp["beta"][1], s=inp["s"])
        if mode == "ef":
            arrays["e_in"] = e_in
            arrays["e_out"] = st.residuals().cpu().numpy()
        if perm is not None:
            arrays["perm"] = perm
        for n, a in arrays.items():
            np.save(os.path.join(tmp, n + ".npy"), np.ascontiguousarray(a))
        n = B * H
        chunks = [(tmp, lay_kw, i * n // 64, (i + 1) * n // 64, 1) for i in range(64)]
        t0 = time.time()
        total = Tally()
        with ProcessPoolExecutor(max_workers=WORKERS, mp_context=mp.get_context("spawn")) as ex:
            for i, tl in enumerate(ex.map(check_heads_chunk, chunks)):
                total.elems += tl.elems
                total.mismatch += tl.mismatch
                total.bad += tl.bad
                total.meta_blocks += tl.meta_blocks
                total.meta_adjacent += tl.meta_adjacent
                total.o_worst = max(total.o_worst, tl.o_worst)
                if i % 16 == 15:
                    print(f"[full] {i + 1}/64 chunks, {time.time() - t0:.0f} s", flush=True)
    print("[tally]", total.summary(), flush=True)
    assert total.elems == n * d * d
    assert not total.bad and total.mismatch <= MAX_FRAC * total.elems and total.o_worst <= 1e-4, total.summary()
