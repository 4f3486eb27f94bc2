"""GPU parity at a state larger than 4 GiB: heads whose regions start past the 32-bit
byte offset, checked against the CPU oracle.

A deployment holds far more than the configurations' layers in HBM (one MI355X has
288 GB), so head offsets, input and output offsets and the allocation pass must not wrap
at 2^32 bytes. These cases step a fresh state of B * H heads whose regions span more
than 4 GiB and compare the first head, the heads on either side of the 4 GiB boundary,
the last head and a few random heads with the oracle (teacher-forced, as the other
decode parity tests)."""
import numpy as np
import pytest

from oracle import layouts as L
from tests.test_gpu_parity import _layout, _state, run_decode

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # (name, layout, B, H, per-row decay, extra layout arguments)
    ("bitalloc", L.BITALLOC, 16384, 32, True, {}),
    ("mixed", L.MIXED, 8192, 32, True, dict(block=32, k_hi=16)),
    ("had-int8", L.HAD_INT8, 8192, 32, False, dict(block=128)),
    ("headalloc", L.HEADALLOC, 16384, 32, True, {}),
]


def _picks(B, H, stride, rng):
    n = B * H
    first_past = -(-(1 << 32) // stride)          # first head whose region starts at >= 4 GiB
    assert first_past < n, "the state must extend past 4 GiB"
    idx = {0, first_past - 1, first_past, first_past + 1, n - 1}
    idx |= {int(i) for i in rng.integers(first_past, n, 3)}
    return sorted((i // H, i % H) for i in idx)


@pytest.mark.parametrize("name,kind,B,H,per_row,extra", CASES, ids=[c[0] for c in CASES])
def test_state_past_four_gib(name, kind, B, H, per_row, extra):
    rng = np.random.default_rng(61)
    lay = _layout(kind, "rtn", B, H, 128, per_row=per_row, **extra)
    perm = np.stack([rng.permutation(128) for _ in range(H)]) if kind == L.MIXED else None
    st = _state(lay, perm)
    stride = st.region_stride()
    assert stride * B * H > (1 << 32)
    picks = _picks(B, H, stride, rng)
    print(f"\n[case] {name}: {B * H} heads, {stride * B * H / 2**30:.2f} GiB of regions, heads {picks}",
          flush=True)
    run_decode(lay, 2, heads=picks, warm=False, seed=62, perm=perm, state=st,
               alloc_every=1 if kind in (L.BITALLOC, L.HEADALLOC) else None)
    del st
    torch.cuda.empty_cache()
