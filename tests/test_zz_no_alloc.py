"""The allocation pass that allocates nothing (state_allocate_bits_static: its workspace
is the library's static device array) against state_allocate_bits on the same states:
stored regions byte for byte, over two calls in a row, the second on a smaller layer
(the array keeps the first call's contents), for the layer-wise budget, the per-head
unit and the per-head budget; a layer whose workspace exceeds the array is refused
before anything runs."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _pair(kind, B, H, budget, seed):
    import linear_attn_decode_amd as wb
    rng = np.random.default_rng(seed)
    S = (rng.standard_normal((B, H, 128, 128)) * np.exp(rng.uniform(-4.0, 1.0, (B, H, 128, 1)))).astype(np.float32)
    S *= np.exp(rng.uniform(-2.0, 2.0, (B, H, 1, 1))).astype(np.float32)
    s = np.exp(rng.uniform(np.log(1e-3), 0.0, (B, H, 128))).astype(np.float32)
    per_row = kind == "bitalloc"
    states = []
    for _ in range(2):
        st = wb.WriteBackState(kind, "rtn", B, H, 128, 128, per_row, bbar=4, bmin=2, bmax=8, budget=budget)
        st.quantize(torch.from_numpy(S).cuda())
        states.append(st)
    return states, torch.from_numpy(s).cuda()


@pytest.mark.parametrize("kind,budget", [("bitalloc", "layer"), ("headalloc", "head"), ("bitalloc", "head")])
def test_static_scratch_allocation_matches_the_allocating_entry_point(kind, budget):
    for B, H, seed in ((4, 16, 5), (1, 4, 6)):          # the second call on a smaller layer
        print(f"[case] allocate_bits_static {kind} budget={budget} B={B} H={H}", flush=True)
        (ref, got), s = _pair(kind, B, H, budget, seed)
        ref.allocate_bits(s)
        got.allocate_bits_static(s)
        torch.cuda.synchronize()
        a, b = ref.regions().cpu().numpy(), got.regions().cpu().numpy()
        assert a.shape == b.shape
        diff = np.argwhere(a != b)
        assert diff.size == 0, diff[:4]
        # a second pass from the new widths, now with the estimators-free decays reversed
        ref.allocate_bits(s.flip(-1).contiguous())
        got.allocate_bits_static(s.flip(-1).contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(ref.regions().cpu().numpy(), got.regions().cpu().numpy())


def test_static_scratch_refuses_a_layer_larger_than_the_array():
    import linear_attn_decode_amd as wb
    # 512 x 32 heads of dk = 128 need 9 * 2^21 bytes of workspace, more than the 16 MiB
    st = wb.WriteBackState("bitalloc", "rtn", 512, 32, 128, 128, True, bbar=4, bmin=2, bmax=8, budget="layer")
    s = torch.full((512, 32, 128), 0.01, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = st.regions().cpu().numpy()[:64].copy()
    with pytest.raises(RuntimeError, match="ESCRATCH|static scratch"):
        st.allocate_bits_static(s)
    torch.cuda.synchronize()
    assert np.array_equal(before, st.regions().cpu().numpy()[:64])
