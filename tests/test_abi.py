"""Host-side tests of the C ABI: the library loads, exports every declared symbol, sizes
its buffers like the storage formats say, and rejects bad arguments before touching
the GPU (no call here launches work)."""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_attn_decode_amd as wb
from oracle import layouts as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wbstate.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(state_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    h = ctypes.CDLL(wb.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(wb.SIGNATURES)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert wb.lib().state_status_str(code)
    assert wb.lib().state_status_str(-99) == b"unknown status"


@pytest.mark.parametrize("kind,dk,extra", [
    ("fp32", 16, {}), ("fp32", 128, {}), ("uniform", 16, {"bits": 4}), ("uniform", 128, {"bits": 2}),
    ("uniform", 128, {"bits": 8}), ("had_int8", 128, {"block": 128}), ("had_int8", 128, {"block": 32}),
    ("mixed", 128, {"block": 32, "k_hi": 16}), ("bitalloc", 128, {"bbar": 4}), ("bitalloc", 128, {"bbar": 3}),
])
@pytest.mark.parametrize("mode", ["rtn", "sr", "ef"])
def test_buffer_sizes_match_the_storage_format(kind, dk, extra, mode):
    B, H = 3, 5
    desc = wb.make_desc(kind, mode, B, H, dk, dk, **extra)
    nbytes, side = wb.buffer_sizes(desc)
    lay = L.Layout(kind=kind, B=B, H=H, dk=dk, dv=dk, mode=mode, **extra)
    expect = lay.region_stride() * B * H
    if kind == "mixed":
        expect += (H * dk + 255) // 256 * 256
    assert nbytes == expect
    assert side == lay.side_elems() * B * H * 4


def _code(desc):
    sb, side = ctypes.c_size_t(), ctypes.c_size_t()
    return wb.lib().state_bytes(ctypes.byref(desc), ctypes.byref(sb), ctypes.byref(side))


def test_descriptor_validation():
    ok = wb.make_desc("mixed", "rtn", 2, 2)
    assert _code(ok) == 0
    bad = [
        (dict(kind=7), -1), (dict(mode=5), -1), (dict(decay=3), -1), (dict(B=0), -1), (dict(mem_bits=1), -1),
        (dict(mode=3, mem_bits=2), -3), (dict(mode=4, mem_bits=2), -3),
        (dict(dk=64), -3), (dict(dv=64), -3), (dict(block=48), -3), (dict(k_hi=0), -3), (dict(k_hi=128), -3),
        (dict(k_hi=20), -3),
    ]
    for fields, code in bad:
        d = wb.make_desc("mixed", "rtn", 2, 2)
        for k, v in fields.items():
            setattr(d, k, v)
        assert _code(d) == code, fields
    d = wb.make_desc("uniform", "rtn", 1, 1, 16, 16, bits=3)
    assert _code(d) == -3
    # one-bit rows: bmin = 1 for the per-row unit; the per-head unit keeps a two-bit floor
    assert _code(wb.make_desc("bitalloc", "rtn", 1, 1, bbar=4, bmin=1)) == 0
    assert _code(wb.make_desc("bitalloc", "rtn", 1, 1, bbar=4, bmin=0)) == -3
    assert _code(wb.make_desc("headalloc", "rtn", 1, 1, bbar=4, bmin=1)) == -3
    assert _code(wb.make_desc("headalloc", "rtn", 1, 4, bbar=4, bmin=2)) == 0
    assert _code(wb.make_desc("headalloc", "rtn", 1, 1, bbar=4, budget="layer")) == -3
    # INT4 tier of the Hadamard layouts: codes two a byte
    assert _code(wb.make_desc("had_int8", "rtn", 1, 1, block=32, int_bits=3)) == -1
    assert _code(wb.make_desc("uniform", "rtn", 1, 1, int_bits=4)) == -1
    d = wb.make_desc("had_int8", "rtn", 2, 3, block=32, int_bits=4)
    assert _code(d) == 0
    assert wb.buffer_sizes(d)[0] == 2 * 3 * -(-(128 * 128 // 2 + 128 * 4 * 4) // 256) * 256
    d = wb.make_desc("mixed", "ef", 1, 2, block=32, k_hi=16, int_bits=4)
    assert wb.buffer_sizes(d)[0] == 2 * -(-(16 * 128 * 2 + 112 * 64 + 112 * 4 * 4) // 256) * 256 + 256
    d = wb.make_desc("bitalloc", "rtn", 1, 1, bbar=4, bmax=9)
    assert _code(d) == -3
    d = wb.make_desc("fp32", "rtn", 1, 1, 32, 32)
    assert _code(d) == -3
    # temporal-memory rules: uniform grid only, 1 <= k <= 8, a float32 side value per element
    for mode in ("dir", "resq"):
        assert _code(wb.make_desc("uniform", mode, 1, 1, 16, 16, mem_bits=0)) == -1
        assert _code(wb.make_desc("uniform", mode, 1, 1, 16, 16, mem_bits=9)) == -1
        d = wb.make_desc("uniform", mode, 2, 3, mem_bits=3)
        assert _code(d) == 0
        assert wb.buffer_sizes(d)[1] == 2 * 3 * 128 * 128 * 4
        assert _code(wb.make_desc("bitalloc", mode, 1, 1, mem_bits=2)) == -3
    # layer-wise width budget: BITALLOC only, at most 4096 rows per sequence; regions
    # sized for every row at bmax, then the allocation workspace (float64 cost and u8
    # width per row)
    assert _code(wb.make_desc("bitalloc", "rtn", 1, 1, budget=2)) == -1
    assert _code(wb.make_desc("mixed", "rtn", 1, 1, budget="layer")) == -3
    assert _code(wb.make_desc("bitalloc", "rtn", 1, 33, budget="layer")) == -3
    d = wb.make_desc("bitalloc", "rtn", 3, 32, budget="layer", bbar=4, bmax=6)
    assert _code(d) == 0
    stride = -(-(128 * 128 * 6 // 8 + 3 * 128) // 256) * 256
    assert wb.buffer_sizes(d)[0] == 3 * 32 * stride + -(-(3 * 32 * 128 * 9) // 256) * 256
    d = wb.make_desc("bitalloc", "rtn", 3, 32, bbar=4, bmax=6)
    assert wb.buffer_sizes(d)[0] == 3 * 32 * -(-(128 * 128 * 4 // 8 + 3 * 128) // 256) * 256


def test_alloc_rejects_bad_buffers_without_touching_the_gpu():
    L_ = wb.lib()
    d = wb.make_desc("mixed", "ef", 2, 2)
    nbytes, side = wb.buffer_sizes(d)
    out = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x10000)            # never dereferenced: validation fails first
    perm = np.tile(np.arange(128, dtype=np.uint8), (2, 1))
    pp = perm.ctypes.data_as(ctypes.c_void_p)
    assert L_.state_alloc(ctypes.byref(d), None, nbytes, fake, side, pp, None, ctypes.byref(out)) == -1
    assert L_.state_alloc(ctypes.byref(d), fake, nbytes - 1, fake, side, pp, None, ctypes.byref(out)) == -2
    assert L_.state_alloc(ctypes.byref(d), ctypes.c_void_p(0x10004), nbytes, fake, side, pp, None,
                          ctypes.byref(out)) == -5
    assert L_.state_alloc(ctypes.byref(d), fake, nbytes, None, side, pp, None, ctypes.byref(out)) == -1
    assert L_.state_alloc(ctypes.byref(d), fake, nbytes, fake, side - 4, pp, None, ctypes.byref(out)) == -2
    assert L_.state_alloc(ctypes.byref(d), fake, nbytes, fake, side, None, None, ctypes.byref(out)) == -1
    bad = perm.copy()
    bad[1, 5] = bad[1, 6]
    assert L_.state_alloc(ctypes.byref(d), fake, nbytes, fake, side, bad.ctypes.data_as(ctypes.c_void_p), None,
                          ctypes.byref(out)) == -1
    bad[1, 5] = 200
    assert L_.state_alloc(ctypes.byref(d), fake, nbytes, fake, side, bad.ctypes.data_as(ctypes.c_void_p), None,
                          ctypes.byref(out)) == -1


def test_calls_reject_null_handles_and_pointers():
    L_ = wb.lib()
    p = ctypes.c_void_p(0x10000)
    assert L_.state_step_decode(None, p, p, p, p, p, p, 0, None) == -1
    assert L_.state_dequant(None, p, None) == -1
    assert L_.state_quantize(None, p, None) == -1
    assert L_.state_allocate_bits(None, p, None, 0, 1, None) == -1
    assert L_.state_allocate_bits_static(None, p, None, 0, 1, None) == -1
    assert L_.state_set_estimators(None, p) == -1
    assert L_.state_step_decode_alloc(None, p, p, p, p, p, p, 0, 0, 1, None) == -1
    assert L_.state_free(None) == -1
    assert L_.state_set_activity(None, p, p) == -1
    assert L_.state_prefill_chunk(None, p, p, p, p, p, p, 8, 64, 8, 0, None) == -1
    a, b, c = ctypes.c_void_p(), ctypes.c_size_t(), ctypes.c_void_p()
    assert L_.state_export(None, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == -1
    assert L_.state_damp_select(None, 1, 1, 128, 128, 32, 16, p, ctypes.c_float(0.01), None, p, None) == -1
    assert L_.state_damp_select(p, 1, 1, 64, 128, 32, 16, p, ctypes.c_float(0.01), None, p, None) == -3
    assert L_.state_damp_select(p, 1, 1, 128, 128, 32, 16, p, ctypes.c_float(0.0), None, p, None) == -1
