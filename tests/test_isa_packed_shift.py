"""The decode kernels that pack rounded levels must not be compiled to ``v_ashr_pk_u8_i32``.

The compiler can merge a saturating byte clamp of two right-shifted 32-bit values and
their packing into one ``v_ashr_pk_u8_i32``, then OR the next two bytes into the upper
half of the same register as if that half were zero. Under stochastic rounding in the
rotated-domain decode step (levels as (2^16 - 1 - z - u) >> 16 clamped to [0, 255]) the
upper two bytes of every packed word then came out with stray bits set (codes OR-ed with
extra bits, every head of a full layer). The kernels keep such values opaque before
packing; this test compiles the decode sources that round and pack codes with a shift
(the rotated-domain and the decay-aware kernels) for gfx950 with the library's own flags
and checks the assembly. No GPU is needed."""
import os
import shutil
import subprocess

import pytest

from linear_attn_decode_amd import build as B


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")), reason="no hipcc")
@pytest.mark.parametrize("src", ["decode_rot.hip", "decode_bitalloc.hip"])
def test_no_packed_byte_shift(src):
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([B._hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", "-"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln.strip() for ln in r.stdout.splitlines() if ln.strip().startswith("v_ashr_pk_")]
    assert not lines, lines[:5]
