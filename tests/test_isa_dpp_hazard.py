"""The rotated-layout decode kernel multiplies with row weights broadcast by DPP inside a
float64 multiply-add (``v_fmac_f64_dpp ... row_newbcast``) written as inline assembly.
On gfx9 a DPP source must not have been written by a vector instruction in the two
preceding wait states, and the compiler's hazard recognizer does not look inside inline
assembly. This test compiles the kernel source to gfx950 assembly with the library's own
flags and checks every such instruction: walking back over the preceding instructions
until two wait states have passed (an ``s_nop N`` counts N + 1), no vector instruction may
write a register of the DPP source operand. No GPU is needed."""
import os
import re
import shutil
import subprocess

import pytest

from linear_attn_decode_amd import build as B

SRC = os.path.join(B.CSRC, "decode_rot.hip")


def _vregs(op: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _instructions(asm: str) -> list:
    out = []
    for line in asm.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        out.append(s)
    return out


def dpp_source_hazards(asm: str) -> tuple:
    """(number of v_fmac_f64_dpp instructions, list of hazards found)."""
    ins = _instructions(asm)
    found, n = [], 0
    for i, s in enumerate(ins):
        if not s.startswith("v_fmac_f64_dpp"):
            continue
        n += 1
        src0 = _vregs(s.split()[2].rstrip(","))
        waits, j = 0, i - 1
        while j >= 0 and waits < 2:
            t = ins[j]
            if t.startswith("s_nop"):
                waits += int(t.split()[1], 0) + 1
            else:
                if t.startswith("v_") and not t.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
                    if _vregs(t.split()[1].rstrip(",")) & src0:
                        found.append((t, s))
                        break
                waits += 1
            j -= 1
    return n, found


def test_checker_flags_a_planted_hazard():
    # a vector write of the DPP source right before the multiply-add is a hazard; the same
    # write two instructions earlier, or behind an s_nop 1, is not
    bad = "v_mov_b32_e32 v22, 0\nv_fmac_f64_dpp v[10:11], v[22:23], v[14:15] row_newbcast:3\n"
    ok1 = "v_mov_b32_e32 v22, 0\nv_add_u32_e32 v1, v1, v2\nv_add_u32_e32 v3, v3, v2\n" \
          "v_fmac_f64_dpp v[10:11], v[22:23], v[14:15] row_newbcast:3\n"
    ok2 = "v_mov_b32_e32 v22, 0\ns_nop 1\nv_fmac_f64_dpp v[10:11], v[22:23], v[14:15] row_newbcast:0\n"
    assert dpp_source_hazards(bad)[1]
    assert not dpp_source_hazards(ok1)[1]
    assert not dpp_source_hazards(ok2)[1]


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")), reason="no hipcc")
def test_rotated_kernel_dpp_sources_have_no_hazard():
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([B._hipcc(), *flags, "--cuda-device-only", "-S", SRC, "-o", "-"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    n, found = dpp_source_hazards(r.stdout)
    assert n > 0, "no DPP multiply-add found: the check no longer covers the kernel"
    assert not found, found[:5]
