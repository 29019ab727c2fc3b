"""Checks on the gfx950 assembly of the backward kernels (CPU only: hipcc cross-compiles).

The dK/dV gradient MFMAs are inline assembly (so that their accumulators stay in AGPRs), and
the compiler's hazard recognizer does not see into inline assembly. A vector ALU write of a
VGPR that an MFMA then reads as its A or B operand needs at least two wait states in between;
these tests compile the kernels the way the library is built and check that no such write sits
in the two instructions before any inline-assembly MFMA, and that the accumulators are given
their wait states before they are read back.
"""
import os
import re
import subprocess

import pytest

from coalesced_varlen_attention_amd import build as B

SRC = os.path.join(B.CSRC, "zl_bwd.hip")


@pytest.fixture(scope="module")
def asm_lines(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("isa") / "zl_bwd.s")
    flags = [f for f in B.DEVICE_FLAGS if f != "-fPIC"] + B.EXTRA_DEVICE_FLAGS["zl_bwd.hip"]
    cmd = [B._hipcc(), *flags, "-I", B.INCLUDE, "-I", B.CSRC, "--cuda-device-only", "-S", SRC, "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-2000:]
    return open(out).read().splitlines()


def _instr(line):
    t = line.strip()
    if not t or t.startswith((";", ".", "_")) or t.endswith(":"):
        return None
    return t


def _vgprs(operand):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", operand)
    return {int(m.group(1))} if m else set()


def _wait_states(instr):
    m = re.fullmatch(r"s_nop (\d+)", instr)
    return int(m.group(1)) + 1 if m else 1


def test_inline_mfma_operands_are_not_written_just_before(asm_lines):
    """Walk back from every inline-assembly MFMA until two wait states have passed (an
    instruction counts one, s_nop N counts N + 1); no vector instruction in that window may
    write the MFMA's A or B operand registers."""
    n_checked = 0
    for i, line in enumerate(asm_lines):
        t = _instr(line)
        if not t or not t.startswith("v_mfma") or not any(";;#ASMSTART" in asm_lines[k] for k in (i - 1, i - 2)):
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        src = _vgprs(ops[1]) | _vgprs(ops[2])
        waited, k = 0, i - 1
        while waited < 2 and k >= 0:
            p = _instr(asm_lines[k])
            k -= 1
            if not p or p.startswith(";;#ASM"):
                continue
            if p.startswith("v_") and not p.startswith("v_mfma"):
                dst = p.split(None, 1)[1].split(",")[0].strip()
                assert not (_vgprs(dst) & src), f"VALU write too close before an inline MFMA: {p!r} -> {t!r}"
            waited += _wait_states(p)
        n_checked += 1
    assert n_checked >= 32, "expected the dK/dV inline MFMAs in the assembly"


def test_accumulators_settle_before_readback(asm_lines):
    text = "\n".join(asm_lines)
    assert text.count("s_nop 15") >= 3, "the accumulator read-back wait states are missing"
