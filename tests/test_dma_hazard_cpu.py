"""The prefill kernel's LDS DMA is written in inline asm (so the compiler adds
no pipeline-draining waits of its own), and the compiler does not pad hazards
before an inline-asm instruction.  A VMEM instruction that reads an SGPR needs
five wait states after a VALU instruction wrote it (CDNA3/CDNA4 ISA, manually
inserted wait states); the asm carries a single s_nop, which is enough only
while the scalar bases come from SALU arithmetic.  If a change to the kernel
makes the compiler reload spilled bases with v_readlane right before the DMA,
the DMA reads a stale base: a GPU memory fault.  This compiles gemm.hip for
gfx950 (no GPU needed) and checks the generated code for that pattern."""
import os
import re
import subprocess
import tempfile

import pytest

from nvfp4_w4a4_gemm_quantize_amd import build as B

WAIT_STATES = 5


def _sgprs(tok):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def hazards(asm_text):
    """(number of LDS DMA instructions, list of hazards) in gfx9 asm text."""
    lines = [l.split(";")[0].strip() for l in asm_text.splitlines()]
    insts = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    found, ndma = [], 0
    for i, ins in enumerate(insts):
        if not ins.startswith("global_load_lds"):
            continue
        ndma += 1
        ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
        base = _sgprs(ops[1]) if len(ops) > 1 else set()
        ws = 0
        for j in range(i - 1, max(-1, i - 16), -1):
            prev = insts[j]
            parts = prev.split(None, 1)
            if parts[0] == "s_nop":
                ws += int(parts[1], 0) + 1
            else:
                dst = parts[1].split(",")[0].strip() if len(parts) > 1 else ""
                if parts[0].startswith("v_") and _sgprs(dst) & base:
                    found.append((prev, ins, ws))
                    break
                ws += 1
            if ws >= WAIT_STATES:
                break
    return ndma, found


def test_scanner_flags_the_pattern():
    bad = "v_readlane_b32 s21, v201, 11\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v104, s[20:21]\n"
    ok = "v_readlane_b32 s21, v201, 11\n\ts_nop 4\n\tglobal_load_lds_dwordx4 v104, s[20:21]\n"
    salu = "s_add_u32 s20, s20, 32\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v104, s[20:21]\n"
    assert len(hazards(bad)[1]) == 1
    assert hazards(ok)[1] == [] and hazards(salu)[1] == []


@pytest.mark.timeout(600)
def test_prefill_dma_has_no_valu_sgpr_hazard():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        cmd = [B.hipcc()] + B.COMMON + B.DEVICE + ["-x", "hip", "--cuda-device-only", "-S",
                                                   os.path.join(B.CSRC, "gemm.hip"), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        ndma, found = hazards(open(out).read())
    assert ndma > 100, "no LDS DMA instructions found: the scan would prove nothing"
    assert not found, "VALU write of an SGPR base within %d wait states of an LDS DMA: %s" % (
        WAIT_STATES, found[:3])
