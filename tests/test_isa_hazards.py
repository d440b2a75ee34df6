"""Host check of the generated gfx950 code of the decode kernels.

The query-key products are written as inline assembly (v_dot2c_f32_bf16 with
a DPP row broadcast), which the compiler's hazard recognizer cannot see
through.  The hardware requires two wait states between a VALU write of a
VGPR and a DPP instruction reading it.  This test compiles decode.hip to
assembly (no GPU needed) and checks every DPP product: none of its VGPR
operands may have been written by a VALU instruction less than two wait
states earlier in the same basic block."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "global_gqa_attention_kv_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _assemble(src):
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Xclang",
               "-target-feature", "-Xclang", "-packed-fp32-ops", "-S",
               "--cuda-device-only", src, "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        return open(out).read()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_dpp_products_respect_wait_states():
    text = _assemble(os.path.join(CSRC, "decode.hip"))
    lines = []
    for raw in text.splitlines():
        l = raw.strip()
        if not l or l.startswith(";") or l.startswith("."):
            continue
        if l.endswith(":"):
            lines.append(("LABEL", l))
            continue
        lines.append(("INSN", l))
    n_dpp = 0
    for i, (kind, l) in enumerate(lines):
        if kind != "INSN" or not l.startswith("v_dot2c_f32_bf16_dpp"):
            continue
        n_dpp += 1
        ops = l.split(None, 1)[1].split(",")[:3]
        reads = set()
        for o in ops:
            reads |= _regs(o)
        waits = 0
        j = i - 1
        while j >= 0 and waits < 2:
            k2, prev = lines[j]
            if k2 == "LABEL":
                break
            op = prev.split()[0]
            if op.startswith("v_"):
                dst = prev.split(None, 1)[1].split(",")[0] if " " in prev else ""
                assert not (_regs(dst) & reads), (
                    "DPP hazard: '%s' then '%s' with %d wait states" %
                    (prev, l, waits))
                waits += 1
            elif op == "s_nop":
                waits += int(prev.split()[1], 0) + 1
            else:
                waits += 1
            j -= 1
    assert n_dpp > 0, "no DPP products found: did the kernel change?"
