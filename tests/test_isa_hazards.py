"""Host check of the generated gfx950 code of the decode kernels.

The query-key and weight-value products are written as inline assembly
(v_dot2c_f32_bf16 with a DPP row broadcast), which the compiler's hazard
recognizer cannot see through.  Two rules are checked on the assembly of decode.hip (no GPU
needed), within each basic block:
  * the hardware requires two wait states between a VALU write of a VGPR
    and a DPP instruction reading it: none of a DPP product's VGPR operands
    may have been written by a VALU instruction less than two wait states
    earlier;
  * a DPP product's result needs more time before a plain read: an
    instruction other than a further product into the same accumulator may
    read it only four or more wait states later (two were measured to lose
    the product)."""
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


def _reads(insn):
    """VGPRs an instruction reads (for VALU: every operand but the
    destination, plus the destination of accumulating forms)."""
    parts = insn.split(None, 1)
    if len(parts) < 2:
        return set()
    op, rest = parts
    ops = [o.strip() for o in rest.split(",")]
    regs = set()
    start = 1 if op.startswith("v_") else 0
    if op.startswith("v_") and ("dot2c" in op or "fmac" in op or "mac_" in op):
        start = 0
    if op.startswith(("global_store", "buffer_store", "ds_write", "ds_store")):
        start = 0
    for o in ops[start:]:
        regs |= _regs(o.split()[0] if o else o)
    return regs


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_dpp_results_settle_before_plain_reads():
    text = _assemble(os.path.join(CSRC, "decode.hip"))
    lines = []
    for raw in text.splitlines():
        l = raw.strip()
        if not l or l.startswith(";") or l.startswith("."):
            continue
        lines.append(("LABEL", l) if l.endswith(":") else ("INSN", l))
    n_dpp = 0
    for i, (kind, l) in enumerate(lines):
        if kind != "INSN" or not l.startswith("v_dot2c_f32_bf16_dpp"):
            continue
        n_dpp += 1
        dst = _regs(l.split(None, 1)[1].split(",")[0])
        waits = 0
        j = i + 1
        while j < len(lines) and waits < 4:
            k2, nxt = lines[j]
            if k2 == "LABEL" or nxt.startswith("s_cbranch") or \
                    nxt.startswith("s_branch"):
                break
            op = nxt.split()[0]
            if op.startswith("v_dot2c_f32_bf16_dpp") and \
                    _regs(nxt.split(None, 1)[1].split(",")[0]) == dst:
                break  # the chain goes on into the same accumulator
            assert not (_reads(nxt) & dst), (
                "DPP result read too early: '%s' then '%s' after %d wait "
                "states" % (l, nxt, waits))
            waits += int(nxt.split()[1], 0) + 1 if op == "s_nop" else 1
            j += 1
    assert n_dpp > 0, "no DPP products found: did the kernel change?"
