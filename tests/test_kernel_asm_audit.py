"""Checks on the compiled device code of the HIP sources (CPU only: hipcc cross-compiles for
gfx950 without a GPU).

* Matrix instructions written as inline assembly (the score product of the kernels with two
  head blocks per wave keeps its accumulators in VGPRs that way) bypass the compiler's hazard
  handling, so the compiled code is checked against the rules those instructions rely on:
  no vector instruction writes an A/B source register in the few instructions before the
  MFMA, and nothing reads or writes the accumulator before the wait block that follows the
  product (s_nop 7), other than the next accumulation step into the same registers.
* No packed f32 vector arithmetic is emitted anywhere (the build turns that feature off).
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_latent_attention_attn_amd import build_lib

HIPCC = build_lib.HIPCC
pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")

HIP_SOURCES = [s for s in build_lib.SOURCES if s.endswith(".hip")]


def device_asm(src: str, tmp_path) -> list[str]:
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *build_lib.COMMON, *build_lib.SOURCES[src], "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(build_lib.CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return [l.strip() for l in out.read_text().split("\n")]


def vregs(tok: str) -> set[int]:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def split(inst: str) -> tuple[str, list[str]]:
    parts = inst.split(None, 1)
    return parts[0], ([t.strip() for t in parts[1].split(",")] if len(parts) > 1 else [])


def audit_inline_mfma(lines: list[str]) -> tuple[int, list[str]]:
    inasm, inside = set(), False
    for i, l in enumerate(lines):
        if l.startswith(";;#ASMSTART"):
            inside = True
        elif l.startswith(";;#ASMEND"):
            inside = False
        elif inside:
            inasm.add(i)
    insts = [(i, l) for i, l in enumerate(lines)
             if l and not l.startswith((";", ".")) and not l.endswith(":")]
    checked, findings = 0, []
    for k, (i, l) in enumerate(insts):
        op, ops = split(l)
        if i not in inasm or not op.startswith("v_mfma") or not ops or not vregs(ops[0]):
            continue
        checked += 1
        dst = vregs(ops[0])
        srcs = vregs(ops[1]) | vregs(ops[2])
        for _, prev in insts[max(0, k - 4):k]:
            pop, pops = split(prev)
            if pop.startswith("v_") and not pop.startswith("v_mfma") and pops and vregs(pops[0]) & srcs:
                findings.append(f"vector write to a source just before: {prev} -> {l}")
        for _, nxt in insts[k + 1:]:
            if nxt.startswith("s_nop 7"):
                break
            nop, nops = split(nxt)
            if nop.startswith("v_mfma") and nops and vregs(nops[0]) == dst and vregs(nops[3]) == dst:
                break
            if any(vregs(t) & dst for t in nops):
                findings.append(f"accumulator used before the wait: {l} | {nxt}")
                break
    return checked, findings


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_device_code(src, tmp_path):
    lines = device_asm(src, tmp_path)
    packed = [l for l in lines if re.match(r"v_pk_(add|mul|fma)_f32\b", l)]
    assert not packed, packed[:5]
    checked, findings = audit_inline_mfma(lines)
    assert not findings, "\n".join(findings[:10])
    if src == "attn_fwd_wide.hip":
        assert checked > 0, "the wide kernels are expected to hold inline-assembly score MFMAs"


def test_audit_catches_a_planted_hazard():
    # the audit function itself: a VGPR write right before the MFMA and an early read of the result
    lines = [";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0", ";;#ASMEND",
             "v_mov_b32_e32 v20, v1", "s_nop 7"]
    assert len(audit_inline_mfma(lines)[1]) == 1
    lines = ["v_mov_b32_e32 v5, 0", ";;#ASMSTART",
             "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]", ";;#ASMEND", "s_nop 7"]
    assert len(audit_inline_mfma(lines)[1]) == 1
