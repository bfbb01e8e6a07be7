"""Wait states around the 256-tile GEMM's matrix instructions.

The 256-tile kernel issues its MFMAs as inline asm, whose result latency the
compiler does not know, so it inserts no wait states after them.  Nothing
may then read an accumulator (v_accvgpr_read, v_accvgpr_mov, any VALU
operand) until the MFMA that wrote it has finished, and no MFMA may take an
accumulator as its C operand right after a VALU write to it.  This test
builds the kernel's gfx950 assembly with the library's own flags and checks
both on every path: a read needs at least 19 wait states after the MFMA (the
longest result latency of a matrix instruction: one per instruction issued
in between, N + 1 per s_nop N), a write at least 2 before the MFMA.  An MFMA
whose C operand is exactly the previous one's result (an accumulation
chain) is served by the hardware and allowed.  CPU only: no kernel runs.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "_ZN5dmuon12_GLOBAL__N_116gemm_bf16_kernelILi256ELi2EEEvPKNS_8GemmTaskEPKNS_7TileRefE"
READ_WAIT = 19
WRITE_WAIT = 2

_MFMA = re.compile(r"v_mfma\S*\s+a\[(\d+):(\d+)\],.*,\s*a\[(\d+):(\d+)\]$")
_AREG = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")


def _kernel_asm(tmp_path, source=None):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    sys.path.insert(0, os.path.join(ROOT, "matrix_optimizer_step_owned_amd"))
    try:
        import _build
    finally:
        sys.path.pop(0)
    out = tmp_path / "gemm.s"
    cmd = [hipcc, *_build.HIPCC_FLAGS, "--cuda-device-only", "-S",
           source or os.path.join(_build.CSRC, "gemm.hip"), "-o", str(out)]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-4000:]
    text = out.read_text().split("\n")
    start = next(i for i, l in enumerate(text) if l.startswith(KERNEL + ":"))
    end = next(i for i in range(start, len(text)) if text[i].startswith(".Lfunc_end"))
    body = []
    for l in text[start:end]:
        t = l.split(";")[0].strip()
        if t and (t.endswith(":") or not t.startswith(".")):
            body.append(t)
    return body


def _agprs(operands):
    regs = set()
    for single, lo, hi in _AREG.findall(operands):
        if single:
            regs.add(int(single))
        else:
            regs.update(range(int(lo), int(hi) + 1))
    return regs


def _wait_states(instr):
    m = re.match(r"s_nop\s+(\d+)", instr)
    return int(m.group(1)) + 1 if m else 1


def _paths(body, k, budget):
    """The instructions that may follow body[k], along every branch, until
    `budget` wait states have passed: yields (instruction, wait states
    before it)."""
    labels = {t[:-1]: i for i, t in enumerate(body) if t.endswith(":")}
    stack = [(k + 1, 0)]
    seen = set()
    while stack:
        i, waited = stack.pop()
        while i < len(body) and waited < budget:
            if (i, waited) in seen:
                break
            seen.add((i, waited))
            t = body[i]
            if t.endswith(":"):
                i += 1
                continue
            yield t, waited
            if t.startswith("s_endpgm"):
                break
            waited += _wait_states(t)
            target = re.match(r"s_(c?)branch\S*\s+(\S+)", t)
            if target:
                if target.group(2) in labels:
                    stack.append((labels[target.group(2)] + 1, waited))
                if not target.group(1):
                    break       # unconditional: no fall-through
            i += 1


def _hazards(body):
    found = []
    for k, t in enumerate(body):
        m = _MFMA.match(t)
        if not m:
            continue
        dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
        chained = set()
        for t2, waited in _paths(body, k, READ_WAIT):
            m2 = _MFMA.match(t2)
            if m2:
                src_c = set(range(int(m2.group(3)), int(m2.group(4)) + 1))
                if src_c & dst and src_c != dst:
                    found.append(f"partial C overlap: {t} -> {t2}")
                continue    # an exact chain: the hardware forwards the result
            ops = t2.split(None, 1)[1] if " " in t2 else ""
            if _agprs(ops) & dst:
                found.append(f"read after {waited} wait states: {t} -> {t2}")
    for k, t in enumerate(body):
        w = re.match(r"v_accvgpr_(?:write|mov)_b32\s+a(\d+),", t)
        if not w:
            continue
        reg = int(w.group(1))
        for t2, waited in _paths(body, k, WRITE_WAIT):
            m2 = _MFMA.match(t2)
            if m2 and int(m2.group(3)) <= reg <= int(m2.group(4)):
                found.append(f"MFMA reads a{reg} {waited} wait states after its write: {t} -> {t2}")
    return found


def test_no_accumulator_read_inside_mfma_latency(tmp_path):
    body = _kernel_asm(tmp_path)
    assert sum(1 for t in body if t.startswith("v_mfma")) >= 512, "the 256-tile kernel's MFMAs were not found"
    found = _hazards(body)
    assert not found, "\n".join(found[:20])


def test_scanner_flags_a_planted_read():
    """The scanner itself: a read right after an MFMA is flagged, the same
    read behind enough wait states and an exact accumulation chain are not."""
    mfma = "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]"
    assert _hazards([mfma, "v_accvgpr_read_b32 v20, a5"])
    assert not _hazards([mfma, "s_nop 7", "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v20, a5"])
    assert not _hazards([mfma, "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]"])
    assert _hazards([mfma, "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[6:9]"])
    assert _hazards(["v_accvgpr_write_b32 a4, 0", mfma])
    assert not _hazards(["v_accvgpr_write_b32 a4, 0", "s_nop 1", mfma])
    # along a branch: the read at the branch target is found, behind the
    # fall-through's wait states it is not
    assert _hazards([mfma, "s_cbranch_scc1 .LBB0_1", "s_nop 7", "s_nop 7", "s_nop 7",
                     ".LBB0_1:", "v_accvgpr_read_b32 v20, a6"])
    assert not _hazards([mfma, "s_nop 7", "s_nop 7", "s_nop 7", "s_cbranch_scc1 .LBB0_1", "s_nop 7",
                         ".LBB0_1:", "v_accvgpr_read_b32 v20, a6"])
