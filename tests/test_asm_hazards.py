"""The backward kernels accumulate dK / dV with MFMAs written as inline asm
(AGPR accumulators).  The compiler inserts no wait states for asm, and an
MFMA that reads a VGPR written by a vector ALU instruction needs two, so the
compiled code must never place such a write in the two instructions before
one of these MFMAs.  This test compiles the backward source to gfx950
assembly (no GPU needed) and scans every such MFMA."""
import os
import re
import shutil
import subprocess

import pytest

from blockwise_ring_attention_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _hazards(asm_lines):
    found = []
    prev = []  # instructions since the last label, newest last
    for line in asm_lines:
        if re.match(r"^\.?[A-Za-z_$][\w.$]*:", line):
            # a block start: keep the fall-through predecessor unless the
            # previous block ended in an unconditional jump
            if prev and re.match(r"\s+s_(branch|endpgm|setpc)", prev[-1]):
                prev = []
            continue
        if not re.match(r"\s+[a-z]", line) or line.strip().startswith(";"):
            continue
        m = re.match(r"\s+v_mfma_\S+\s+a\[\d+:\d+\],\s*(v\[\d+:\d+\]|v\d+),\s*(v\[\d+:\d+\]|v\d+)", line)
        if m:
            srcs = _vregs(m.group(1)) | _vregs(m.group(2))
            for p in prev[-2:]:
                pm = re.match(r"\s+(v_\w+)\s+(v\[\d+:\d+\]|v\d+)", p)
                if pm and not pm.group(1).startswith("v_mfma") and _vregs(pm.group(2)) & srcs:
                    found.append((p.strip(), line.strip()))
        if re.match(r"\s+s_nop\s+([1-9]|1[0-5])\b", line):
            prev = []  # two or more wait states
        else:
            prev.append(line)
    return found


def test_agpr_mfma_operands_have_wait_states(tmp_path):
    src = os.path.join(build.CSRC, "bwd_bf16.hip")
    out = tmp_path / "bwd.s"
    cmd = [build._hipcc(), *build.FLAGS, *build.SOURCE_FLAGS.get("bwd_bf16.hip", []), "-x", "hip",
           "--cuda-device-only", "-S", src, "-o", str(out)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = out.read_text().splitlines()
    n_acc = sum(1 for l in lines if re.match(r"\s+v_mfma_\S+\s+a\[", l))
    assert n_acc > 0, "no AGPR-accumulating MFMA found: the scan would prove nothing"
    bad = _hazards(lines)
    assert not bad, f"{len(bad)} VALU writes right before an asm MFMA, e.g. {bad[:3]}"


def test_scanner_catches_a_planted_hazard():
    planted = ["\tv_mov_b32_e32 v5, v7", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    assert _hazards(planted)
    padded = ["\tv_mov_b32_e32 v5, v7", "\ts_nop 1", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"]
    assert not _hazards(padded)
