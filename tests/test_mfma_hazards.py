"""MFMA result hazards in the emitted gfx950 code (CPU only; needs hipcc).

The hardware does not interlock a VALU, LDS or memory instruction that reads
the destination of an MFMA: the code must leave wait states between them.
The compiler inserts them, but a uniform branch between an MFMA and the
first reader of its result has been seen to leave the branch-taken path
without them, which made results depend on code layout.  These tests compile
the MFMA kernels to assembly and follow every path (taken branches included)
from each MFMA to the first instruction that reads its result.
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_split_amd import build as B

MIN_WAIT_STATES = 8   # below anything the compiler leaves on a straight-line path in these kernels
_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)")


def _regs(tok):
    m = _REG.fullmatch(tok)
    if not m:
        return set()
    if m.group(1):
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok}


def _parse(text):
    ins, labels = [], {}
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            labels[line[:-1]] = len(ins)
            continue
        if line.startswith("."):
            continue
        ins.append(re.split(r"[ ,]+", line))
    return ins, labels


def early_reads(text, min_ws=MIN_WAIT_STATES):
    """(mfma index, reader text, wait states) for every read of an MFMA result
    reached with fewer than min_ws wait states along some path."""
    ins, labels = _parse(text)
    found = []

    def walk(j, dst, ws, depth, seen, src):
        while j < len(ins) and ws < min_ws:
            t = ins[j]
            op = t[0]
            if op == "s_nop":
                ws += int(t[1]) + 1
                j += 1
                continue
            if op == "s_endpgm":
                return
            if op.startswith(("s_cbranch", "s_branch")):
                tgt = t[1]
                if tgt in labels and depth < 4 and (tgt, ws) not in seen:
                    seen.add((tgt, ws))
                    walk(labels[tgt], dst, ws + 1, depth + 1, seen, src)
                if op == "s_branch":
                    return
                ws += 1
                j += 1
                continue
            if op.startswith("v_mfma"):
                if set().union(*map(_regs, t[2:4])) & dst:      # read as A or B operand
                    found.append((src, " ".join(t), ws))
                    return
                if _regs(t[1]) & dst:                            # accumulates onto it: new result
                    return
                ws += 1
                j += 1
                continue
            if set().union(*map(_regs, t[2:])) & dst:
                found.append((src, " ".join(t), ws))
                return
            if len(t) > 1 and (_regs(t[1]) & dst) and op.startswith("v_"):
                return                                           # overwritten first
            ws += 1
            j += 1

    for i, t in enumerate(ins):
        if t[0].startswith("v_mfma"):
            walk(i + 1, _regs(t[1]), 0, 0, set(), i)
    return found


def _device_asm(source):
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = subprocess.run([B.hipcc(), *flags, "--offload-device-only", "-S", f"-I{B.INCLUDE}", f"-I{B.CSRC}",
                          os.path.join(B.CSRC, source), "-o", "-"], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    return out.stdout


needs_hipcc = pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                                 reason="hipcc not available")


@needs_hipcc
@pytest.mark.parametrize("source", ["split_kernel.hip", "qk_kernel.hip"])
def test_no_mfma_result_read_too_early(source):
    text = _device_asm(source)
    assert text.count("v_mfma") > 50
    bad = early_reads(text)
    assert not bad, f"{len(bad)} early reads, e.g. {bad[:3]}"


def test_scan_catches_a_read_on_the_taken_path():
    planted = """
    v_mfma_f32_16x16x32_f16 v[4:7], v[8:11], a[0:3], v[4:7]
    s_cbranch_vccnz .LBB0_2
    v_cndmask_b32_e64 v4, v4, v1, s[0:1]
    s_nop 7
    s_nop 3
.LBB0_2:
    v_max3_f32 v9, v9, v4, v5
    s_endpgm
"""
    bad = early_reads(planted)
    assert sorted(b[1].split()[0] for b in bad) == ["v_cndmask_b32_e64", "v_max3_f32"]   # both paths


def test_scan_accepts_enough_wait_states_and_accumulation():
    ok = """
    v_mfma_f32_16x16x32_f16 v[4:7], v[8:11], a[0:3], v[4:7]
    v_mfma_f32_16x16x32_f16 v[4:7], v[12:15], a[4:7], v[4:7]
    s_nop 7
    s_nop 3
    v_max3_f32 v9, v9, v4, v5
    s_endpgm
"""
    assert early_reads(ok) == []
