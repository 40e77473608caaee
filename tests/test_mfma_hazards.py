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

# Wait states needed between an XDL MFMA that writes a VGPR and the first
# VALU, LDS, memory or MFMA source-A/B read of it.  The CDNA3 ISA's MAI
# dependency table gives passes + 3 for this case (2, 4, 8, 16 passes -> 5, 7,
# 11, 19); gfx950 needs one more once an MFMA has more than two passes.  The
# compiler's own hazard model agrees on the one MFMA these kernels use: it
# places s_nop 7 (8 wait states) between v_mfma_f32_16x16x32_f16, a 4-pass XDL
# operation on gfx950, and a VALU reader of its result.  An MFMA missing from
# the table fails the scan, so the table grows with the kernels.
XDL_PASSES = {
    "v_mfma_f32_16x16x32_f16": 4,
    "v_mfma_f32_16x16x32_bf16": 4,
    "v_mfma_f32_32x32x16_f16": 8,
    "v_mfma_f32_32x32x16_bf16": 8,
}


def required_wait_states(op):
    if op not in XDL_PASSES:
        raise KeyError(f"no pass count for {op}: add it to XDL_PASSES")
    p = XDL_PASSES[op]
    return p + 3 + (1 if p > 2 else 0)


MIN_WAIT_STATES = None   # None: each MFMA's own requirement from XDL_PASSES
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
    reached with fewer wait states than that MFMA needs (min_ws, when given,
    replaces the per-MFMA requirement) along some path."""
    ins, labels = _parse(text)
    found = []

    def walk(j, dst, ws, depth, seen, src, need):
        while j < len(ins) and ws < need:
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
                    walk(labels[tgt], dst, ws + 1, depth + 1, seen, src, need)
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
            need = required_wait_states(t[0]) if min_ws is None else min_ws

            walk(i + 1, _regs(t[1]), 0, 0, set(), i, need)
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


def test_requirement_follows_the_pass_count():
    # an 8-pass MFMA read after ten wait states is still too early (it needs 12);
    # a 4-pass one is too early after seven and fine after eight
    planted = """
    v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], v[20:23], v[0:15]
    s_nop 7
    s_nop 1
    v_add_f32_e32 v30, v1, v31
    s_endpgm
"""
    bad = early_reads(planted)
    assert len(bad) == 1 and bad[0][2] == 10
    four = """
    v_mfma_f32_16x16x32_f16 v[4:7], v[8:11], a[0:3], v[4:7]
    s_nop 6
    v_add_f32_e32 v30, v5, v31
    s_endpgm
"""
    assert [b[2] for b in early_reads(four)] == [7]
    assert early_reads(four.replace("s_nop 6", "s_nop 7")) == []


def test_unknown_mfma_is_refused():
    with pytest.raises(KeyError):
        early_reads("    v_mfma_f32_4x4x4_16b_f16 v[0:3], v[4:5], v[6:7], v[0:3]\n    s_endpgm\n")
