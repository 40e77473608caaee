"""Build ``libdfv.so`` (gfx950 kernels + C ABI) in-tree with hipcc.

Run ``python -m long_context_split_amd.build`` or call :func:`build`.  The
library lands next to this file; the ctypes binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdfv.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# measurement probe (page-read ceiling), loaded only by the benchmark
PROBE_NAME = "libdfv_probe.so"
PROBE_PATH = os.path.join(PKG, PROBE_NAME)
PROBE_SOURCES = ["probe_kernel.hip"]
ARCH = "gfx950"

SOURCES = ["split_kernel.hip", "combine_kernel.hip", "qk_kernel.hip", "kv_append_kernel.hip", "dfv_api.cpp",
           "noalloc.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # packed FP32 instructions stay off: the compiler's own plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the split kernel's O tiles otherwise bounce
    # between VGPRs and AGPRs every key tile
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _link(sources, exports, out_path, verbose):
    with tempfile.TemporaryDirectory() as tmp:
        vs = os.path.join(tmp, "exports.map")
        with open(vs, "w") as f:
            f.write("{ global: %s; local: *; };\n" % exports)
        out_tmp = os.path.join(tmp, os.path.basename(out_path))
        cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
               *[os.path.join(CSRC, s) for s in sources],
               f"-Wl,--version-script={vs}", "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed building {os.path.basename(out_path)}")
        shutil.move(out_tmp, out_path)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the libraries; returns the path of libdfv.so."""
    _link(SOURCES, "dfv_*", LIB_PATH, verbose)
    _link(PROBE_SOURCES, "dfv_probe_*", PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
