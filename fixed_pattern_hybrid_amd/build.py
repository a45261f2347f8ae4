"""Compile the HIP sources into the in-tree shared library libsaf_hybrid.so.

Usage: ``python -m fixed_pattern_hybrid_amd.build`` (or ``build()``).
Cross-compiles for gfx950 with hipcc; no GPU is needed to build.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsaf_hybrid.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.hip", "kern_pattern.hip", "kern_fwd.hip", "kern_bwd.hip", "kern_f32.hip", "kern_pgrad.hip", "kern_fit.hip", "kern_calib.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax/rescale VALU work touches them
    # every tile, and AGPR accumulators would need a copy each way
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        ln for ln in p.stdout.splitlines() if "is not a recognized feature for this target" not in ln
    )
    return p.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
            failed = True
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB_PATH + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
