"""Build libkda.so (all HIP sources, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
STAMPS_LIB = os.path.join(PKG, "libkda_stamps.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed fp32 arithmetic stays off on this hardware (hand-written or compiler-generated)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators stay in ordinary VGPRs (the scan reads them on the vector ALUs every step)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _cmd(out: str, defines=()) -> list:
    return [HIPCC, *FLAGS, *defines, "-I", INCLUDE, "-I", CSRC, "-o", out, *sources()]


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ into chunked_gated_delta_amd/libkda.so, and beside it
    libkda_stamps.so, the same library with the segment pass's phase stamps compiled in (a
    measurement build that bench.py --phase-stamps loads; the product never does).  Always rebuilds;
    the two compile in parallel."""
    jobs = [(LIB, []), (STAMPS_LIB, ["-DKDA_PHASE_STAMPS=1"])]
    procs = []
    for out, defines in jobs:
        cmd = _cmd(out + ".tmp", defines)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    noise = "is not a recognized feature for this target"
    failed = []
    for (out, _), pr in zip(jobs, procs):
        text, _ = pr.communicate()
        msgs = [ln for ln in text.splitlines() if noise not in ln]
        if pr.returncode != 0:
            failed.append(f"hipcc failed for {os.path.basename(out)}:\n" + "\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs), file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(failed))
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
