"""Compile libmsa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and
beside it libmsa_timeline.so: the same sources with -DMSA_TIMELINE, which adds
the wall-clock marks and the two read-out calls of include/msa_timeline.h
(a diagnostic build; the binding loads libmsa.so unless told otherwise)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmsa.so")
TIMELINE_LIB = os.path.join(PKG, "libmsa_timeline.so")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def command(out: str, timeline: bool = False):
    return ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: the epilogues (max-pool, softmax)
            # then read them without a v_accvgpr_read per value
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-result"] + (["-DMSA_TIMELINE"] if timeline else []) + [
            "-I", os.path.join(ROOT, "include"), "-I", CSRC] + sources() + ["-o", out]


def build(verbose: bool = False, timeline: bool = True) -> str:
    """Builds libmsa.so and (timeline) libmsa_timeline.so, the two hipcc runs
    side by side; returns the path of libmsa.so.  Each library replaces the
    old one only once its own build has succeeded."""
    targets = [(LIB, False)] + ([(TIMELINE_LIB, True)] if timeline else [])
    procs = []
    for lib, tl in targets:
        cmd = command(lib + ".tmp", timeline=tl)
        if verbose:
            print(" ".join(cmd))
        procs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    noise = "is not a recognized feature for this target"
    failed = []
    for lib, p in procs:
        _, stderr = p.communicate()
        err = "\n".join(l for l in stderr.splitlines() if noise not in l)
        if p.returncode != 0:
            failed.append("%s:\n%s" % (os.path.basename(lib), err))
            continue
        if verbose and err.strip():
            print(err)
        os.replace(lib + ".tmp", lib)
    if failed:
        raise RuntimeError("hipcc failed for " + "\n".join(failed))
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
