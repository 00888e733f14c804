"""Compile the gfx950 HIP sources into ``libsdtw.so`` (in-tree, beside this file),
and the same sources with SDTW_STRESS=1 into ``libsdtw_stress.so`` (pseudo-random
delays at every hand-off, for the stress tests only).

    python -m differentiable_series_alignment_amd.build [-v]

hipcc cross-compiles for gfx950 without a GPU.  Packed fp32 instructions are
disabled for the device code (``-packed-fp32-ops``); the host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsdtw.so")
# Debug build of the same sources with pseudo-random sleeps at every hand-off
# (SDTW_STRESS=1): loaded only by the hand-off stress tests.
STRESS_LIB = os.path.join(HERE, "libsdtw_stress.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _cmd(out: str, extra) -> list:
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC, *extra, *sources(), "-o", out]


def build(verbose: bool = False, extra=(), stress: bool = True) -> str:
    """Builds libsdtw.so and (stress=True) the stress variant, the two
    compilations side by side; returns the path of libsdtw.so."""
    jobs = [(LIB, tuple(extra))]
    if stress:
        jobs.append((STRESS_LIB, tuple(extra) + ("-DSDTW_STRESS=1",)))
    procs = []
    for out, ex in jobs:
        cmd = _cmd(out + ".tmp", ex)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    noise = "is not a recognized feature for this target"
    errors = []
    for out, pr in procs:
        text, _ = pr.communicate()
        msgs = [ln for ln in text.splitlines() if ln.strip() and noise not in ln]
        if pr.returncode != 0:
            errors.append(f"{os.path.basename(out)}:\n" + "\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs))
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    for out, _ in procs:
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
