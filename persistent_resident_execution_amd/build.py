"""Build the engine's shared library (libpre.so) in-tree with hipcc for gfx950.

    python -m persistent_resident_execution_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpre.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["engine.hip", "plan.cpp"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    # packed fp32 vector ops stay off: plain fp32 FMAs only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 into libpre.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out: str) -> None:
    """Write the gfx950 assembly of engine.hip to `out` (for reading VGPR use)."""
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           "-o", out, os.path.join(CSRC, "engine.hip")]
    subprocess.check_call(cmd)


if __name__ == "__main__":
    print(build(verbose=True))
