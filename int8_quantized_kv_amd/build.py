"""Compile the gfx950 HIP library libdattn.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdattn.so")
SOURCES = [os.path.join(CSRC, "dattn.hip")]
ARCH = os.environ.get("DATTN_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: str) -> list:
    return [
        os.environ.get("HIPCC", "hipcc"), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU ops stay off: the compiler emits them from plain float code otherwise
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
