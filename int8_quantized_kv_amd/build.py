"""Compile the gfx950 HIP library libdattn.so in-tree with hipcc.

The host code (dattn.hip) and the four kernel units (kernels.hip for each
head_dim x softcap pair) compile in parallel into objects under _build/,
which are then linked into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdattn.so")
OBJDIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("DATTN_OFFLOAD_ARCH", "gfx950")

# (object name, source, extra defines)
UNITS = [("dattn", "dattn.hip", [])] + [
    (f"kernels_d{d}_cap{c}", "kernels.hip", [f"-DDATTN_D={d}", f"-DDATTN_CAP={c}"])
    for d in (64, 128) for c in (0, 1)
] + [
    (f"shared_d{d}_cap{c}", "kernels.hip", [f"-DDATTN_D={d}", f"-DDATTN_CAP={c}", "-DDATTN_SHARED=1"])
    for d in (64, 128) for c in (0, 1)
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "hipcc")


def compile_command(src: str, obj: str, defines: list) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
        # packed fp32 VALU ops stay off: the compiler emits them from plain float code otherwise
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, *defines, os.path.join(CSRC, src), "-o", obj,
    ]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd: list) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs, cmds = [], []
    for name, src, defines in UNITS:
        obj = os.path.join(OBJDIR, name + ".o")
        objs.append(obj)
        cmds.append(compile_command(src, obj, defines))
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    cmd = link_command(objs, tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
