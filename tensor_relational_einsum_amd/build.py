"""Builds libjagg.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libjagg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["abi.cpp", "relayout.hip", "join.hip", "elementwise.hip", "stream.hip", "flat.hip", "attention.hip", "contract_bf16.hip", "contract_f32.hip", "norm.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # keep the compiler from forming packed fp32 ops
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


CALIB_LIB = os.path.join(HERE, "libjagg_calib.so")


def build_calib() -> str:
    """libjagg_calib.so: the matrix-core probe the benchmark measures the
    machine's MFMA rate with (include/jagg_calib.h)."""
    tmp = CALIB_LIB + ".tmp"
    subprocess.run([HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "calib.hip"), "-o", tmp], check=True)
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "is not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text, file=sys.stderr)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    build_calib()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
