"""Build libtclora.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m tenant_composite_lora_amd.build   (or build() from Python)
The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtclora.so")
SOURCES = ["plan.hip", "apply.hip", "tile.hip", "pack.hip", "gate.hip", "factor.hip", "sched.cpp", "host.cpp"]
ARCH = os.environ.get("TCL_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 VALU forms are switched off for the device code: the compiler
# otherwise forms them from plain float code on gfx950.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = True, jobs: int = 4) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs, verbose)
            procs = []
    _wait(procs, verbose)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout)
    os.replace(tmp, LIB)
    return LIB


def _wait(procs, verbose):
    errs = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln
                 and "is not a recognized feature" not in ln]
        if verbose and lines:
            print("\n".join(lines), flush=True)
        if p.returncode != 0:
            errs.append(f"{src}: hipcc failed\n{text}")
    if errs:
        raise RuntimeError("\n".join(errs))


if __name__ == "__main__":
    path = build(verbose="-q" not in sys.argv)
    print(path)
