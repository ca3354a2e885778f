"""Build libep_mi355x.so in-tree with hipcc for gfx950.

    python -m combine_ep_plan_02_amd.build

One translation unit (csrc/ep_abi.hip includes the kernel headers), so the
device error word needs no relocatable device code.  Packed-fp32 instructions
are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ep_abi.hip")
HEADERS = [os.path.join(PKG, "csrc", h) for h in
           ("ep_common.h", "ep_plan_kernels.h", "ep_row_kernels.h")] + \
          [os.path.join(ROOT, "include", "ep_mi355x.h")]
LIB = os.path.join(PKG, "libep_mi355x.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            "-o", out, SRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libep_mi355x.so")
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in [SRC] + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
