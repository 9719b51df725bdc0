"""Compile libbsa.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libbsa.so")
SOURCES = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 ops stay off: the kernels are written for scalar fp32 VALU
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, *extra, *SOURCES, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libbsa.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
