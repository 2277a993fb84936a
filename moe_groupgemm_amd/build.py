"""Build the HIP library ``libmoe_mk.so`` (megakernel + C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_mk.so")
SOURCES = [os.path.join(HERE, "csrc", "megakernel.hip"), os.path.join(HERE, "csrc", "host.cpp")]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         # no packed fp32 instructions anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, *SOURCES, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
