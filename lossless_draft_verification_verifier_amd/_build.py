"""Build libsvd.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsvd.so")
SOURCES = [os.path.join(CSRC, "svd_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions stay off (-packed-fp32-ops); no fast-math anywhere,
# so the fp64 draw rounds as written.
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-Wall", "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
