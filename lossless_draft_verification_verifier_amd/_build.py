"""Build the HIP libraries for gfx950 with hipcc (in-tree, next to this file).

libsvd.so        the product library (include/svd.h); keeps no state between calls
libsvd_timed.so  the same sources with kernel timing compiled in
                 (include/svd_timing.h), for benchmarks and profiles
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsvd.so")
TIMED_LIB = os.path.join(PKG, "libsvd_timed.so")
SOURCES = [os.path.join(CSRC, "svd_api.hip"), os.path.join(CSRC, "svd_noalloc.hip")]
TIMED_SOURCES = SOURCES + [os.path.join(CSRC, "svd_timing.hip")]
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


def _compile(out: str, sources, defines=(), verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-o", tmp] + list(sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, out: str = LIB, defines=(), timed_out: str = TIMED_LIB) -> str:
    """Compile both libraries (in parallel); returns the product library's path.
    timed_out=None skips the timing build."""
    jobs = [(out, SOURCES, tuple(defines))]
    if timed_out:
        jobs.append((timed_out, TIMED_SOURCES, tuple(defines) + ("SVD_KERNEL_TIMING",)))
    with ThreadPoolExecutor(len(jobs)) as ex:
        for f in [ex.submit(_compile, o, s, d, verbose) for o, s, d in jobs]:
            f.result()
    return out


if __name__ == "__main__":
    print(build(verbose=True))
