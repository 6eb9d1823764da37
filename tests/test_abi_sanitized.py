"""The library's host-side checks under AddressSanitizer and UBSan (every check
fatal): libsvd's sources are rebuilt with the sanitizers on the host code only
(the gfx950 code is unchanged), and tests/abi_sanitized_run.py calls every C
entry point with arguments its checks reject, dtype and rule values outside
the enumerators included, in a child process with clang's sanitizer runtime
preloaded.  It must run clean and return the product library's status codes.
No HIP call is reached, so no GPU is needed."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUN = os.path.join(ROOT, "tests", "abi_sanitized_run.py")
CSRC = os.path.join(ROOT, "lossless_draft_verification_verifier_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _runtime():
    try:
        res = subprocess.run([CLANG, "--print-resource-dir"], capture_output=True, text=True,
                             check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    hits = glob.glob(os.path.join(res, "lib", "*", "libclang_rt.asan*x86_64*.so"))
    return hits[0] if hits else None


def _run(lib, env):
    r = subprocess.run([sys.executable, RUN, lib], env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout.strip().splitlines(), r.stderr


def test_host_checks_run_clean_under_sanitizers(tmp_path):
    rt = _runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    lib = str(tmp_path / "libsvd_hostsan.so")
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-fast-math",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC] + san +
                   ["-shared-libsan", "-o", lib, os.path.join(CSRC, "svd_api.hip"),
                    os.path.join(CSRC, "svd_noalloc.hip")], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out, err = _run(lib, env)
    assert rc == 0, err[-4000:]
    product = os.path.join(ROOT, "lossless_draft_verification_verifier_amd", "libsvd.so")
    rc0, out0, err0 = _run(product, dict(os.environ))
    assert rc0 == 0, err0[-4000:]
    assert out[-1] == out0[-1]
