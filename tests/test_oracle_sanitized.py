"""The oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer (every
check fatal): tests/oracle_sanitized_run.py drives every entry point through
the edge cases the rules define (NaN, +inf and all -inf rows, out-of-range
tokens and pool indices, planted EOS, ties at the top, forced decisions, one
and two threads) against a sanitizer build of svd_oracle.c, in a child process
with the sanitizer runtime preloaded.  It must run clean and give the same bits
as the normal build."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUN = os.path.join(ROOT, "tests", "oracle_sanitized_run.py")
SRC = os.path.join(ROOT, "oracle", "svd_oracle.c")


def _run(env):
    r = subprocess.run([sys.executable, RUN], env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout.split(), r.stderr


def test_oracle_runs_clean_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O2", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib, SRC,
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, SVD_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out, err = _run(env)
    assert rc == 0, err[-4000:]
    assert out[0] == lib  # the sanitizer build was the one loaded
    plain = dict(os.environ)
    plain.pop("SVD_ORACLE_LIB", None)
    rc0, out0, err0 = _run(plain)
    assert rc0 == 0, err0[-4000:]
    assert out[1] == out0[1]  # the same bits as the normal build
