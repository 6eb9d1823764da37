"""The C ABI without a GPU: the library loads, exports every function that
include/svd.h declares, sizes its workspace, and rejects bad arguments on the
host before any HIP call.  The timing build exports svd.h and svd_timing.h;
the product library exports no timing call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svd.h")
TIMING_HEADER = os.path.join(ROOT, "include", "svd_timing.h")


@pytest.fixture(scope="module")
def svd():
    pkg = os.path.join(ROOT, "lossless_draft_verification_verifier_amd")
    if not all(os.path.exists(os.path.join(pkg, f)) for f in ("libsvd.so", "libsvd_timed.so")):
        from lossless_draft_verification_verifier_amd import _build
        _build.build()
    import lossless_draft_verification_verifier_amd as m
    return m


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(svd_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("svd_verify", "svd_select_and_verify", "svd_workspace_bytes", "svd_strerror",
              "svd_greedy_verify", "svd_greedy_select_and_verify"):
        assert n in names


def test_every_declared_symbol_is_exported(svd):
    lib = ctypes.CDLL(svd.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", svd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (svd_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(svd.C_EXPORTS) == set(declared_functions())
    # the product library keeps no timing state and exports no timing call
    assert not exported & set(declared_functions(TIMING_HEADER))


def test_timing_build_exports_both_headers(svd):
    out = subprocess.run(["nm", "-D", "--defined-only", svd.TIMED_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (svd_\w+)", out))
    timing = set(declared_functions(TIMING_HEADER))
    assert timing == set(svd.TIMING_EXPORTS)
    assert set(declared_functions()) | timing <= exported
    t = svd.timing_library()
    assert t.svd_workspace_bytes(256, 1, 8, 152064) == svd.svd_workspace_bytes(256, 1, 8, 152064)
    assert t.svd_profile_enable(()) == svd.SVD_OK
    ms, n = t.svd_profile_read()
    assert ms == [0.0] * len(svd.KERNELS) and n == [0] * len(svd.KERNELS)
    with pytest.raises(RuntimeError):
        svd._default.svd_profile_read()


def test_product_library_has_no_mutable_namespace_scope_state():
    # every object with static storage in the product library's source is
    # const or constexpr (the timing state lives in svd_timing.hip only)
    src = open(os.path.join(ROOT, "lossless_draft_verification_verifier_amd", "csrc",
                            "svd_api.hip")).read()
    src = re.sub(r"//[^\n]*", "", src)
    assert "g_prof" not in src and "Profiler" not in src
    assert not re.search(r"^static\s+(?!const|constexpr|inline)", src, flags=re.M)


def test_workspace_bytes(svd):
    a = svd.svd_workspace_bytes(256, 1, 8, 152064)
    b = svd.svd_workspace_bytes(512, 1, 8, 152064)
    c = svd.svd_workspace_bytes(256, 16, 32, 152064)
    assert 0 < a < b and a < c
    assert a % 256 == 0
    # well below the logits it serves: under 1% of one batch of bf16 rows
    assert a < 0.01 * 256 * 8 * 2 * 152064 * 2
    assert svd.svd_workspace_bytes(1, 1, 1, 1) > 0
    for bad in [(0, 1, 1, 1), (1, 0, 1, 1), (1, 1, 0, 1), (1, 1, 1, 0), (1, 65, 1, 1),
                (1, 1, 4097, 1), (1 << 40, 1, 1, 1)]:
        assert svd.svd_workspace_bytes(*bad) == 0, bad


def test_strerror(svd):
    for st in (0, -1, -2, -3, -4, -5):
        assert isinstance(svd.svd_strerror(st), str) and svd.svd_strerror(st)
    assert svd.svd_strerror(12345) == "unknown status"


def _call(svd, **kw):
    # fake, never dereferenced addresses: validation returns before any HIP call
    a = dict(p=4096, q=8192, d=12288, dtype=svd.SVD_BF16, B=2, K=2, G=3, V=100, tp=1.0, tq=1.0,
             sel=16384, L=20480, tok=24576, ws=1 << 20, n=0)
    a.update(kw)
    return svd.svd_select_and_verify(a["p"], a["q"], a["d"], a["dtype"], a["B"], a["K"], a["G"],
                                     a["V"], a["tp"], a["tq"], 0, 0, a["sel"], a["L"], a["tok"],
                                     None, None, None, a["ws"], a["n"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(p=None), -1), (dict(q=None), -1), (dict(d=None), -1), (dict(sel=None), -1),
    (dict(L=None), -1), (dict(tok=None), -1), (dict(ws=None), -1),
    (dict(dtype=2), -2), (dict(B=0), -1), (dict(K=0), -1), (dict(K=65), -1), (dict(G=0), -1),
    (dict(G=4097), -1), (dict(V=0), -1), (dict(tp=0.0), -1), (dict(tq=-1.0), -1),
    (dict(tp=float("nan")), -1), (dict(tq=float("inf")), -1), (dict(ws=(1 << 20) + 64), -1),
    # log2(e)/T overflows fp32 below T ~ 4.2e-39 (a subnormal temperature)
    (dict(tp=1e-40), -1), (dict(tq=4.0e-39), -1), (dict(tp=1e-45), -1),
    (dict(tp=4.5e-39), -3),  # still a valid temperature: only the workspace is missing
    (dict(), -3),  # workspace of 0 bytes
])
def test_host_side_argument_errors(svd, kw, want):
    assert _call(svd, **kw) == want


def test_verify_argument_errors(svd):
    ws = 1 << 20
    rc = svd.svd_verify(4096, 8192, None, svd.SVD_BF16, 1, 2, 10, 1.0, 1.0, 0, 0, 16384, 20480,
                        None, None, ws, 0, None)
    assert rc == svd.SVD_EINVAL
    rc = svd.svd_verify(4096, 8192, 12288, svd.SVD_F32, 1, 2, 10, 1.0, 1.0, 0, 0, 16384, 20480,
                        None, None, ws, 0, None)
    assert rc == svd.SVD_EWORKSPACE


def _greedy(svd, **kw):
    a = dict(p=4096, d=12288, dtype=svd.SVD_BF16, B=2, K=2, G=3, V=100, tp=1.0, sel=16384,
             L=20480, tok=24576, ws=1 << 20, n=0)
    a.update(kw)
    return svd.svd_greedy_select_and_verify(a["p"], a["d"], a["dtype"], a["B"], a["K"], a["G"],
                                            a["V"], a["tp"], 0, 0, a["sel"], a["L"], a["tok"],
                                            None, None, a["ws"], a["n"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(p=None), -1), (dict(d=None), -1), (dict(sel=None), -1), (dict(L=None), -1),
    (dict(tok=None), -1), (dict(ws=None), -1), (dict(dtype=7), -2), (dict(B=0), -1),
    (dict(K=65), -1), (dict(G=0), -1), (dict(V=0), -1), (dict(tp=0.0), -1),
    (dict(tp=float("inf")), -1), (dict(ws=(1 << 20) + 32), -1), (dict(tp=2e-39), -1),
    (dict(), -3),  # workspace of 0 bytes
])
def test_greedy_host_side_argument_errors(svd, kw, want):
    assert _greedy(svd, **kw) == want


def test_greedy_verify_argument_errors(svd):
    rc = svd.svd_greedy_verify(4096, None, svd.SVD_BF16, 1, 2, 10, 1.0, 0, 0, 16384, 20480, None,
                               1 << 20, 0, None)
    assert rc == svd.SVD_EINVAL
    rc = svd.svd_greedy_verify(4096, 12288, svd.SVD_F32, 1, 2, 10, 1.0, 0, 0, 16384, 20480, None,
                               1 << 20, 0, None)
    assert rc == svd.SVD_EWORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    # a copy of the package without libsvd.so must refuse to import
    import shutil
    import sys
    src = os.path.join(ROOT, "lossless_draft_verification_verifier_amd", "__init__.py")
    pkg = tmp_path / "svdcopy"
    pkg.mkdir()
    shutil.copy(src, pkg / "__init__.py")
    code = "import sys; sys.path.insert(0, %r); import svdcopy" % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode != 0 and "libsvd.so is not built" in r.stderr


def test_profile_kernel_names_follow_the_header(svd):
    # the binding's KERNELS tuple is indexed by the timing header's SVD_KERNEL_* ids
    text = open(TIMING_HEADER).read()
    ids = {m.group(1).lower(): int(m.group(2))
           for m in re.finditer(r"SVD_KERNEL_([A-Z_]+) = (\d+)", text)}
    count = ids.pop("count")
    assert len(svd.KERNELS) == count
    assert {name: i for i, name in enumerate(svd.KERNELS)} == ids


def test_noalloc_host_side_errors(svd):
    # sizes are checked on the host before any HIP call (fake addresses)
    def call(B, K, G, V):
        return svd.svd_select_and_verify_noalloc(4096, 8192, 12288, svd.SVD_BF16, B, K, G, V, 1.0,
                                                 1.0, 0, 0, 16384, 20480, 24576, None, None,
                                                 None, None)
    assert svd.svd_workspace_bytes(2048, 1, 8, 152064) > svd.SVD_NOALLOC_SCRATCH_BYTES
    assert call(2048, 1, 8, 152064) == svd.SVD_ESCRATCH
    for bad in [(0, 1, 8, 100), (1, 65, 8, 100), (1, 1, 0, 100), (1, 1, 8, 0)]:
        assert call(*bad) == svd.SVD_EINVAL, bad
    # every other argument error too, before the scratch array's lookup (a HIP call)
    def call2(dtype=svd.SVD_BF16, tp=1.0, sel=16384):
        return svd.svd_select_and_verify_noalloc(4096, 8192, 12288, dtype, 2, 1, 8, 100, tp, 1.0,
                                                 0, 0, sel, 20480, 24576, None, None, None, None)
    assert call2(dtype=5) == svd.SVD_EDTYPE
    assert call2(tp=0.0) == svd.SVD_EINVAL
    assert call2(sel=None) == svd.SVD_EINVAL
    text = open(HEADER).read()
    assert "#define SVD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert svd.SVD_NOALLOC_SCRATCH_BYTES == 16 << 20


def test_adl_host_side_errors(svd):
    # fake addresses: every rejection happens before any HIP call
    def call(**kw):
        a = dict(d=4096, sel=8192, L=12288, gb=None, eos=-1, B=4, K=2, G=8, k_min=1, k_max=16,
                 step=4, shift=2, slack=64, avg=16384, nxt=20480)
        a.update(kw)
        return svd.svd_adl_next(a["d"], a["sel"], a["L"], a["gb"], a["eos"], a["B"], a["K"],
                                a["G"], a["k_min"], a["k_max"], a["step"], a["shift"], a["slack"],
                                a["avg"], a["nxt"], None)
    for kw in (dict(d=None), dict(sel=None), dict(L=None), dict(avg=None), dict(nxt=None),
               dict(B=0), dict(K=0), dict(K=65), dict(G=0), dict(G=4097), dict(k_min=0),
               dict(k_min=9, k_max=8), dict(k_max=4097), dict(step=-1), dict(step=4097),
               dict(shift=-1), dict(shift=17), dict(slack=-1), dict(slack=(1 << 20) + 1)):
        assert call(**kw) == svd.SVD_EINVAL, kw
