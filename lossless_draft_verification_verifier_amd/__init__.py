"""Lossless draft verification with self-selection on MI355X (gfx950).

Thin ctypes binding over ``libsvd.so`` (C ABI in ``include/svd.h``).  Every step
of the verification runs in the library's HIP kernels; this module only
marshals arguments.  PyTorch supplies device memory and the current stream.

Raw entry points (same names and argument order as the C ABI; pointer
arguments take an int address or a tensor):
    svd_workspace_bytes, svd_verify, svd_select_and_verify, svd_greedy_verify,
    svd_greedy_select_and_verify, svd_rows_workspace_bytes, svd_select_and_verify_rows,
    svd_verify_window, svd_cps_workspace_bytes, svd_cps_lattice, svd_cps_beam,
    svd_adl_next, svd_select_and_verify_noalloc, svd_strerror
Tensor conveniences that allocate the outputs and the workspace with torch:
    verify, select_and_verify, greedy_verify, greedy_select_and_verify,
    select_and_verify_rows, verify_window, cps_lattice, cps_beam, adl_next, workspace_bytes
Kernel timing: timing_library() loads ``libsvd_timed.so`` (the same kernels with
HIP-event timing compiled in, ``include/svd_timing.h``) as a Library whose raw
entry points are those above plus svd_profile_enable and svd_profile_read.

Importing fails with ImportError when ``libsvd.so`` has not been built; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsvd.so")
TIMED_LIB_PATH = os.path.join(_PKG, "libsvd_timed.so")

SVD_F32, SVD_BF16 = 0, 1
SVD_OK, SVD_EINVAL, SVD_EDTYPE, SVD_EWORKSPACE, SVD_EHIP, SVD_ESCRATCH = 0, -1, -2, -3, -4, -5
SVD_NOALLOC_SCRATCH_BYTES = 16 << 20
SVD_MAX_K, SVD_MAX_GAMMA = 64, 4096
# kernel ids of the timing build (SVD_KERNEL_* in include/svd_timing.h)
KERNELS = ("rowstats", "select", "draw_pass", "draw_pick", "beta", "mark", "pool_stats",
           "alpha_rows", "lattice", "beam", "lattice_len", "combine", "rowstats_split",
           "rowstats_live", "adl", "beta_combine")
SVD_RULE_STANDARD, SVD_RULE_GREEDY = 0, 1

C_EXPORTS = ("svd_workspace_bytes", "svd_verify", "svd_select_and_verify", "svd_greedy_verify",
             "svd_greedy_select_and_verify", "svd_rows_workspace_bytes",
             "svd_select_and_verify_rows", "svd_verify_window", "svd_cps_workspace_bytes",
             "svd_cps_lattice", "svd_cps_beam", "svd_adl_next", "svd_select_and_verify_noalloc",
             "svd_strerror")
TIMING_EXPORTS = ("svd_profile_enable", "svd_profile_read")

_M64 = 0xFFFFFFFFFFFFFFFF


class SvdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, svd_strerror(status), status))


def _declare(L: ctypes.CDLL, timing: bool) -> ctypes.CDLL:
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
    L.svd_workspace_bytes.restype = sz
    L.svd_workspace_bytes.argtypes = [i64, i32, i32, i32]
    L.svd_verify.restype = ctypes.c_int
    L.svd_verify.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, i32, f32, f32, u64, u64,
                             vp, vp, vp, vp, vp, sz, vp]
    L.svd_select_and_verify.restype = ctypes.c_int
    L.svd_select_and_verify.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, i32, i32, f32, f32,
                                        u64, u64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.svd_greedy_verify.restype = ctypes.c_int
    L.svd_greedy_verify.argtypes = [vp, vp, ctypes.c_int, i64, i32, i32, f32, u64, u64, vp, vp,
                                    vp, vp, sz, vp]
    L.svd_greedy_select_and_verify.restype = ctypes.c_int
    L.svd_greedy_select_and_verify.argtypes = [vp, vp, ctypes.c_int, i64, i32, i32, i32, f32, u64,
                                               u64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.svd_rows_workspace_bytes.restype = sz
    L.svd_rows_workspace_bytes.argtypes = [i64, i32, i32, i32, i64, i64]
    L.svd_select_and_verify_rows.restype = ctypes.c_int
    L.svd_select_and_verify_rows.argtypes = [ctypes.c_int, vp, i64, vp, vp, i64, vp, vp,
                                             ctypes.c_int, i64, i32, i32, i32, f32, f32, u64, u64,
                                             vp, vp, vp, vp, vp, vp, sz, vp]
    L.svd_verify_window.restype = ctypes.c_int
    L.svd_verify_window.argtypes = [ctypes.c_int, vp, vp, vp, vp, i32, i32, ctypes.c_int, i64, i32,
                                    i32, i32, f32, f32, u64, u64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.svd_cps_workspace_bytes.restype = sz
    L.svd_cps_workspace_bytes.argtypes = [i64, i32]
    L.svd_cps_lattice.restype = ctypes.c_int
    L.svd_cps_lattice.argtypes = [vp, ctypes.c_int, i64, i32, i32, f32, f32, i32, i32, vp, vp, vp,
                                  vp, vp, sz, vp]
    L.svd_cps_beam.restype = ctypes.c_int
    L.svd_cps_beam.argtypes = [vp, vp, vp, vp, vp, f32, i64, i32, i32, i32, vp, vp, vp, vp]
    L.svd_adl_next.restype = ctypes.c_int
    L.svd_adl_next.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                               vp]
    L.svd_select_and_verify_noalloc.restype = ctypes.c_int
    L.svd_select_and_verify_noalloc.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, i32, i32, f32,
                                                f32, u64, u64, vp, vp, vp, vp, vp, vp, vp]
    L.svd_strerror.restype = ctypes.c_char_p
    L.svd_strerror.argtypes = [ctypes.c_int]
    if timing:
        L.svd_profile_enable.restype = ctypes.c_int
        L.svd_profile_enable.argtypes = [ctypes.c_uint]
        L.svd_profile_read.restype = ctypes.c_int
        L.svd_profile_read.argtypes = [vp, vp, ctypes.c_int]
    return L


def _addr(x):
    """Device address of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


class Library:
    """The raw C ABI of one built library (argument marshalling only)."""

    def __init__(self, path: str = LIB_PATH, timing: bool = False):
        if not os.path.exists(path):
            raise ImportError(
                "%s is not built (expected at %s); build it with __graft_entry__.build() or "
                "python -m lossless_draft_verification_verifier_amd._build"
                % (os.path.basename(path), path))
        self.path = path
        self.timing = timing
        self._lib = _declare(ctypes.CDLL(path), timing)

    def svd_workspace_bytes(self, B: int, K: int, gamma: int, V: int) -> int:
        return int(self._lib.svd_workspace_bytes(B, K, gamma, V))

    def svd_verify(self, p_logits, q_logits, draft, dtype, B, gamma, V, temp_p, temp_q, seed,
                   row_base, accept_len, next_token, alpha, beta, workspace, workspace_bytes,
                   hip_stream) -> int:
        return int(self._lib.svd_verify(
            _addr(p_logits), _addr(q_logits), _addr(draft), int(dtype), int(B), int(gamma),
            int(V), float(temp_p), float(temp_q), int(seed) & _M64, int(row_base) & _M64,
            _addr(accept_len), _addr(next_token), _addr(alpha), _addr(beta), _addr(workspace),
            int(workspace_bytes), _addr(hip_stream)))

    def svd_select_and_verify(self, p_logits, q_logits, drafts, dtype, B, K, gamma, V, temp_p,
                              temp_q, seed, row_base, selected, accept_len, next_token, scores,
                              alpha, beta, workspace, workspace_bytes, hip_stream) -> int:
        return int(self._lib.svd_select_and_verify(
            _addr(p_logits), _addr(q_logits), _addr(drafts), int(dtype), int(B), int(K),
            int(gamma), int(V), float(temp_p), float(temp_q), int(seed) & _M64,
            int(row_base) & _M64, _addr(selected), _addr(accept_len), _addr(next_token),
            _addr(scores), _addr(alpha), _addr(beta), _addr(workspace), int(workspace_bytes),
            _addr(hip_stream)))

    def svd_greedy_verify(self, p_logits, draft, dtype, B, gamma, V, temp_p, seed, row_base,
                          accept_len, next_token, alpha, workspace, workspace_bytes,
                          hip_stream) -> int:
        return int(self._lib.svd_greedy_verify(
            _addr(p_logits), _addr(draft), int(dtype), int(B), int(gamma), int(V), float(temp_p),
            int(seed) & _M64, int(row_base) & _M64, _addr(accept_len), _addr(next_token),
            _addr(alpha), _addr(workspace), int(workspace_bytes), _addr(hip_stream)))

    def svd_greedy_select_and_verify(self, p_logits, drafts, dtype, B, K, gamma, V, temp_p, seed,
                                     row_base, selected, accept_len, next_token, scores, alpha,
                                     workspace, workspace_bytes, hip_stream) -> int:
        return int(self._lib.svd_greedy_select_and_verify(
            _addr(p_logits), _addr(drafts), int(dtype), int(B), int(K), int(gamma), int(V),
            float(temp_p), int(seed) & _M64, int(row_base) & _M64, _addr(selected),
            _addr(accept_len), _addr(next_token), _addr(scores), _addr(alpha), _addr(workspace),
            int(workspace_bytes), _addr(hip_stream)))

    def svd_rows_workspace_bytes(self, B: int, K: int, gamma: int, V: int, n_p_rows: int,
                                 n_q_rows: int) -> int:
        return int(self._lib.svd_rows_workspace_bytes(B, K, gamma, V, n_p_rows, n_q_rows))

    def svd_select_and_verify_rows(self, rule, p_rows, n_p_rows, p_index, q_rows, n_q_rows,
                                   q_index, drafts, dtype, B, K, gamma, V, temp_p, temp_q, seed,
                                   row_base, selected, accept_len, next_token, scores, alpha,
                                   workspace, workspace_bytes, hip_stream) -> int:
        return int(self._lib.svd_select_and_verify_rows(
            int(rule), _addr(p_rows), int(n_p_rows), _addr(p_index), _addr(q_rows),
            int(n_q_rows), _addr(q_index), _addr(drafts), int(dtype), int(B), int(K), int(gamma),
            int(V), float(temp_p), float(temp_q), int(seed) & _M64, int(row_base) & _M64,
            _addr(selected), _addr(accept_len), _addr(next_token), _addr(scores), _addr(alpha),
            _addr(workspace), int(workspace_bytes), _addr(hip_stream)))

    def svd_verify_window(self, rule, p_logits, q_logits, drafts, gamma_b, eos, early_exit, dtype,
                          B, K, gamma, V, temp_p, temp_q, seed, row_base, selected, accept_len,
                          next_token, scores, alpha, workspace, workspace_bytes,
                          hip_stream) -> int:
        return int(self._lib.svd_verify_window(
            int(rule), _addr(p_logits), _addr(q_logits), _addr(drafts), _addr(gamma_b), int(eos),
            int(early_exit), int(dtype), int(B), int(K), int(gamma), int(V), float(temp_p),
            float(temp_q), int(seed) & _M64, int(row_base) & _M64, _addr(selected),
            _addr(accept_len), _addr(next_token), _addr(scores), _addr(alpha), _addr(workspace),
            int(workspace_bytes), _addr(hip_stream)))

    def svd_cps_workspace_bytes(self, B: int, G: int) -> int:
        return int(self._lib.svd_cps_workspace_bytes(B, G))

    def svd_cps_lattice(self, q_logits, dtype, B, G, V, temp_q, tau, m_max, eos, cand, cand_logp,
                        n_cand, length, workspace, workspace_bytes, hip_stream) -> int:
        return int(self._lib.svd_cps_lattice(
            _addr(q_logits), int(dtype), int(B), int(G), int(V), float(temp_q), float(tau),
            int(m_max), int(eos), _addr(cand), _addr(cand_logp), _addr(n_cand), _addr(length),
            _addr(workspace), int(workspace_bytes), _addr(hip_stream)))

    def svd_cps_beam(self, cand, cand_logp, n_cand, length, fluency, lam, B, G, m_max, beam,
                     paths, path_score, path_len, hip_stream) -> int:
        return int(self._lib.svd_cps_beam(
            _addr(cand), _addr(cand_logp), _addr(n_cand), _addr(length), _addr(fluency),
            float(lam), int(B), int(G), int(m_max), int(beam), _addr(paths), _addr(path_score),
            _addr(path_len), _addr(hip_stream)))

    def svd_adl_next(self, drafts, selected, accept_len, gamma_b, eos, B, K, gamma, k_min, k_max,
                     step, shift, slack, avg, next_gamma, hip_stream) -> int:
        return int(self._lib.svd_adl_next(
            _addr(drafts), _addr(selected), _addr(accept_len), _addr(gamma_b), int(eos), int(B),
            int(K), int(gamma), int(k_min), int(k_max), int(step), int(shift), int(slack),
            _addr(avg), _addr(next_gamma), _addr(hip_stream)))

    def svd_select_and_verify_noalloc(self, p_logits, q_logits, drafts, dtype, B, K, gamma, V,
                                      temp_p, temp_q, seed, row_base, selected, accept_len,
                                      next_token, scores, alpha, beta, hip_stream) -> int:
        return int(self._lib.svd_select_and_verify_noalloc(
            _addr(p_logits), _addr(q_logits), _addr(drafts), int(dtype), int(B), int(K),
            int(gamma), int(V), float(temp_p), float(temp_q), int(seed) & _M64,
            int(row_base) & _M64, _addr(selected), _addr(accept_len), _addr(next_token),
            _addr(scores), _addr(alpha), _addr(beta), _addr(hip_stream)))

    def svd_strerror(self, status: int) -> str:
        return self._lib.svd_strerror(int(status)).decode()

    # -- the timing build only ------------------------------------------------
    def svd_profile_enable(self, kernels=()) -> int:
        """Time the named kernels (names from KERNELS; "all" for every one) in
        later calls; an empty selection stops timing."""
        if not self.timing:
            raise RuntimeError("kernel timing needs the timing build (timing_library())")
        if kernels == "all":
            kernels = KERNELS
        mask = 0
        for k in kernels:
            mask |= 1 << KERNELS.index(k)
        return int(self._lib.svd_profile_enable(mask))

    def svd_profile_read(self):
        """(milliseconds per kernel, launches per kernel), indexed like KERNELS."""
        if not self.timing:
            raise RuntimeError("kernel timing needs the timing build (timing_library())")
        n = len(KERNELS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        st = self._lib.svd_profile_read(ctypes.cast(ms, ctypes.c_void_p),
                                        ctypes.cast(cnt, ctypes.c_void_p), n)
        if st != SVD_OK:
            raise SvdError(st, "svd_profile_read")
        return list(ms), list(cnt)


_default = Library(LIB_PATH)
_timed = []


def timing_library() -> Library:
    """The timing build, loaded once (ImportError when it is not built)."""
    if not _timed:
        _timed.append(Library(TIMED_LIB_PATH, timing=True))
    return _timed[0]


svd_workspace_bytes = _default.svd_workspace_bytes
svd_verify = _default.svd_verify
svd_select_and_verify = _default.svd_select_and_verify
svd_greedy_verify = _default.svd_greedy_verify
svd_greedy_select_and_verify = _default.svd_greedy_select_and_verify
svd_rows_workspace_bytes = _default.svd_rows_workspace_bytes
svd_select_and_verify_rows = _default.svd_select_and_verify_rows
svd_verify_window = _default.svd_verify_window
svd_cps_workspace_bytes = _default.svd_cps_workspace_bytes
svd_cps_lattice = _default.svd_cps_lattice
svd_cps_beam = _default.svd_cps_beam
svd_select_and_verify_noalloc = _default.svd_select_and_verify_noalloc
svd_adl_next = _default.svd_adl_next
svd_strerror = _default.svd_strerror


# --------------------------------------------------------------------------
# Tensor conveniences

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SVD_BF16
    if t.dtype == torch.float32:
        return SVD_F32
    raise TypeError("logits must be torch.bfloat16 or torch.float32, got %s" % t.dtype)


def _check(t, name, device):
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_bytes(B, K, gamma, V) -> int:
    n = svd_workspace_bytes(B, K, gamma, V)
    if n == 0:
        raise ValueError("sizes out of range: B=%d K=%d gamma=%d V=%d" % (B, K, gamma, V))
    return n


def alloc_workspace(B, K, gamma, V, device):
    import torch
    n = workspace_bytes(B, K, gamma, V)
    return torch.empty(n, dtype=torch.uint8, device=device)  # torch allocations are 256-B aligned


def select_and_verify(p, q, drafts, temp_p=1.0, temp_q=None, seed=0, row_base=0,
                      want_alpha=False, want_beta=False, want_scores=False, workspace=None,
                      stream=None):
    """p [B,K,gamma+1,V], q [B,K,gamma,V] (bf16 or fp32), drafts [B,K,gamma] int32."""
    import torch
    dev = p.device
    for t, n in ((p, "p"), (q, "q"), (drafts, "drafts")):
        _check(t, n, dev)
    if drafts.dtype != torch.int32:
        raise TypeError("drafts must be int32")
    if p.dtype != q.dtype:
        raise TypeError("p and q must share one dtype")
    if p.dim() != 4 or q.dim() != 4 or drafts.dim() != 3:
        raise ValueError("expected p [B,K,G+1,V], q [B,K,G,V], drafts [B,K,G]")
    B, K, G1, V = p.shape
    G = G1 - 1
    if tuple(q.shape) != (B, K, G, V) or tuple(drafts.shape) != (B, K, G):
        raise ValueError("shape mismatch: p %s q %s drafts %s" % (tuple(p.shape), tuple(q.shape),
                                                                 tuple(drafts.shape)))
    temp_q = temp_p if temp_q is None else temp_q
    out = {
        "selected": torch.empty(B, dtype=torch.int32, device=dev),
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "scores": torch.empty((B, K), dtype=torch.float32, device=dev) if want_scores else None,
        "alpha": torch.empty((B, K, G), dtype=torch.float32, device=dev) if want_alpha else None,
        "beta": torch.empty((B, K, G), dtype=torch.float32, device=dev) if want_beta else None,
    }
    ws = alloc_workspace(B, K, G, V, dev) if workspace is None else workspace
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    rc = svd_select_and_verify(p, q, drafts, _dtype_code(p), B, K, G, V, temp_p, temp_q, seed,
                               row_base, out["selected"], out["accept_len"], out["next_token"],
                               out["scores"], out["alpha"], out["beta"], ws, ws.numel(), st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_select_and_verify")
    return out


def verify(p, q, draft, temp_p=1.0, temp_q=None, seed=0, row_base=0, want_alpha=False,
           want_beta=False, workspace=None, stream=None):
    """p [B,gamma+1,V], q [B,gamma,V] (bf16 or fp32), draft [B,gamma] int32."""
    import torch
    dev = p.device
    for t, n in ((p, "p"), (q, "q"), (draft, "draft")):
        _check(t, n, dev)
    if draft.dtype != torch.int32:
        raise TypeError("draft must be int32")
    if p.dtype != q.dtype:
        raise TypeError("p and q must share one dtype")
    B, G1, V = p.shape
    G = G1 - 1
    if tuple(q.shape) != (B, G, V) or tuple(draft.shape) != (B, G):
        raise ValueError("shape mismatch")
    temp_q = temp_p if temp_q is None else temp_q
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "alpha": torch.empty((B, G), dtype=torch.float32, device=dev) if want_alpha else None,
        "beta": torch.empty((B, G), dtype=torch.float32, device=dev) if want_beta else None,
    }
    ws = alloc_workspace(B, 1, G, V, dev) if workspace is None else workspace
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    rc = svd_verify(p, q, draft, _dtype_code(p), B, G, V, temp_p, temp_q, seed, row_base,
                    out["accept_len"], out["next_token"], out["alpha"], out["beta"], ws,
                    ws.numel(), st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_verify")
    return out


def greedy_select_and_verify(p, drafts, temp_p=1.0, seed=0, row_base=0, want_alpha=False,
                             want_scores=False, workspace=None, stream=None):
    """Greedy acceptance: p [B,K,gamma+1,V] (bf16 or fp32), drafts [B,K,gamma] int32."""
    import torch
    dev = p.device
    for t, n in ((p, "p"), (drafts, "drafts")):
        _check(t, n, dev)
    if drafts.dtype != torch.int32:
        raise TypeError("drafts must be int32")
    if p.dim() != 4 or drafts.dim() != 3:
        raise ValueError("expected p [B,K,G+1,V], drafts [B,K,G]")
    B, K, G1, V = p.shape
    G = G1 - 1
    if tuple(drafts.shape) != (B, K, G):
        raise ValueError("shape mismatch: p %s drafts %s" % (tuple(p.shape), tuple(drafts.shape)))
    out = {
        "selected": torch.empty(B, dtype=torch.int32, device=dev),
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "scores": torch.empty((B, K), dtype=torch.float32, device=dev) if want_scores else None,
        "alpha": torch.empty((B, K, G), dtype=torch.float32, device=dev) if want_alpha else None,
    }
    ws = alloc_workspace(B, K, G, V, dev) if workspace is None else workspace
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    rc = svd_greedy_select_and_verify(p, drafts, _dtype_code(p), B, K, G, V, temp_p, seed,
                                      row_base, out["selected"], out["accept_len"],
                                      out["next_token"], out["scores"], out["alpha"], ws,
                                      ws.numel(), st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_greedy_select_and_verify")
    return out


def greedy_verify(p, draft, temp_p=1.0, seed=0, row_base=0, want_alpha=False, workspace=None,
                  stream=None):
    """Greedy acceptance, one draft: p [B,gamma+1,V] (bf16 or fp32), draft [B,gamma] int32."""
    import torch
    dev = p.device
    for t, n in ((p, "p"), (draft, "draft")):
        _check(t, n, dev)
    if draft.dtype != torch.int32:
        raise TypeError("draft must be int32")
    B, G1, V = p.shape
    G = G1 - 1
    if tuple(draft.shape) != (B, G):
        raise ValueError("shape mismatch")
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "alpha": torch.empty((B, G), dtype=torch.float32, device=dev) if want_alpha else None,
    }
    ws = alloc_workspace(B, 1, G, V, dev) if workspace is None else workspace
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    rc = svd_greedy_verify(p, draft, _dtype_code(p), B, G, V, temp_p, seed, row_base,
                           out["accept_len"], out["next_token"], out["alpha"], ws, ws.numel(), st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_greedy_verify")
    return out


def select_and_verify_rows(p_pool, p_index, q_pool, q_index, drafts, rule="standard", temp_p=1.0,
                           temp_q=None, seed=0, row_base=0, want_alpha=False, want_scores=False,
                           workspace=None, stream=None):
    """Shared rows: p_pool [NP,V], p_index [B,K,gamma+1] int32, q_pool [NQ,V] and
    q_index [B,K,gamma] int32 (None for rule="greedy"), drafts [B,K,gamma] int32."""
    import torch
    greedy = rule == "greedy"
    if rule not in ("standard", "greedy"):
        raise ValueError("rule must be 'standard' or 'greedy'")
    dev = p_pool.device
    tens = [(p_pool, "p_pool"), (p_index, "p_index"), (drafts, "drafts")]
    if not greedy:
        tens += [(q_pool, "q_pool"), (q_index, "q_index")]
        if q_pool.dtype != p_pool.dtype:
            raise TypeError("p_pool and q_pool must share one dtype")
    for t, n in tens:
        _check(t, n, dev)
    for t, n in ((p_index, "p_index"), (drafts, "drafts")) + (() if greedy else ((q_index, "q_index"),)):
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % n)
    B, K, G = drafts.shape
    V = p_pool.shape[1]
    if tuple(p_index.shape) != (B, K, G + 1) or (not greedy and tuple(q_index.shape) != (B, K, G)):
        raise ValueError("index tables must be [B,K,gamma+1] and [B,K,gamma]")
    if not greedy and q_pool.shape[1] != V:
        raise ValueError("pools must share V")
    NP = p_pool.shape[0]
    NQ = 0 if greedy else q_pool.shape[0]
    out = {
        "selected": torch.empty(B, dtype=torch.int32, device=dev),
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "scores": torch.empty((B, K), dtype=torch.float32, device=dev) if want_scores else None,
        "alpha": torch.empty((B, K, G), dtype=torch.float32, device=dev) if want_alpha else None,
    }
    if workspace is None:
        n = svd_rows_workspace_bytes(B, K, G, V, NP, NQ)
        if n == 0:
            raise ValueError("sizes out of range")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    temp_q = temp_p if temp_q is None else temp_q
    rc = svd_select_and_verify_rows(
        SVD_RULE_GREEDY if greedy else SVD_RULE_STANDARD, p_pool, NP, p_index,
        None if greedy else q_pool, NQ, None if greedy else q_index, drafts, _dtype_code(p_pool),
        B, K, G, V, temp_p, temp_q, seed, row_base, out["selected"], out["accept_len"],
        out["next_token"], out["scores"], out["alpha"], workspace, workspace.numel(), st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_select_and_verify_rows")
    return out


def verify_window(p, q, drafts, gamma_b=None, eos=-1, rule="standard", early_exit=False,
                  temp_p=1.0, temp_q=None, seed=0, row_base=0, want_alpha=False,
                  want_scores=False, workspace=None, stream=None):
    """Ragged, EOS-aware windows: p [B,K,gamma+1,V], q [B,K,gamma,V] (None for
    rule="greedy"), drafts [B,K,gamma] int32, gamma_b [B] int32 or None, eos a token or -1.
    early_exit (K = 1): stream positions only up to each prefix's first rejection."""
    import torch
    greedy = rule == "greedy"
    if rule not in ("standard", "greedy"):
        raise ValueError("rule must be 'standard' or 'greedy'")
    dev = p.device
    tens = [(p, "p"), (drafts, "drafts")] + ([] if greedy else [(q, "q")])
    if gamma_b is not None:
        tens.append((gamma_b, "gamma_b"))
    for t, n in tens:
        _check(t, n, dev)
    B, K, G1, V = p.shape
    G = G1 - 1
    if tuple(drafts.shape) != (B, K, G) or (gamma_b is not None and tuple(gamma_b.shape) != (B,)):
        raise ValueError("drafts must be [B,K,gamma] and gamma_b [B]")
    out = {
        "selected": torch.empty(B, dtype=torch.int32, device=dev),
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "scores": torch.empty((B, K), dtype=torch.float32, device=dev) if want_scores else None,
        "alpha": torch.empty((B, K, G), dtype=torch.float32, device=dev) if want_alpha else None,
    }
    ws = alloc_workspace(B, K, G, V, dev) if workspace is None else workspace
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    temp_q = temp_p if temp_q is None else temp_q
    rc = svd_verify_window(SVD_RULE_GREEDY if greedy else SVD_RULE_STANDARD, p,
                           None if greedy else q, drafts, gamma_b, eos, int(bool(early_exit)),
                           _dtype_code(p), B, K, G, V, temp_p, temp_q, seed, row_base,
                           out["selected"], out["accept_len"], out["next_token"], out["scores"],
                           out["alpha"], ws, ws.numel(), st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_verify_window")
    return out


def cps_lattice(q, temp_q=1.0, tau=0.8, m_max=15, eos=-1, stream=None, lib=None):
    """Candidate lattice of drafter logits q [B, G, V] (bf16 or fp32); lib: the
    Library to call (default: the product library)."""
    import torch
    dev = q.device
    _check(q, "q", dev)
    B, G, V = q.shape
    out = {"cand": torch.empty((B, G, m_max), dtype=torch.int32, device=dev),
           "cand_logp": torch.empty((B, G, m_max), dtype=torch.float32, device=dev),
           "n_cand": torch.empty((B, G), dtype=torch.int32, device=dev),
           "len": torch.empty(B, dtype=torch.int32, device=dev)}
    n = svd_cps_workspace_bytes(B, G)
    if n == 0:
        raise ValueError("sizes out of range")
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    lib = _default if lib is None else lib
    rc = lib.svd_cps_lattice(q, _dtype_code(q), B, G, V, temp_q, tau, m_max, eos, out["cand"],
                             out["cand_logp"], out["n_cand"], out["len"], ws, n, st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_cps_lattice")
    return out


def cps_beam(lat, fluency=None, lam=1.0, beam=3, stream=None, lib=None):
    """Beam search over a lattice from cps_lattice; fluency [B, G, m_max, m_max] fp32 or None;
    lib: the Library to call (default: the product library)."""
    import torch
    cand = lat["cand"]
    dev = cand.device
    B, G, M = cand.shape
    if fluency is not None:
        _check(fluency, "fluency", dev)
        if fluency.dtype != torch.float32 or tuple(fluency.shape) != (B, G, M, M):
            raise ValueError("fluency must be float32 [B, G, m_max, m_max]")
    out = {"paths": torch.empty((B, beam, G), dtype=torch.int32, device=dev),
           "score": torch.empty((B, beam), dtype=torch.float32, device=dev),
           "path_len": torch.empty((B, beam), dtype=torch.int32, device=dev)}
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    lib = _default if lib is None else lib
    rc = lib.svd_cps_beam(cand, lat["cand_logp"], lat["n_cand"], lat["len"], fluency, lam, B, G,
                          M, beam, out["paths"], out["score"], out["path_len"], st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_cps_beam")
    return out


def adl_next(drafts, selected, accept_len, avg, gamma_b=None, eos=-1, k_min=1, k_max=64, step=4,
             shift=2, slack=64, stream=None):
    """Adaptive draft length: the next window of every prefix, on the device.
    drafts [B,K,gamma] int32 and selected, accept_len [B] int32 (a verification
    call's inputs and outputs), gamma_b [B] int32 or None, avg [B,2] int32
    updated in place.  Returns next [B] int32."""
    import torch
    dev = drafts.device
    tens = [(drafts, "drafts"), (selected, "selected"), (accept_len, "accept_len"),
            (avg, "avg")] + ([] if gamma_b is None else [(gamma_b, "gamma_b")])
    for t, n in tens:
        _check(t, n, dev)
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % n)
    B, K, G = drafts.shape
    if (tuple(selected.shape) != (B,) or tuple(accept_len.shape) != (B,) or
            tuple(avg.shape) != (B, 2) or (gamma_b is not None and tuple(gamma_b.shape) != (B,))):
        raise ValueError("selected, accept_len, gamma_b must be [B] and avg [B, 2]")
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    rc = svd_adl_next(drafts, selected, accept_len, gamma_b, eos, B, K, G, k_min, k_max, step,
                      shift, slack, avg, nxt, st)
    if rc != SVD_OK:
        raise SvdError(rc, "svd_adl_next")
    return nxt
