"""Plain double-precision CPU oracle for lossless draft verification.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``lossless_draft_verification_verifier_amd``) and the
library never imports it.

The arithmetic lives in ``svd_oracle.c`` (scalar loops in double, sequential
sums, no contraction, no fast-math); this module compiles it with gcc and wraps
it with ctypes so that tests can hand it numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_BONUS = 1, 2, 3


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (strict IEEE: no contraction, no fast-math)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, _LIB)
    return _LIB


class _Diag(ctypes.Structure):
    _fields_ = [("select_gap", ctypes.c_double), ("emit_margin", ctypes.c_double),
                ("draw_z", ctypes.c_double), ("draw_t", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # SVD_ORACLE_LIB: another build of the same source (the sanitizer test's)
        path = os.environ.get("SVD_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        u64, i32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_double, ctypes.c_void_p)
        L.svdo_splitmix64.restype = u64
        L.svdo_splitmix64.argtypes = [u64]
        L.svdo_key.restype = u64
        L.svdo_key.argtypes = [u64, u64, u64, u64]
        L.svdo_uniform.restype = dbl
        L.svdo_uniform.argtypes = [u64, u64, u64, u64]
        L.svdo_softmax_row.restype = ctypes.c_int
        L.svdo_softmax_row.argtypes = [vp, ctypes.c_int, i32, ctypes.c_float, vp]
        L.svdo_inverse_cdf.restype = i32
        L.svdo_inverse_cdf.argtypes = [vp, i32, dbl, vp, vp]
        L.svdo_draw_weights.restype = dbl
        L.svdo_draw_weights.argtypes = [vp, vp, i32, vp]
        L.svdo_select_and_verify.restype = ctypes.c_int
        L.svdo_select_and_verify.argtypes = [
            vp, vp, vp, ctypes.c_int, i64, i32, i32, i32, ctypes.c_float, ctypes.c_float,
            u64, u64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        L.svdo_window_select_and_verify.restype = ctypes.c_int
        L.svdo_window_select_and_verify.argtypes = [
            ctypes.c_int, vp, vp, vp, vp, i32, ctypes.c_int, i64, i32, i32, i32, ctypes.c_float,
            ctypes.c_float, u64, u64, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        L.svdo_greedy_select_and_verify.restype = ctypes.c_int
        L.svdo_greedy_select_and_verify.argtypes = [
            vp, vp, ctypes.c_int, i64, i32, i32, i32, ctypes.c_float, u64, u64, vp, vp, vp, vp,
            vp, vp, vp, vp, vp, ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(a: np.ndarray):
    """Accept float32 logits, or bf16 logits given as their uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("logits must be float32, or uint16 holding bf16 bit patterns")


def splitmix64(x: int) -> int:
    return int(lib().svdo_splitmix64(x & 0xFFFFFFFFFFFFFFFF))


def key(seed: int, row: int, pos: int, purpose: int) -> int:
    m = 0xFFFFFFFFFFFFFFFF
    return int(lib().svdo_key(seed & m, row & m, pos & m, purpose & m))


def uniform(seed: int, row: int, pos: int, purpose: int) -> float:
    m = 0xFFFFFFFFFFFFFFFF
    return float(lib().svdo_uniform(seed & m, row & m, pos & m, purpose & m))


def softmax_row(z: np.ndarray, temp: float = 1.0):
    """Probabilities of one logit row in double, or None for an invalid row."""
    z, dt = _logits(z)
    out = np.empty(z.shape[-1], dtype=np.float64)
    ok = lib().svdo_softmax_row(_ptr(z), dt, z.shape[-1], temp, _ptr(out))
    return out if ok else None


def draw_weights(p: np.ndarray, q: np.ndarray | None):
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.float64)
    r = np.empty_like(p)
    Z = lib().svdo_draw_weights(_ptr(p), _ptr(q), p.shape[0], _ptr(r))
    return r, float(Z)


def inverse_cdf(r: np.ndarray, t: float):
    r = np.ascontiguousarray(r, dtype=np.float64)
    lo, hi = ctypes.c_double(), ctypes.c_double()
    v = lib().svdo_inverse_cdf(_ptr(r), r.shape[0], t, ctypes.byref(lo), ctypes.byref(hi))
    return int(v), lo.value, hi.value


@dataclass
class OracleResult:
    selected: np.ndarray        # [B] int32
    accept_len: np.ndarray      # [B] int32
    next_token: np.ndarray      # [B] int32
    scores: np.ndarray          # [B, K] float64
    alpha: np.ndarray           # [B, K, gamma] float64
    beta: np.ndarray | None     # [B, K, gamma] float64
    px: np.ndarray              # [B, K, gamma] float64
    qx: np.ndarray              # [B, K, gamma] float64
    accept_margin: np.ndarray   # [B, gamma] float64
    select_gap: np.ndarray      # [B]
    emit_margin: np.ndarray     # [B]
    draw_z: np.ndarray          # [B]
    draw_t: np.ndarray          # [B]


def select_and_verify(p_logits, q_logits, drafts, temp_p=1.0, temp_q=None, seed=0,
                      row_base=0, want_beta=False, force_k=None, force_L=None,
                      nthreads=None) -> OracleResult:
    """Run the oracle on host arrays.

    p_logits [B, K, gamma+1, V], q_logits [B, K, gamma, V] (float32, or uint16
    bf16 bit patterns; the two must agree), drafts [B, K, gamma] int32.
    """
    p, dt = _logits(p_logits)
    q, dq = _logits(q_logits)
    if dt != dq:
        raise TypeError("p and q logits must share one dtype")
    if p.ndim != 4 or q.ndim != 4:
        raise ValueError("expected p [B,K,gamma+1,V] and q [B,K,gamma,V]")
    B, K, G1, V = p.shape
    G = G1 - 1
    if q.shape != (B, K, G, V):
        raise ValueError("q shape %s does not match p shape %s" % (q.shape, p.shape))
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    if d.shape != (B, K, G):
        raise ValueError("drafts shape %s, expected %s" % (d.shape, (B, K, G)))
    if temp_q is None:
        temp_q = temp_p
    if nthreads is None:
        nthreads = min(os.cpu_count() or 1, 16)
    fk = None if force_k is None else np.ascontiguousarray(force_k, dtype=np.int32)
    fl = None if force_L is None else np.ascontiguousarray(force_L, dtype=np.int32)
    sel = np.empty(B, np.int32)
    L = np.empty(B, np.int32)
    tok = np.empty(B, np.int32)
    scores = np.full((B, K), np.nan)
    alpha = np.full((B, K, G), np.nan)
    beta = np.full((B, K, G), np.nan) if want_beta else None
    px = np.full((B, K, G), np.nan)
    qx = np.full((B, K, G), np.nan)
    am = np.full((B, G), np.nan)
    diag = (_Diag * B)()
    rc = lib().svdo_select_and_verify(
        _ptr(p), _ptr(q), _ptr(d), dt, B, K, G, V, float(temp_p), float(temp_q),
        seed & 0xFFFFFFFFFFFFFFFF, row_base & 0xFFFFFFFFFFFFFFFF, _ptr(fk), _ptr(fl),
        _ptr(sel), _ptr(L), _ptr(tok), _ptr(scores), _ptr(alpha), _ptr(beta), _ptr(px),
        _ptr(qx), _ptr(am), ctypes.cast(diag, ctypes.c_void_p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    dg = np.frombuffer(diag, dtype=np.float64).reshape(B, 4) if B else np.zeros((0, 4))
    return OracleResult(sel, L, tok, scores, alpha, beta, px, qx, am,
                        dg[:, 0].copy(), dg[:, 1].copy(), dg[:, 2].copy(), dg[:, 3].copy())


def greedy_select_and_verify(p_logits, drafts, temp_p=1.0, seed=0, row_base=0, force_k=None,
                             force_L=None, nthreads=None) -> OracleResult:
    """Greedy acceptance (alpha = p(x); a rejected token is resampled from p with
    that token zeroed).  p_logits [B, K, gamma+1, V], drafts [B, K, gamma]."""
    p, dt = _logits(p_logits)
    if p.ndim != 4:
        raise ValueError("expected p [B,K,gamma+1,V]")
    B, K, G1, V = p.shape
    G = G1 - 1
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    if d.shape != (B, K, G):
        raise ValueError("drafts shape %s, expected %s" % (d.shape, (B, K, G)))
    if nthreads is None:
        nthreads = min(os.cpu_count() or 1, 16)
    fk = None if force_k is None else np.ascontiguousarray(force_k, dtype=np.int32)
    fl = None if force_L is None else np.ascontiguousarray(force_L, dtype=np.int32)
    sel = np.empty(B, np.int32)
    L = np.empty(B, np.int32)
    tok = np.empty(B, np.int32)
    scores = np.full((B, K), np.nan)
    alpha = np.full((B, K, G), np.nan)
    am = np.full((B, G), np.nan)
    diag = (_Diag * B)()
    rc = lib().svdo_greedy_select_and_verify(
        _ptr(p), _ptr(d), dt, B, K, G, V, float(temp_p), seed & 0xFFFFFFFFFFFFFFFF,
        row_base & 0xFFFFFFFFFFFFFFFF, _ptr(fk), _ptr(fl), _ptr(sel), _ptr(L), _ptr(tok),
        _ptr(scores), _ptr(alpha), _ptr(am), ctypes.cast(diag, ctypes.c_void_p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    dg = np.frombuffer(diag, dtype=np.float64).reshape(B, 4) if B else np.zeros((0, 4))
    return OracleResult(sel, L, tok, scores, alpha, None, alpha.copy(), np.full((B, K, G), np.nan),
                        am, dg[:, 0].copy(), dg[:, 1].copy(), dg[:, 2].copy(), dg[:, 3].copy())


def _gather_rows(pool: np.ndarray, index: np.ndarray) -> np.ndarray:
    """Rows of a pool at index[...] -> array of shape index.shape + (V,); an index
    outside the pool gives a row of NaN logits (so the prefix reading it is invalid)."""
    idx = np.asarray(index, dtype=np.int64)
    ok = (idx >= 0) & (idx < pool.shape[0])
    out = pool[np.where(ok, idx, 0)]
    nan = np.uint16(0x7FC0) if pool.dtype == np.uint16 else np.float32(np.nan)
    out[~ok] = nan
    return out


def select_and_verify_rows(p_pool, p_index, q_pool, q_index, drafts, temp_p=1.0, temp_q=None,
                           seed=0, row_base=0, greedy=False, force_k=None, force_L=None,
                           nthreads=None) -> OracleResult:
    """Verification over shared rows: p row (b, k, j) is p_pool[p_index[b, k, j]] and q row
    (b, k, j) is q_pool[q_index[b, k, j]].  By definition this is the dense rule on the
    gathered rows; an index outside its pool reads as a row of NaN logits.
    greedy: the greedy-acceptance rule (q_pool and q_index unused)."""
    p_pool, _ = _logits(p_pool)
    p = _gather_rows(p_pool, p_index)
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    if greedy:
        return greedy_select_and_verify(p, d, temp_p=temp_p, seed=seed, row_base=row_base,
                                        force_k=force_k, force_L=force_L, nthreads=nthreads)
    q_pool, _ = _logits(q_pool)
    q = _gather_rows(q_pool, q_index)
    return select_and_verify(p, q, d, temp_p=temp_p, temp_q=temp_q, seed=seed,
                             row_base=row_base, force_k=force_k, force_L=force_L,
                             nthreads=nthreads)


def window_select_and_verify(p_logits, q_logits, drafts, gamma_b=None, eos=-1, greedy=False,
                             temp_p=1.0, temp_q=None, seed=0, row_base=0, force_k=None,
                             force_L=None, nthreads=None) -> OracleResult:
    """Ragged, EOS-aware windows: prefix b drafts gamma_b[b] positions of the padded
    arrays (None: all gamma); with eos >= 0 a draft's usable positions end at its first
    drafted EOS, and an accepted window ending in EOS draws nothing (next_token -2).
    greedy: the greedy-acceptance rule (q_logits unused, may be None)."""
    p, dt = _logits(p_logits)
    B, K, G1, V = p.shape
    G = G1 - 1
    q = None
    if not greedy:
        q, dq = _logits(q_logits)
        if dq != dt or q.shape != (B, K, G, V):
            raise ValueError("q must be [B,K,gamma,V] of p's dtype")
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    if d.shape != (B, K, G):
        raise ValueError("drafts shape %s, expected %s" % (d.shape, (B, K, G)))
    gb = None if gamma_b is None else np.ascontiguousarray(gamma_b, dtype=np.int32)
    if gb is not None and gb.shape != (B,):
        raise ValueError("gamma_b must be [B]")
    if temp_q is None:
        temp_q = temp_p
    if nthreads is None:
        nthreads = min(os.cpu_count() or 1, 16)
    fk = None if force_k is None else np.ascontiguousarray(force_k, dtype=np.int32)
    fl = None if force_L is None else np.ascontiguousarray(force_L, dtype=np.int32)
    sel = np.empty(B, np.int32)
    L = np.empty(B, np.int32)
    tok = np.empty(B, np.int32)
    scores = np.full((B, K), np.nan)
    alpha = np.full((B, K, G), np.nan)
    am = np.full((B, G), np.nan)
    diag = (_Diag * B)()
    rc = lib().svdo_window_select_and_verify(
        int(bool(greedy)), _ptr(p), _ptr(q), _ptr(d), _ptr(gb), int(eos), dt, B, K, G, V,
        float(temp_p), float(temp_q), seed & 0xFFFFFFFFFFFFFFFF, row_base & 0xFFFFFFFFFFFFFFFF,
        _ptr(fk), _ptr(fl), _ptr(sel), _ptr(L), _ptr(tok), _ptr(scores), _ptr(alpha), _ptr(am),
        ctypes.cast(diag, ctypes.c_void_p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    dg = np.frombuffer(diag, dtype=np.float64).reshape(B, 4) if B else np.zeros((0, 4))
    return OracleResult(sel, L, tok, scores, alpha, None, alpha.copy(),
                        np.full((B, K, G), np.nan), am, dg[:, 0].copy(), dg[:, 1].copy(),
                        dg[:, 2].copy(), dg[:, 3].copy())


def cps_lattice(q_logits, temp_q=1.0, tau=0.8, m_max=15, eos=-1) -> dict:
    """The pruned candidate lattice of every drafter row: q_logits [B, G, V]."""
    q, dt = _logits(q_logits)
    B, G, V = q.shape
    cand = np.empty((B, G, m_max), np.int32)
    logp = np.empty((B, G, m_max), np.float64)
    n = np.empty((B, G), np.int32)
    ln = np.empty(B, np.int32)
    cm = np.empty((B, G), np.float64)
    L = lib()
    L.svdo_cps_lattice.restype = ctypes.c_int
    L.svdo_cps_lattice.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_float, ctypes.c_double,
                                   ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 5
    rc = L.svdo_cps_lattice(_ptr(q), dt, B, G, V, float(temp_q), float(tau), int(m_max), int(eos),
                            _ptr(cand), _ptr(logp), _ptr(n), _ptr(ln), _ptr(cm))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return {"cand": cand, "cand_logp": logp, "n_cand": n, "len": ln, "cum_margin": cm}


def cps_beam(lat: dict, fluency=None, lam=1.0, beam=3) -> dict:
    """Beam search over a lattice from cps_lattice; fluency [B, G, m_max, m_max] float32
    or None."""
    cand, logp = np.ascontiguousarray(lat["cand"]), np.ascontiguousarray(lat["cand_logp"])
    n, ln = np.ascontiguousarray(lat["n_cand"]), np.ascontiguousarray(lat["len"])
    B, G, M = cand.shape
    f = None if fluency is None else np.ascontiguousarray(fluency, dtype=np.float32)
    if f is not None and f.shape != (B, G, M, M):
        raise ValueError("fluency must be [B, G, m_max, m_max]")
    paths = np.empty((B, beam, G), np.int32)
    score = np.empty((B, beam), np.float64)
    plen = np.empty((B, beam), np.int32)
    rm = np.empty(B, np.float64)
    L = lib()
    L.svdo_cps_beam.restype = ctypes.c_int
    L.svdo_cps_beam.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_double, ctypes.c_int64,
                                                        ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.c_int32] + [ctypes.c_void_p] * 4
    rc = L.svdo_cps_beam(_ptr(cand), _ptr(logp), _ptr(n), _ptr(ln), _ptr(f), float(lam), B, G, M,
                         int(beam), _ptr(paths), _ptr(score), _ptr(plen), _ptr(rm))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return {"paths": paths, "score": score, "path_len": plen, "rank_margin": rm}


def adl_next(drafts, selected, accept_len, avg, gamma_b=None, eos=-1, k_min=1, k_max=64,
             step=4, shift=2, slack=64):
    """Adaptive draft length: the next window of every prefix and the updated
    state.  drafts [B, K, gamma] int32; selected, accept_len, gamma_b [B]
    int32; avg [B, 2] int32 (recent accepted and generated lengths in 1/256ths
    of a token).  Returns (next [B] int32, avg' [B, 2] int32)."""
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    B, K, G = d.shape
    sel = np.ascontiguousarray(selected, dtype=np.int32)
    L = np.ascontiguousarray(accept_len, dtype=np.int32)
    gb = None if gamma_b is None else np.ascontiguousarray(gamma_b, dtype=np.int32)
    st = np.array(avg, dtype=np.int32, copy=True).reshape(B, 2)
    nxt = np.empty(B, np.int32)
    lb = lib()
    lb.svdo_adl_next.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lb.svdo_adl_next.argtypes = [ctypes.c_void_p] * 4 + [i32, ctypes.c_int64, i32, i32, i32, i32,
                                                         i32, i32, i32] + [ctypes.c_void_p] * 2
    rc = lb.svdo_adl_next(_ptr(d), _ptr(sel), _ptr(L), _ptr(gb), int(eos), B, K, G, int(k_min),
                          int(k_max), int(step), int(shift), int(slack), _ptr(st), _ptr(nxt))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return nxt, st
