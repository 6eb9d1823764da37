"""Runs every oracle entry point on small seeded inputs with the edge cases the
rules define, and prints one SHA-256 over all outputs.  Run by
tests/test_oracle_sanitized.py, once against the sanitizer build of the oracle
(SVD_ORACLE_LIB) and once against the normal build."""
import dataclasses
import hashlib
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402

H = hashlib.sha256()


def feed(x):
    if x is None:
        H.update(b"none")
    elif dataclasses.is_dataclass(x):
        for f in dataclasses.fields(x):
            feed(getattr(x, f.name))
    elif isinstance(x, dict):
        for k in sorted(x):
            feed(x[k])
    elif isinstance(x, (tuple, list)):
        for v in x:
            feed(v)
    else:
        H.update(np.ascontiguousarray(np.asarray(x)).tobytes())


def to_bf16(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


rng = np.random.default_rng(2026)
B, K, G, V = 7, 3, 4, 37
zp = (rng.standard_normal((B, K, G + 1, V)) * 2).astype(np.float32)
zq = (zp[:, :, :G] + rng.standard_normal((B, K, G, V))).astype(np.float32)
d = rng.integers(0, V, (B, K, G)).astype(np.int32)
zp[2, 1, 0, 5] = np.nan                # a NaN verifier row
zq[3, 0, 1, :] = -np.inf               # an all -inf drafter row
zp[4, 2, 2, 7] = np.inf                # a +inf logit
d[5, 0, 0], d[5, 1, 2] = -1, V         # drafted tokens out of range
zq[6] = zp[6, :, :G]                   # q = p: every draft accepted, bonus draws
for nt in (1, 2):
    feed(oracle.select_and_verify(zp, zq, d, temp_p=0.8, temp_q=1.1, seed=11, row_base=5,
                                  want_beta=True, nthreads=nt))
    feed(oracle.select_and_verify(to_bf16(zp), to_bf16(zq), d, temp_p=0.7, seed=12,
                                  nthreads=nt))
    feed(oracle.greedy_select_and_verify(zp, d, temp_p=0.9, seed=13, nthreads=nt))
fk = (np.arange(B) % K).astype(np.int32)
fl = (np.arange(B) % (G + 1)).astype(np.int32)
feed(oracle.select_and_verify(zp, zq, d, seed=14, force_k=fk, force_L=fl))
gb = np.array([1, 4, 2, 3, 4, 1, 2], np.int32)
d2 = d.copy()
d2[1, :, 1] = 9                        # an EOS drafted inside the window
for greedy in (False, True):
    feed(oracle.window_select_and_verify(zp, zq, d2, gamma_b=gb, eos=9, greedy=greedy, seed=15,
                                         nthreads=2))
pool_p = zp.reshape(-1, V)[:40].copy()
pool_q = zq.reshape(-1, V)[:30].copy()
pi = rng.integers(-1, 41, (B, K, G + 1)).astype(np.int32)   # -1 and 40: outside the pool
qi = rng.integers(0, 31, (B, K, G)).astype(np.int32)        # 30: outside the pool
feed(oracle.select_and_verify_rows(pool_p, pi, pool_q, qi, d, seed=16, nthreads=2))
feed(oracle.select_and_verify_rows(pool_p, pi, pool_q, qi, d, seed=17, greedy=True))
zl = (rng.standard_normal((4, 6, 50)) * 2).astype(np.float32)
zl[1, 2, 3] = zl[1, 2].max() + 3.0     # EOS (token 3) on top: the lattice stops there
zl[2, 4, :] = np.nan                   # an invalid row
zl[3, 0, :8] = zl[3, 0].max() + 1.0    # ties at the top
for m_max in (1, 15, 16):
    lat = oracle.cps_lattice(zl, temp_q=0.9, tau=0.8, m_max=m_max, eos=3)
    feed(lat)
    flu = rng.standard_normal((4, 6, m_max, m_max)).astype(np.float32)
    flu[0, 1, 0, 0] = np.nan
    for beam in (1, 3, 8):
        feed(oracle.cps_beam(lat, flu, lam=0.5, beam=beam))
    feed(oracle.cps_beam(lat, None, beam=2))
sel = rng.integers(-1, K, B).astype(np.int32)
L = rng.integers(-1, G + 1, B).astype(np.int32)
avg = rng.integers(0, 256 * G, (B, 2)).astype(np.int32)
feed(oracle.adl_next(d2, sel, L, avg, gamma_b=gb, eos=9, k_min=1, k_max=G, step=2))
for t in (0.0, 0.3, 1.7, 2.0):
    r, Z = oracle.draw_weights(np.array([0.1, 0.5, 0.0, 0.4]), np.array([0.2, 0.1, 0.3, 0.4]))
    feed((r, Z, oracle.inverse_cdf(r, t * Z / 2.0)))
feed(oracle.softmax_row(zp[0, 0, 0], 0.5))
feed(oracle.softmax_row(zp[2, 1, 0], 1.0))
feed([oracle.uniform(s, 3, 4, 2) for s in range(5)])
print(oracle.lib()._name)
print(H.hexdigest())
