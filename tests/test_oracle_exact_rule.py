"""The oracle's whole rule against the same rule in 50-digit decimal arithmetic.

Each prefix is recomputed here with Python's decimal module (exp correctly
rounded at 50 digits) and the counter-hash uniforms of tests/hash_ref.py (big
integers from the published SplitMix64 definition), following the pages' order
(SpecDiff-2 section 2 and section 5.2; DiffuSpec section 3):

* softmax of z / T per row, alpha_j = min(1, p_j(x_j) / q_j(x_j));
* the streak score sum_j prod_{i<=j} alpha_i of every draft, the kept draft
  its argmax (lowest k on a tie);
* the first j with U(seed, row_base + b, j, 1) >= alpha_j, or gamma;
* the token: the first v whose running sum of r exceeds U(seed, row_base + b,
  L, 2) * Z, with r = max(0, p_L - q_L) of the kept draft (p_L when the
  residual has no mass), or, when all gamma are accepted, of r = p_gamma with
  U(seed, row_base + b, gamma, 3).

selected, accept_len and next_token must equal the oracle's wherever the
exact values keep their decision at least 1e-12 (relative) away from a tie, so
a wrong uniform (position, purpose or row), a wrong row of the draw or a wrong
comparison fails here even though the committed tokens' law would not change.
Forced decisions (force_k, force_L) reach every position and the bonus draw.
"""
from decimal import Decimal, localcontext

import numpy as np
import pytest

from hash_ref import uniform_bits

TIE = Decimal("1e-12")
TWO53 = Decimal(2) ** -53  # exact: 38 significant digits


def _widen(z):
    """Exact decimals of the logits (float32, or bf16 bit patterns)."""
    if z.dtype == np.uint16:
        z = (z.astype(np.uint32) << 16).view(np.float32)
    return [Decimal(float(v)) for v in z]


def _softmax(z, T):
    s = [v / T for v in z]
    m = max(s)
    w = [(v - m).exp() for v in s]
    S = sum(w)
    return [v / S for v in w]


def _u(seed, row, pos, purpose):
    return Decimal(uniform_bits(seed, row, pos, purpose)) * TWO53


def _draw(r, t):
    """First v with running sum > t (the last positive when none), and whether
    t lies within TIE * total of a running sum."""
    Z = sum(r)
    c = Decimal(0)
    tok, near, last = None, False, None
    for v, rv in enumerate(r):
        if rv > 0:
            last = v
        c += rv
        if abs(c - t) <= TIE * Z:
            near = True
        if tok is None and rv > 0 and c > t:
            tok = v
    return (last if tok is None else tok), near


def exact_prefix(zp, zq, d, Tp, Tq, seed, row, force_k=None, force_L=None):
    """(selected, L, token, excused) of one prefix: zp [K, G+1, V], zq [K, G, V]."""
    K, G1, V = zp.shape
    G = G1 - 1
    P = [[_softmax(_widen(zp[k, j]), Tp) for j in range(G1)] for k in range(K)]
    Q = [[_softmax(_widen(zq[k, j]), Tq) for j in range(G)] for k in range(K)]
    alpha = [[Decimal(1) if Q[k][j][d[k, j]] <= P[k][j][d[k, j]]
              else P[k][j][d[k, j]] / Q[k][j][d[k, j]] for j in range(G)] for k in range(K)]
    scores = []
    for k in range(K):
        prod, s = Decimal(1), Decimal(0)
        for j in range(G):
            prod *= alpha[k][j]
            s += prod
        scores.append(s)
    excused = False
    if force_k is None:
        best = max(scores)
        ks = min(k for k in range(K) if scores[k] == best)
        others = [s for k, s in enumerate(scores) if k != ks]
        # an exact tie (every alpha of both drafts exactly 1, say) is decided
        # by the lowest index on both sides; only a gap within TIE is excused
        if others and 0 < best - max(others) <= TIE * best:
            excused = True
    else:
        ks = force_k
    if force_L is None:
        L = G
        for j in range(G):
            u = _u(seed, row, j, 1)
            if abs(u - alpha[ks][j]) <= TIE:
                excused = True
            if not u < alpha[ks][j]:
                L = j
                break
    else:
        L = force_L
    if L < G:
        r = [max(Decimal(0), a - b) for a, b in zip(P[ks][L], Q[ks][L])]
        if sum(r) == 0:
            r = P[ks][L]
        t = _u(seed, row, L, 2) * sum(r)
    else:
        r = P[ks][G]
        t = _u(seed, row, G, 3) * sum(r)
    tok, near = _draw(r, t)
    return ks, L, tok, excused or near


def _batch(rng, B, K, G, V, noise, bf16):
    zp = (rng.standard_normal((B, K, G + 1, V)) * 1.5).astype(np.float32)
    zq = (zp[:, :, :G] + rng.standard_normal((B, K, G, V)) * noise).astype(np.float32)
    if bf16:  # round to bf16 bit patterns (nearest even)
        def to_bf16(a):
            u = a.view(np.uint32)
            return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        zp, zq = to_bf16(zp), to_bf16(zq)
    # drafts: the drafter's most likely token or a random one
    top = (zq.astype(np.float32) if not bf16 else
           (zq.astype(np.uint32) << 16).view(np.float32)).argmax(axis=-1)
    rnd = rng.integers(0, V, size=(B, K, G))
    d = np.where(rng.random((B, K, G)) < 0.6, top, rnd).astype(np.int32)
    return zp, zq, d


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("noise", [0.05, 0.6])
def test_oracle_rule_equals_exact_arithmetic(orc, bf16, noise):
    rng = np.random.default_rng(int(noise * 100) + 7 * bf16)
    B, K, G, V = 10, 3, 4, 37
    Tp, Tq = np.float32(0.8), np.float32(1.1)
    seed, row_base = 0x5EED0000 + int(noise * 1000), 4242
    zp, zq, d = _batch(rng, B, K, G, V, noise, bf16)
    r = orc.select_and_verify(zp, zq, d, temp_p=float(Tp), temp_q=float(Tq), seed=seed,
                              row_base=row_base)
    checked = 0
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            ks, L, tok, excused = exact_prefix(zp[b], zq[b], d[b], Decimal(float(Tp)),
                                               Decimal(float(Tq)), seed, row_base + b)
            if excused:
                continue
            checked += 1
            assert (r.selected[b], r.accept_len[b], r.next_token[b]) == (ks, L, tok), b
    assert checked >= B - 2


def test_forced_positions_and_bonus_equal_exact_arithmetic(orc):
    # every position of a forced draft, and L = gamma (the bonus draw from p row
    # gamma with purpose 3), on prefixes with distinct rows and row numbers
    rng = np.random.default_rng(99)
    B, K, G, V = 12, 2, 3, 29
    zp, zq, d = _batch(rng, B, K, G, V, 0.4, False)
    fk = (np.arange(B) % K).astype(np.int32)
    fl = (np.arange(B) % (G + 1)).astype(np.int32)
    seed, row_base = 77, (1 << 40) + 3
    r = orc.select_and_verify(zp, zq, d, temp_p=1.0, seed=seed, row_base=row_base,
                              force_k=fk, force_L=fl)
    checked = 0
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            ks, L, tok, excused = exact_prefix(zp[b], zq[b], d[b], Decimal(1), Decimal(1), seed,
                                               row_base + b, force_k=int(fk[b]),
                                               force_L=int(fl[b]))
            assert (r.selected[b], r.accept_len[b]) == (ks, L)
            if excused:
                continue
            checked += 1
            assert r.next_token[b] == tok, b
    assert checked >= B - 1


def test_exact_reference_catches_a_wrong_purpose(orc):
    # the reference is sharp enough to see the uniform's purpose: drawing the
    # residual with purpose 3 instead of 2 changes some tokens
    rng = np.random.default_rng(5)
    B, K, G, V = 16, 1, 2, 31
    zp, zq, d = _batch(rng, B, K, G, V, 1.0, False)
    fl = np.zeros(B, np.int32)
    r = orc.select_and_verify(zp, zq, d, seed=3, force_k=np.zeros(B, np.int32), force_L=fl)
    differ = 0
    with localcontext() as ctx:
        ctx.prec = 50
        for b in range(B):
            P = _softmax(_widen(zp[b, 0, 0]), Decimal(1))
            Q = _softmax(_widen(zq[b, 0, 0]), Decimal(1))
            res = [max(Decimal(0), a - c) for a, c in zip(P, Q)]
            wrong, _ = _draw(res, _u(3, b, 0, 3) * sum(res))
            differ += wrong != r.next_token[b]
    assert differ >= 4
