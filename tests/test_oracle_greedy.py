"""Pins of the oracle's greedy-acceptance mode.

SpecDiff-2 section 5.2 verifies the kept draft without its drafting
probabilities; appendix B.4 states the rule: the uniform is compared with the
verifier probability of the drafted token, and a rejected token is resampled
from the verifier distribution with that token zeroed out.  The pins:

* exact law by enumeration (V = 3, gamma = 2, K = 1..3): with argmax
  self-selection over several drafts, the first committed token still follows
  p_0, and the second follows p_1 (the standard rule fails this at K > 1);
* chi-square over 200k seeded trials at K = 4: every committed position j
  follows p_j given that the window reached it;
* the same harness fails on a planted mistake (the rejected token not zeroed);
* the rule is the standard one with q the point mass at the drafted token;
* special cases: p one-hot at the drafted token always accepts; a drafted token
  of probability zero is always rejected and never redrawn.
"""
import itertools

import numpy as np
from scipy.special import softmax

from stats_util import _chisq_p


def _rows(seed, V, G, K, scale=1.2):
    rng = np.random.default_rng(seed)
    zp = (rng.standard_normal((1, 1, G + 1, V)) * scale).astype(np.float32)
    zq = (zp[:, :, :G, :] + rng.standard_normal((1, 1, G, V))).astype(np.float32)
    return (np.ascontiguousarray(np.broadcast_to(zp, (1, K, G + 1, V))),
            np.ascontiguousarray(np.broadcast_to(zq, (1, K, G, V))))


def _zeroed(p, x):
    r = p.copy()
    r[x] = 0.0
    return r / r.sum()


def _exact_greedy_law(orc, zp, zq, K):
    """Exact law of (y_0, y_1) for gamma = 2 over every combination of K drafts,
    each draft's tokens drawn from the q rows; alpha and the selection come
    from the oracle, the residual is p_j with the drafted token zeroed."""
    _, _, G1, V = zp.shape
    G = G1 - 1
    assert G == 2
    P = [softmax(zp[0, 0, j].astype(np.float64)) for j in range(G + 1)]
    Q = [softmax(zq[0, 0, j].astype(np.float64)) for j in range(G)]
    seqs = list(itertools.product(range(V), repeat=G))
    combos = list(itertools.product(range(len(seqs)), repeat=K))
    drafts = np.array([[seqs[i] for i in c] for c in combos], np.int32)
    n = len(combos)
    bp = np.ascontiguousarray(np.broadcast_to(zp, (n,) + zp.shape[1:]))
    res = orc.greedy_select_and_verify(bp, drafts)
    first = np.zeros(V)
    law = np.zeros((V, V))  # P(y_0 = a, y_1 = b, L >= 1)
    for c in range(n):
        w = np.prod([Q[j][drafts[c, k, j]] for k in range(K) for j in range(G)])
        ks = res.selected[c]
        x = drafts[c, ks]
        a = res.alpha[c, ks]
        assert abs(a[0] - P[0][x[0]]) < 1e-14 and abs(a[1] - P[1][x[1]]) < 1e-14
        first[x[0]] += w * a[0]
        first += w * (1 - a[0]) * _zeroed(P[0], x[0])
        law[x[0], x[1]] += w * a[0] * a[1]
        law[x[0]] += w * a[0] * (1 - a[1]) * _zeroed(P[1], x[1])
    return P, first, law


def test_exact_law_with_self_selection(orc):
    for K in (1, 2, 3):
        for seed in range(2):
            zp, zq = _rows(seed, V=3, G=2, K=K)
            P, first, law = _exact_greedy_law(orc, zp, zq, K)
            assert abs(first.sum() - 1) < 1e-12
            assert np.max(np.abs(first - P[0])) < 1e-12, (K, seed, first, P[0])
            for a in range(3):
                tot = law[a].sum()
                if tot > 1e-12:
                    assert np.max(np.abs(law[a] / tot - P[1])) < 1e-12


def _sample(rng, probs, size):
    c = np.cumsum(probs)
    return np.minimum(np.searchsorted(c / c[-1], rng.random(size), side="right"), len(probs) - 1)


def _greedy_trials(orc, n, K=4, V=32, G=4, seed=5):
    zp, zq = _rows(seed, V=V, G=G, K=K, scale=2.0)
    rng = np.random.default_rng(seed + 1)
    drafts = np.empty((n, K, G), np.int32)
    for j in range(G):
        drafts[:, :, j] = _sample(rng, softmax(zq[0, 0, j].astype(np.float64)), (n, K))
    bp = np.ascontiguousarray(np.broadcast_to(zp, (n,) + zp.shape[1:]))
    r = orc.greedy_select_and_verify(bp, drafts, seed=11, row_base=0)
    return zp, drafts, r


def _committed_pvalues(zp, drafts, sel, L, tok):
    G = drafts.shape[-1]
    V = zp.shape[-1]
    kept = drafts[np.arange(len(sel)), sel]  # [n, G]
    pv = []
    for j in range(G + 1):
        m = L >= j
        y = np.where(L[m] == j, tok[m], kept[m, min(j, G - 1)])
        pv.append(_chisq_p(np.bincount(y, minlength=V), softmax(zp[0, 0, j].astype(np.float64))))
    return pv


def test_chi_square_at_four_drafts(orc):
    zp, drafts, r = _greedy_trials(orc, 200_000)
    assert np.all(r.accept_len >= 0) and np.all(r.next_token >= 0)
    assert len(np.unique(r.selected)) == 4  # the selection is not trivial
    pv = _committed_pvalues(zp, drafts, r.selected, r.accept_len, r.next_token)
    assert min(pv) > 1e-3 / len(pv), pv


def test_chi_square_detects_a_planted_mistake(orc):
    # the rejected token not zeroed: replacements redrawn from the full p row
    zp, drafts, r = _greedy_trials(orc, 200_000)
    rng = np.random.default_rng(3)
    bad = r.next_token.copy()
    G = drafts.shape[-1]
    for j in range(G):
        m = r.accept_len == j
        bad[m] = _sample(rng, softmax(zp[0, 0, j].astype(np.float64)), m.sum())
    pv = _committed_pvalues(zp, drafts, r.selected, r.accept_len, bad)
    assert min(pv) < 1e-6, pv


def test_equals_standard_rule_with_point_mass_drafter(orc):
    rng = np.random.default_rng(21)
    B, K, G, V = 64, 3, 5, 50
    zp = (rng.standard_normal((B, K, G + 1, V)) * 2).astype(np.float32)
    drafts = rng.integers(0, V, (B, K, G)).astype(np.int32)
    zq = np.full((B, K, G, V), -np.inf, np.float32)
    np.put_along_axis(zq, drafts[..., None], 0.0, axis=-1)
    g = orc.greedy_select_and_verify(zp, drafts, temp_p=0.8, seed=4, row_base=9)
    s = orc.select_and_verify(zp, zq, drafts, temp_p=0.8, temp_q=1.0, seed=4, row_base=9)
    assert np.max(np.abs(g.alpha - s.alpha)) < 1e-13
    assert np.max(np.abs(g.scores - s.scores)) < 1e-12
    near = (g.select_gap < 1e-9) | (np.min(g.accept_margin, axis=1) < 1e-9) | (g.emit_margin < 1e-9)
    ok = ~near
    assert ok.sum() > 50
    for f in ("selected", "accept_len", "next_token"):
        assert np.array_equal(getattr(g, f)[ok], getattr(s, f)[ok]), f


def test_special_cases(orc):
    B, K, G, V = 8, 2, 3, 16
    rng = np.random.default_rng(2)
    drafts = rng.integers(0, V, (B, K, G)).astype(np.int32)
    # p one-hot at every drafted token: alpha = 1, the whole window is accepted
    zp = np.full((B, K, G + 1, V), -np.inf, np.float32)
    np.put_along_axis(zp[:, :, :G], drafts[..., None], 1.5, axis=-1)
    zp[:, :, G] = rng.standard_normal((B, K, V)).astype(np.float32)
    r = orc.greedy_select_and_verify(zp, drafts, seed=1)
    assert np.all(r.alpha == 1.0) and np.all(r.accept_len == G)
    assert np.all((r.next_token >= 0) & (r.next_token < V))
    # drafted token with probability zero: rejected at once, never redrawn
    zp = rng.standard_normal((B, K, G + 1, V)).astype(np.float32)
    np.put_along_axis(zp[:, :, :G], drafts[..., None], -np.inf, axis=-1)
    r = orc.greedy_select_and_verify(zp, drafts, seed=1)
    assert np.all(r.alpha == 0.0) and np.all(r.accept_len == 0)
    assert np.all(r.next_token != drafts[np.arange(B), r.selected, 0])
    # a drafted token outside the vocabulary invalidates its prefix only
    d2 = drafts.copy()
    d2[3, 1, 2] = V
    r = orc.greedy_select_and_verify(rng.standard_normal((B, K, G + 1, V)).astype(np.float32), d2)
    assert r.selected[3] == -1 and r.accept_len[3] == -1 and r.next_token[3] == -1
    assert np.all(np.delete(r.accept_len, 3) >= 0)
