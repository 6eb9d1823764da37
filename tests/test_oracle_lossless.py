"""Losslessness of the oracle: committed tokens follow the verifier.

SpecDiff-2 section 2 and DiffuSpec section 3: accepting or resampling as the
rule says leaves the committed tokens distributed exactly as the verifier's own
samples would be.  Two pins:

* brute force: for a tiny vocabulary and window, enumerate every draft and
  compute the exact law of the committed tokens from the oracle's alpha and
  draw weights; each committed position must follow its verifier row;
* chi-square: the tiny workload (V = 32, gamma = 4, fp32) with 10^6 seeded
  trials, each with fresh drafts and its own uniform stream (row = trial).

Self-selection over K > 1 drafts followed by this rule is not lossless; the
brute-force check documents that too.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import chi2

import workloads as W
from stats_util import accepted_length_pvalue, committed_token_pvalues, tiny_trials


def _tiny_rows(seed, V, G, K=1):
    rng = np.random.default_rng(seed)
    zp = (rng.standard_normal((1, 1, G + 1, V)) * 1.2).astype(np.float32)
    zq = (zp[:, :, :G, :] + rng.standard_normal((1, 1, G, V))).astype(np.float32)
    zp = np.ascontiguousarray(np.broadcast_to(zp, (1, K, G + 1, V)))
    zq = np.ascontiguousarray(np.broadcast_to(zq, (1, K, G, V)))
    return zp, zq


def _exact_law(orc, zp, zq, K):
    """Exact law of (y_0, y_1, accepted length) for gamma = 2, from oracle pieces."""
    _, _, G1, V = zp.shape
    G = G1 - 1
    assert G == 2
    P = [orc.softmax_row(zp[0, 0, j]) for j in range(G + 1)]
    Q = [orc.softmax_row(zq[0, 0, j]) for j in range(G)]
    R = []
    for j in range(G):
        r, Z = orc.draw_weights(P[j], Q[j])
        R.append(r / Z)
    seqs = list(itertools.product(range(V), repeat=G))
    # every combination of K drafts
    combos = list(itertools.product(range(len(seqs)), repeat=K))
    drafts = np.array([[seqs[i] for i in c] for c in combos], np.int32)
    n = len(combos)
    bp = np.ascontiguousarray(np.broadcast_to(zp, (n,) + zp.shape[1:]))
    bq = np.ascontiguousarray(np.broadcast_to(zq, (n,) + zq.shape[1:]))
    res = orc.select_and_verify(bp, bq, drafts)
    law = np.zeros((V, V))        # P(y_0 = a, y_1 = b, L >= 1)
    first = np.zeros(V)           # P(y_0 = a)
    for c in range(n):
        w = np.prod([Q[j][drafts[c, k, j]] for k in range(K) for j in range(G)])
        ks = res.selected[c]
        x = drafts[c, ks]
        a = res.alpha[c, ks]
        first += w * (1 - a[0]) * R[0]
        first[x[0]] += w * a[0]
        # L >= 1: y_0 = x_0, then position 1 either accepts or draws from R[1]
        law[x[0]] += w * a[0] * (1 - a[1]) * R[1]
        law[x[0], x[1]] += w * a[0] * a[1]
    return P, first, law


def test_brute_force_single_draft_is_lossless(orc):
    for seed in range(3):
        zp, zq = _tiny_rows(seed, V=3, G=2)
        P, first, law = _exact_law(orc, zp, zq, K=1)
        assert np.max(np.abs(first - P[0])) < 1e-12
        for a in range(3):
            tot = law[a].sum()
            if tot > 0:
                assert np.max(np.abs(law[a] / tot - P[1])) < 1e-12


def test_brute_force_four_tokens(orc):
    zp, zq = _tiny_rows(9, V=4, G=2)
    P, first, law = _exact_law(orc, zp, zq, K=1)
    assert np.max(np.abs(first - P[0])) < 1e-12


def test_brute_force_argmax_selection_is_biased(orc):
    # two drafts from the same marginals, argmax of the expected streak, then
    # the standard rule: the first committed token no longer follows p_0
    zp, zq = _tiny_rows(0, V=3, G=2, K=2)
    P, first, _ = _exact_law(orc, zp, zq, K=2)
    assert abs(first.sum() - 1) < 1e-12
    assert np.max(np.abs(first - P[0])) > 1e-3


@pytest.mark.slow
def test_tiny_workload_chi_square_1e6(orc):
    n = W.get_config(1).trials
    assert n == 1_000_000
    cfg, zp, zq, drafts, L, tok = tiny_trials(orc, n)
    assert np.all(L >= 0) and np.all(tok >= 0)
    pv = committed_token_pvalues(zp, zq, drafts, L, tok, cfg.temp)
    G = drafts.shape[-1]
    # Bonferroni over gamma + 1 positions at 1e-3
    assert min(pv) > 1e-3 / (G + 1), pv
    assert accepted_length_pvalue(zp, zq, L, cfg.temp) > 1e-3


def test_chi_square_detects_a_planted_mistake(orc):
    # the same harness must fail when the residual ignores q (drawing from p):
    # a plausible mistake, planted on the CPU by replacing the draws
    cfg, zp, zq, drafts, L, tok = tiny_trials(orc, 200_000)
    rng = np.random.default_rng(0)
    bad = tok.copy()
    for j in range(drafts.shape[-1]):
        sel = L == j
        pj = softmax(zp[0, 0, j].astype(np.float64))
        bad[sel] = rng.choice(len(pj), size=sel.sum(), p=pj)
    pv = committed_token_pvalues(zp, zq, drafts, L, bad, cfg.temp)
    assert min(pv) < 1e-6
    pv_ok = committed_token_pvalues(zp, zq, drafts, L, tok, cfg.temp)
    assert min(pv_ok) > 1e-3 / 5
