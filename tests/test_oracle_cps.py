"""Pins of the oracle's causal-consistency path search (DiffuSpec section 4.2:
prune each position's candidates by cumulative mass, stop at the first EOS,
beam-search paths scored by drafter confidence and a causal-proxy fluency;
settings B = 3, M_max = 15, tau = 0.8 in section 5.3).

* the lattice equals scipy's softmax and numpy's ordering (logit descending,
  lower index on a tie) cut at cumulative mass tau, capped at m_max;
* the lattice stops at the first position whose top token is EOS;
* a beam as wide as the number of paths is exhaustive: the top paths by total
  score, against brute-force enumeration;
* a beam of one is the greedy path, computed directly;
* exact ties keep the earlier expansion.
"""
import itertools

import numpy as np
from scipy.special import softmax

import oracle


def _rows(seed, B, G, V, scale=2.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, G, V)) * scale).astype(np.float32)


def test_lattice_matches_sorted_softmax():
    z = _rows(0, 3, 5, 200)
    z[0, 1, 17] = z[0, 1, 18] = z[0, 1].max() + 1.0  # a tie at the top
    for tau, m_max, T in ((0.8, 15, 1.0), (0.5, 4, 0.7), (0.99, 30, 1.3)):
        lat = oracle.cps_lattice(z, temp_q=T, tau=tau, m_max=m_max)
        for b in range(3):
            for j in range(5):
                row = z[b, j].astype(np.float64)
                p = softmax(row / np.float64(np.float32(T)))
                order = np.lexsort((np.arange(200), -row))
                cum = np.cumsum(p[order])
                n = min(int(np.searchsorted(cum, tau) + 1), m_max)
                while n > 1 and cum[n - 2] >= tau:
                    n -= 1
                assert lat["n_cand"][b, j] == n, (tau, b, j)
                assert list(lat["cand"][b, j, :n]) == list(order[:n])
                assert np.all(lat["cand"][b, j, n:] == -1)
                assert np.allclose(lat["cand_logp"][b, j, :n], np.log(p[order[:n]]), atol=1e-12)
        assert np.all(lat["len"] == 5)
    lat = oracle.cps_lattice(z, tau=0.8)
    assert list(lat["cand"][0, 1, :2]) == [17, 18]


def test_lattice_stops_at_the_first_eos():
    z = _rows(1, 2, 6, 50)
    eos = 7
    z[0, 3, eos] = z[0, 3].max() + 3.0   # EOS on top at position 3 of prefix 0
    z[0, 5, eos] = z[0, 5].max() + 3.0   # and again later: irrelevant
    z[1, 2, eos] = z[1, 2].max() - 0.01  # a close second only: no stop
    lat = oracle.cps_lattice(z, tau=0.8, m_max=6, eos=eos)
    assert list(lat["len"]) == [4, 6]
    assert lat["n_cand"][0, 3] == 1 and lat["cand"][0, 3, 0] == eos
    assert np.all(lat["n_cand"][0, 4:] == 0) and np.all(lat["cand"][0, 4:] == -1)
    assert lat["n_cand"][1, 2] >= 2


def _paths_by_brute_force(lat, f, lam, b):
    n, ln = lat["n_cand"][b], lat["len"][b]
    out = []
    for ranks in itertools.product(*[range(n[j]) for j in range(ln)]):
        s, prev = 0.0, 0
        for j, i in enumerate(ranks):
            s += lat["cand_logp"][b, j, i] + (lam * float(f[b, j, prev, i]) if f is not None else 0)
            prev = i
        out.append((s, [int(lat["cand"][b, j, i]) for j, i in enumerate(ranks)]))
    out.sort(key=lambda t: -t[0])
    return out


def test_wide_beam_is_exhaustive():
    z = _rows(2, 4, 3, 40, scale=0.7)
    lat = oracle.cps_lattice(z, tau=0.6, m_max=3)
    rng = np.random.default_rng(3)
    f = rng.standard_normal((4, 3, 3, 3)).astype(np.float32)
    width = int(np.max(np.prod(lat["n_cand"], axis=1)))
    res = oracle.cps_beam(lat, f, lam=0.5, beam=width)
    for b in range(4):
        ref = _paths_by_brute_force(lat, f, 0.5, b)
        for r, (s, toks) in enumerate(ref):
            assert abs(res["score"][b, r] - s) < 1e-12
            assert list(res["paths"][b, r, :len(toks)]) == toks
        assert np.all(res["path_len"][b, len(ref):] == 0)


def test_beam_of_one_is_the_greedy_path():
    z = _rows(4, 3, 6, 60, scale=1.0)
    lat = oracle.cps_lattice(z, tau=0.9, m_max=5)
    f = np.random.default_rng(5).standard_normal((3, 6, 5, 5)).astype(np.float32)
    res = oracle.cps_beam(lat, f, lam=2.0, beam=1)
    for b in range(3):
        prev, s, toks = 0, 0.0, []
        for j in range(6):
            n = lat["n_cand"][b, j]
            vals = [lat["cand_logp"][b, j, i] + 2.0 * float(f[b, j, prev, i]) for i in range(n)]
            i = int(np.argmax(vals))
            s += vals[i]
            toks.append(int(lat["cand"][b, j, i]))
            prev = i
        assert list(res["paths"][b, 0]) == toks and abs(res["score"][b, 0] - s) < 1e-12


def test_exact_ties_keep_the_earlier_expansion():
    lat = {"cand": np.array([[[5, 6], [8, 9]]], np.int32),
           "cand_logp": np.full((1, 2, 2), -1.0), "n_cand": np.array([[2, 2]], np.int32),
           "len": np.array([2], np.int32)}
    res = oracle.cps_beam(lat, None, beam=3)
    assert res["paths"][0].tolist() == [[5, 8], [5, 9], [6, 8]]
    assert res["rank_margin"][0] == 0.0


def test_nan_proxy_scores_rank_last():
    # a proxy score of NaN makes its expansion unusable: it ranks below every
    # finite one, as if the score were -inf
    lat = {"cand": np.array([[[5, 6], [8, 9]]], np.int32),
           "cand_logp": np.full((1, 2, 2), -1.0), "n_cand": np.array([[2, 2]], np.int32),
           "len": np.array([2], np.int32)}
    f = np.zeros((1, 2, 2, 2), np.float32)
    f[0, 0, 0, 0] = np.nan  # candidate 0 after the context
    res = oracle.cps_beam(lat, f, lam=0.5, beam=2)
    assert res["paths"][0].tolist() == [[6, 8], [6, 9]]
    # on random lattices, NaN entries act as -inf entries
    z = _rows(6, 3, 4, 50, scale=1.0)
    lat = oracle.cps_lattice(z, tau=0.9, m_max=4)
    rng = np.random.default_rng(7)
    f = rng.standard_normal((3, 4, 4, 4)).astype(np.float32)
    hole = rng.random(f.shape) < 0.1
    a = oracle.cps_beam(lat, np.where(hole, np.float32(np.nan), f), lam=0.5, beam=3)
    b = oracle.cps_beam(lat, np.where(hole, np.float32(-np.inf), f), lam=0.5, beam=3)
    assert np.array_equal(a["paths"], b["paths"]) and np.array_equal(a["score"], b["score"])
