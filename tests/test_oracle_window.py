"""Pins of the oracle's ragged, EOS-aware windows (DiffuSpec section 3,
"Accepted prefix length": a step commits the kept draft's accepted tokens and
an accepted EOS finishes the sequence; section 4.3: k_t is chosen per step).

* full windows without EOS reproduce the dense oracle bit for bit;
* a window of n positions equals the dense oracle on the arrays cut to n
  positions (p rows 0..n, bonus row n, uniforms of position n), bit for bit;
* with EOS and one draft, the result equals the dense oracle on the window cut
  after the draft's first EOS, except that a fully accepted window ending in EOS
  draws nothing (next_token -2);
* each draft's score stops at its first EOS (K > 1: every draft cut alone);
* the first committed token still follows the verifier row 0 (chi-square).
"""
import numpy as np
from scipy.special import softmax

import oracle
import workloads as W
from stats_util import _chisq_p


def _case(seed, B=12, K=1, G=6, V=64, dt="f32", boost=4.0):
    cfg = W.Config(81, "custom", B=B, K=K, gamma=G, V=V, dtype=dt, sigma0=0.6, sigma_step=0.0,
                   temp=1.0, boost=boost, boost_prob=1.0)
    d = W.generate(cfg, data_seed=seed)
    return W.to_host(d["p"]), W.to_host(d["q"]), W.to_host(d["drafts"])


def _eq(a, b, fields=("selected", "accept_len", "next_token")):
    for f in fields:
        assert np.array_equal(getattr(a, f), getattr(b, f)), (f, getattr(a, f), getattr(b, f))


def test_full_windows_equal_the_dense_rule():
    hp, hq, hd = _case(1, K=3)
    B, K, G1, _ = hp.shape
    full = np.full(B, G1 - 1, np.int32)
    for greedy in (False, True):
        a = oracle.window_select_and_verify(hp, hq, hd, gamma_b=full, greedy=greedy, seed=4)
        b = (oracle.greedy_select_and_verify(hp, hd, seed=4) if greedy else
             oracle.select_and_verify(hp, hq, hd, seed=4))
        _eq(a, b, ("selected", "accept_len", "next_token", "scores", "emit_margin"))


def _cut(hp, hq, hd, b, n):
    """Prefix b's arrays cut to a window of n positions (bonus row n)."""
    p = np.ascontiguousarray(np.concatenate([hp[b:b + 1, :, :n], hp[b:b + 1, :, n:n + 1]], 2))
    return p, np.ascontiguousarray(hq[b:b + 1, :, :n]), np.ascontiguousarray(hd[b:b + 1, :, :n])


def test_ragged_windows_equal_cut_arrays():
    hp, hq, hd = _case(2, K=2, B=16)
    B, K, G1, _ = hp.shape
    G = G1 - 1
    n = (np.arange(B) % G + 1).astype(np.int32)
    for greedy in (False, True):
        r = oracle.window_select_and_verify(hp, hq, hd, gamma_b=n, greedy=greedy, seed=9,
                                            row_base=100)
        for b in range(B):
            p, q, d = _cut(hp, hq, hd, b, int(n[b]))
            ref = (oracle.greedy_select_and_verify(p, d, seed=9, row_base=100 + b) if greedy else
                   oracle.select_and_verify(p, q, d, seed=9, row_base=100 + b))
            for f in ("selected", "accept_len", "next_token"):
                assert getattr(r, f)[b] == getattr(ref, f)[0], (greedy, b, f)
            assert np.array_equal(r.scores[b], ref.scores[0])
            assert np.all(np.isnan(r.alpha[b, :, n[b]:]))


def test_window_outside_its_range_invalidates_the_prefix():
    hp, hq, hd = _case(3, B=4)
    n = np.array([0, 3, 7, 6], np.int32)
    r = oracle.window_select_and_verify(hp, hq, hd, gamma_b=n, seed=1)
    assert list(r.accept_len[[0, 2]]) == [-1, -1] and np.all(r.accept_len[[1, 3]] >= 0)


def test_eos_with_one_draft_equals_the_window_cut_after_it():
    hp, hq, hd = _case(4, B=40, G=6, V=16, boost=6.0)
    B, _, G1, _ = hp.shape
    G = G1 - 1
    eos = 5
    hd = hd.copy()
    hd[::3, 0, 2] = eos  # every third prefix drafts EOS at position 2
    for greedy in (False, True):
        r = oracle.window_select_and_verify(hp, hq, hd, eos=eos, greedy=greedy, seed=2)
        ended = 0
        for b in range(B):
            hits = np.nonzero(hd[b, 0] == eos)[0]
            m = int(hits[0]) + 1 if len(hits) else G
            p, q, d = _cut(hp, hq, hd, b, m)
            ref = (oracle.greedy_select_and_verify(p, d, seed=2, row_base=b) if greedy else
                   oracle.select_and_verify(p, q, d, seed=2, row_base=b))
            assert r.accept_len[b] == ref.accept_len[0]
            if len(hits) and ref.accept_len[0] == m:
                assert r.next_token[b] == -2  # the accepted EOS ends the commit
                ended += 1
            else:
                assert r.next_token[b] == ref.next_token[0]
        assert ended > 0


def test_each_score_stops_at_its_drafts_eos():
    hp, hq, hd = _case(5, B=6, K=4, G=8, V=16, boost=6.0)
    eos = 3
    hd = hd.copy()
    hd[:, 1, 1] = eos
    hd[:, 2, 5] = eos
    r = oracle.window_select_and_verify(hp, hq, hd, eos=eos, seed=7)
    G = hd.shape[-1]
    for b in range(hp.shape[0]):
        for k in range(4):
            hits = np.nonzero(hd[b, k] == eos)[0]
            m = int(hits[0]) + 1 if len(hits) else G
            p = np.ascontiguousarray(np.concatenate([hp[b:b + 1, k:k + 1, :m],
                                                     hp[b:b + 1, k:k + 1, m:m + 1]], 2))
            ref = oracle.select_and_verify(p, np.ascontiguousarray(hq[b:b + 1, k:k + 1, :m]),
                                           np.ascontiguousarray(hd[b:b + 1, k:k + 1, :m]), seed=7)
            assert r.scores[b, k] == ref.scores[0, 0]


def test_first_committed_token_follows_the_verifier_with_eos():
    cfg = W.get_config(1)
    base = W.generate(cfg)
    zp, zq = W.to_host(base["p"]), W.to_host(base["q"])
    n = 100_000
    drafts = W.tiny_trial_drafts(base["q"], n, cfg.temp, seed=77).numpy()
    eos = int(np.argmax(zq[0, 0, 0]))  # the drafter's favourite first token ends windows often
    bp = np.ascontiguousarray(np.broadcast_to(zp, (n,) + zp.shape[1:]))
    bq = np.ascontiguousarray(np.broadcast_to(zq, (n,) + zq.shape[1:]))
    r = oracle.window_select_and_verify(bp, bq, drafts, eos=eos, seed=3)
    assert np.mean(r.next_token == -2) > 0.05
    y0 = np.where(r.accept_len == 0, r.next_token, drafts[:, 0, 0])
    p0 = softmax(zp[0, 0, 0].astype(np.float64))
    assert _chisq_p(np.bincount(y0, minlength=zp.shape[-1]), p0) > 1e-3
