"""Pins of the oracle's shared-row layout (drafter rows shared by the K drafts
of one denoising pass, SpecDiff-2 section 5.2; verifier rows shared by drafts
with a common prefix, the flattened draft tree of SpecDiff-2 appendix B.8).

The layout is defined as the dense rule on the gathered rows, so the pins check
the gather: identity indices reproduce the dense oracle bit for bit, shared
rows reproduce the dense oracle on the broadcast rows bit for bit, a permuted
pool with permuted indices changes nothing, and an index outside a pool
invalidates exactly the prefixes that read it.
"""
import numpy as np

import oracle
import workloads as W


def _dense_case(seed, B=5, K=3, G=4, V=300):
    cfg = W.Config(80, "custom", B=B, K=K, gamma=G, V=V, dtype="bf16", sigma0=1.0,
                   sigma_step=0.0, temp=0.9, boost=5.0, boost_prob=1.0)
    d = W.generate(cfg, data_seed=seed)
    return W.to_host(d["p"]), W.to_host(d["q"]), W.to_host(d["drafts"])


def _same(a, b):
    for f in ("selected", "accept_len", "next_token"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    for f in ("alpha", "scores", "emit_margin"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(np.nan_to_num(x, nan=-7), np.nan_to_num(y, nan=-7)), f


def test_identity_indices_equal_the_dense_rule():
    hp, hq, hd = _dense_case(1)
    B, K, G1, V = hp.shape
    G = G1 - 1
    p_pool = hp.reshape(-1, V)
    q_pool = hq.reshape(-1, V)
    p_index = np.arange(B * K * G1, dtype=np.int32).reshape(B, K, G1)
    q_index = np.arange(B * K * G, dtype=np.int32).reshape(B, K, G)
    for greedy in (False, True):
        a = oracle.select_and_verify_rows(p_pool, p_index, q_pool, q_index, hd, temp_p=0.9,
                                          seed=3, row_base=2, greedy=greedy)
        if greedy:
            b = oracle.greedy_select_and_verify(hp, hd, temp_p=0.9, seed=3, row_base=2)
        else:
            b = oracle.select_and_verify(hp, hq, hd, temp_p=0.9, seed=3, row_base=2)
        _same(a, b)


def test_shared_rows_equal_the_dense_rule_on_broadcast_rows():
    cfg = W.get_config("shared_marginal")
    d = W.generate_pooled(cfg, B=4, V=500)
    pp, pi = W.to_host(d["p_pool"]), W.to_host(d["p_index"])
    qp, qi, hd = W.to_host(d["q_pool"]), W.to_host(d["q_index"]), W.to_host(d["drafts"])
    # the drafter rows are shared by the K drafts and row 0 of p by all drafts
    assert np.all(qi == qi[:, :1]) and np.all(pi[:, :, 0] == pi[:, :1, 0])
    assert pp.shape[0] < pi.size and qp.shape[0] < qi.size
    dense_p = np.ascontiguousarray(pp[pi])
    dense_q = np.ascontiguousarray(qp[qi])
    for greedy in (False, True):
        a = oracle.select_and_verify_rows(pp, pi, qp, qi, hd, temp_p=cfg.temp, seed=5,
                                          greedy=greedy)
        b = (oracle.greedy_select_and_verify(dense_p, hd, temp_p=cfg.temp, seed=5) if greedy
             else oracle.select_and_verify(dense_p, dense_q, hd, temp_p=cfg.temp, seed=5))
        _same(a, b)


def test_permuted_pools_change_nothing():
    hp, hq, hd = _dense_case(2)
    B, K, G1, V = hp.shape
    G = G1 - 1
    rng = np.random.default_rng(0)
    pp = rng.permutation(B * K * G1)
    qp = rng.permutation(B * K * G)
    p_pool = np.empty((B * K * G1, V), hp.dtype)
    p_pool[pp] = hp.reshape(-1, V)
    q_pool = np.empty((B * K * G, V), hq.dtype)
    q_pool[qp] = hq.reshape(-1, V)
    a = oracle.select_and_verify_rows(p_pool, pp.reshape(B, K, G1).astype(np.int32), q_pool,
                                      qp.reshape(B, K, G).astype(np.int32), hd, temp_p=0.9,
                                      seed=4)
    _same(a, oracle.select_and_verify(hp, hq, hd, temp_p=0.9, seed=4))


def test_an_index_outside_the_pool_invalidates_its_prefix_only():
    hp, hq, hd = _dense_case(3, B=6)
    B, K, G1, V = hp.shape
    G = G1 - 1
    p_pool, q_pool = hp.reshape(-1, V), hq.reshape(-1, V)
    pi = np.arange(B * K * G1, dtype=np.int32).reshape(B, K, G1)
    qi = np.arange(B * K * G, dtype=np.int32).reshape(B, K, G)
    pi[1, 2, 1] = p_pool.shape[0]       # scored verifier row
    qi[3, 0, 2] = -1                    # scored drafter row
    r = oracle.select_and_verify_rows(p_pool, pi, q_pool, qi, hd, temp_p=0.9, seed=1)
    bad = {1, 3}
    for b in range(B):
        if b in bad:
            assert r.selected[b] == -1 and r.accept_len[b] == -1 and r.next_token[b] == -1
        else:
            assert r.accept_len[b] >= 0 and r.next_token[b] >= 0
    # a bonus row outside the pool matters only when the bonus is drawn
    ref = oracle.select_and_verify(hp, hq, hd, temp_p=0.9, seed=1)
    pi2 = np.arange(B * K * G1, dtype=np.int32).reshape(B, K, G1)
    pi2[:, :, G] = -5
    r2 = oracle.select_and_verify_rows(p_pool, pi2, q_pool, qi * 0 + np.arange(
        B * K * G, dtype=np.int32).reshape(B, K, G), hd, temp_p=0.9, seed=1)
    full = ref.accept_len == G
    assert 0 < full.sum() < B
    assert np.all(r2.accept_len[full] == -1)
    assert np.array_equal(r2.next_token[~full], ref.next_token[~full])
