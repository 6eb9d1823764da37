"""Pins of the oracle's acceptance, overlap mass, streak score and self-selection.

Each check rests on a fact fixed by the pages or by mathematics, not on the
oracle's own formulas:
  * immediate acceptance whenever q(x) <= p(x) (SpecDiff-2 section 2);
  * a one-hot drafter turns the rule into the greedy rule that compares a
    uniform with p(x) (SpecDiff-2 appendix B.4), so alpha must equal p(x);
  * sum_v min(p_v, q_v) = 1 - TV(p, q) = 1 - 0.5 sum_v |p_v - q_v|;
  * the chance of accepting position 0 with a fresh draft x ~ q is sum min(p, q);
  * for a fixed draft, E[accepted length] = sum_j prod_{i<=j} alpha_i, so the
    mean accepted length over independent uniforms pins the streak score;
  * a closed form of that sum for constant alpha;
  * self-selection keeps the draft of greatest score, the lowest on a tie
    (SpecDiff-2 section 5.2).
"""
import numpy as np
import pytest
from scipy.special import softmax


def rows(rng, K, G, V, sigma=1.0, boost=6.0):
    zp = rng.standard_normal((1, K, G + 1, V)) * 2.0
    for k in range(K):
        for j in range(G + 1):
            zp[0, k, j, rng.integers(V)] += boost
    zq = zp[:, :, :G, :] + sigma * rng.standard_normal((1, K, G, V))
    return zp.astype(np.float32), zq.astype(np.float32)


def probs(z, T=1.0):
    return softmax(z.astype(np.float64) / np.float64(np.float32(T)), axis=-1)


def run(orc, zp, zq, d, **kw):
    return orc.select_and_verify(zp, zq, np.asarray(d, np.int32), **kw)


def test_alpha_is_one_whenever_q_le_p(orc):
    rng = np.random.default_rng(1)
    zp, zq = rows(rng, 1, 6, 40)
    P, Q = probs(zp[0, 0, :6]), probs(zq[0, 0])
    # pick, for every position, a token with q <= p and one with q > p
    d_le = np.array([[[int(np.flatnonzero(Q[j] <= P[j])[0]) for j in range(6)]]])
    d_gt = np.array([[[int(np.flatnonzero(Q[j] > P[j])[0]) for j in range(6)]]])
    r = run(orc, zp, zq, d_le)
    assert np.all(r.alpha == 1.0)
    r = run(orc, zp, zq, d_gt)
    assert np.all(r.alpha < 1.0) and np.all(r.alpha > 0.0)


def test_identical_drafter_accepts_everything(orc):
    rng = np.random.default_rng(2)
    zp, _ = rows(rng, 2, 5, 33)
    zq = np.ascontiguousarray(zp[:, :, :5, :])
    d = rng.integers(0, 33, (1, 2, 5))
    for seed in range(20):
        r = run(orc, zp, zq, d, seed=seed, want_beta=True)
        assert np.all(r.alpha == 1.0)
        assert np.max(np.abs(r.beta - 1.0)) < 1e-15
        assert r.accept_len[0] == 5
        assert np.all(r.scores == 5.0)
        assert r.selected[0] == 0  # exact tie: lowest k


def test_one_hot_drafter_gives_greedy_acceptance(orc):
    rng = np.random.default_rng(3)
    V, G = 50, 4
    zp, _ = rows(rng, 1, G, V)
    d = rng.integers(0, V, (1, 1, G))
    zq = np.full((1, 1, G, V), -np.inf, np.float32)
    for j in range(G):
        zq[0, 0, j, d[0, 0, j]] = 0.0
    r = run(orc, zp, zq, d)
    P = probs(zp[0, 0, :G])
    want = P[np.arange(G), d[0, 0]]
    assert np.max(np.abs(r.alpha[0, 0] - want)) < 1e-15
    assert np.all(r.qx == 1.0)


def test_zero_drafter_mass_accepts_and_zero_verifier_mass_rejects(orc):
    rng = np.random.default_rng(4)
    zp, zq = rows(rng, 1, 3, 16)
    d = np.array([[[2, 5, 7]]])
    zq[0, 0, 0, 2] = -np.inf          # q(x_0) = 0 -> accept
    zp[0, 0, 1, 5] = -np.inf          # p(x_1) = 0 < q(x_1) -> reject
    for seed in range(10):
        r = run(orc, zp, zq, d, seed=seed)
        assert r.alpha[0, 0, 0] == 1.0 and r.alpha[0, 0, 1] == 0.0
        assert r.accept_len[0] == 1
        # the residual at position 1 never re-emits the rejected token
        assert r.next_token[0] != 5


def test_beta_is_one_minus_total_variation(orc):
    rng = np.random.default_rng(5)
    zp, zq = rows(rng, 3, 7, 97, sigma=1.3)
    d = rng.integers(0, 97, (1, 3, 7))
    r = run(orc, zp, zq, d, want_beta=True, temp_p=0.7)
    P, Q = probs(zp[0, :, :7], 0.7), probs(zq[0], 0.7)
    tv = 0.5 * np.abs(P - Q).sum(-1)
    assert np.max(np.abs(r.beta[0] - (1.0 - tv))) < 1e-13


def _stack(zp, zq, n):
    return (np.ascontiguousarray(np.broadcast_to(zp, (n,) + zp.shape[1:])),
            np.ascontiguousarray(np.broadcast_to(zq, (n,) + zq.shape[1:])))


def test_acceptance_rate_at_position_zero_is_beta(orc):
    # fresh drafts x ~ q_0: P(accept position 0) = sum_v min(p_v, q_v)
    rng = np.random.default_rng(6)
    V, n = 24, 200_000
    zp, zq = rows(rng, 1, 1, V, sigma=1.0, boost=3.0)
    P, Q = probs(zp[0, 0, :1])[0], probs(zq[0, 0])[0]
    beta = np.minimum(P, Q).sum()
    d = rng.choice(V, size=(n, 1, 1), p=Q)
    bp, bq = _stack(zp, zq, n)
    r = run(orc, bp, bq, d, seed=77)
    rate = (r.accept_len >= 1).mean()
    sd = np.sqrt(beta * (1 - beta) / n)
    assert abs(rate - beta) < 5 * sd


def test_streak_score_closed_form(orc):
    # identical rows and tokens at every position give a constant alpha = a;
    # then sum_{j<G} a^{j+1} = (a - a^{G+1}) / (1 - a)
    rng = np.random.default_rng(7)
    V, G = 40, 9
    zp1, zq1 = rows(rng, 1, 1, V)
    P, Q = probs(zp1[0, 0, 0]), probs(zq1[0, 0, 0])
    x = int(np.flatnonzero(Q > P)[0])
    zp = np.ascontiguousarray(np.broadcast_to(zp1[:, :, :1, :], (1, 1, G + 1, V)))
    zq = np.ascontiguousarray(np.broadcast_to(zq1[:, :, :1, :], (1, 1, G, V)))
    r = run(orc, zp, zq, np.full((1, 1, G), x))
    a = r.alpha[0, 0, 0]
    assert a < 1 and np.all(r.alpha == a)
    assert abs(r.scores[0, 0] - (a - a ** (G + 1)) / (1 - a)) < 1e-14


def test_score_is_expected_accepted_length(orc):
    # fixed draft, independent uniform streams (one per row): mean L -> score
    rng = np.random.default_rng(8)
    V, G, n = 30, 6, 100_000
    zp, zq = rows(rng, 1, G, V, sigma=0.6)
    d = rng.integers(0, V, (1, 1, G))
    Q = probs(zq[0, 0])
    d[0, 0] = Q.argmax(-1)  # likely tokens keep alpha away from 0
    bp, bq = _stack(zp, zq, n)
    r = run(orc, bp, bq, np.broadcast_to(d, (n, 1, G)), seed=5)
    S = r.scores[0, 0]
    L = r.accept_len.astype(np.float64)
    assert abs(L.mean() - S) < 5 * L.std() / np.sqrt(n)
    # and the law of L: P(L >= j) = prod_{i<j} alpha_i
    a = r.alpha[0, 0]
    for j in range(1, G + 1):
        pj = np.prod(a[:j])
        sd = np.sqrt(pj * (1 - pj) / n) + 1e-12
        assert abs((L >= j).mean() - pj) < 5 * sd + 1e-9


def test_selection_keeps_the_best_draft(orc):
    rng = np.random.default_rng(9)
    V, G, K = 64, 5, 6
    zp, zq = rows(rng, K, G, V, sigma=1.5)
    d = rng.integers(0, V, (1, K, G))
    # draft 3 copies the verifier exactly: alpha == 1, score == G, the maximum
    zq[0, 3] = zp[0, 3, :G]
    r = run(orc, zp, zq, d)
    assert r.scores[0, 3] == G
    assert r.selected[0] == 3
    assert np.all(r.scores[0] <= G)


def test_exact_tie_goes_to_lowest_index(orc):
    rng = np.random.default_rng(10)
    V, G, K = 20, 4, 5
    zp, zq = rows(rng, 1, G, V, sigma=1.5)
    zpK = np.ascontiguousarray(np.broadcast_to(zp, (1, K, G + 1, V)))
    zqK = np.ascontiguousarray(np.broadcast_to(zq, (1, K, G, V)))
    d = np.broadcast_to(rng.integers(0, V, (1, 1, G)), (1, K, G))
    r = run(orc, zpK, zqK, d)
    assert np.all(r.scores[0] == r.scores[0, 0])
    assert r.selected[0] == 0
    # make draft 2 strictly better at its last position only
    zqK[0, 2, G - 1] = zpK[0, 2, G - 1]
    r2 = run(orc, zpK, zqK, d)
    if r2.scores[0, 2] > r.scores[0, 0]:
        assert r2.selected[0] == 2


def test_acceptance_stops_at_first_rejection(orc):
    rng = np.random.default_rng(11)
    V, G = 30, 8
    zp, zq = rows(rng, 1, G, V, sigma=2.0)
    d = rng.integers(0, V, (1, 1, G))
    for seed in range(50):
        r = run(orc, zp, zq, d, seed=seed)
        L = r.accept_len[0]
        u = np.array([orc.uniform(seed, 0, j, 1) for j in range(G)])
        a = r.alpha[0, 0]
        assert np.all(u[:L] < a[:L])
        if L < G:
            assert u[L] >= a[L]
        assert np.allclose(r.accept_margin[0], np.abs(u - a), atol=0)


@pytest.mark.parametrize("case", ["token_high", "token_neg", "nan_p", "inf_q", "allneg_p"])
def test_invalid_inputs_give_minus_one(orc, case):
    rng = np.random.default_rng(12)
    V, G, K = 16, 3, 2
    zp, zq = rows(rng, K, G, V)
    zp = np.ascontiguousarray(np.concatenate([zp, zp], 0))
    zq = np.ascontiguousarray(np.concatenate([zq, zq], 0))
    d = rng.integers(0, V, (2, K, G)).astype(np.int32)
    if case == "token_high":
        d[1, 1, 2] = V
    elif case == "token_neg":
        d[1, 0, 0] = -1
    elif case == "nan_p":
        zp[1, 1, 1, 3] = np.nan
    elif case == "inf_q":
        zq[1, 0, 2, 0] = np.inf
    elif case == "allneg_p":
        zp[1, 0, 0, :] = -np.inf
    r = run(orc, zp, zq, d)
    assert r.selected[1] == -1 and r.accept_len[1] == -1 and r.next_token[1] == -1
    assert r.selected[0] >= 0 and r.accept_len[0] >= 0 and r.next_token[0] >= 0


def test_invalid_bonus_row_only_matters_when_used(orc):
    rng = np.random.default_rng(13)
    V, G = 16, 3
    zp, _ = rows(rng, 1, G, V)
    zq = np.ascontiguousarray(zp[:, :, :G, :])  # alpha == 1: the bonus row is drawn
    zp[0, 0, G, :] = np.nan
    r = run(orc, zp, zq, rng.integers(0, V, (1, 1, G)))
    assert r.accept_len[0] == -1 and r.next_token[0] == -1


def test_forcing_own_decisions_reproduces(orc):
    rng = np.random.default_rng(14)
    zp, zq = rows(rng, 4, 6, 50, sigma=1.2)
    d = rng.integers(0, 50, (1, 4, 6))
    r = run(orc, zp, zq, d, seed=3)
    r2 = run(orc, zp, zq, d, seed=3, force_k=r.selected, force_L=r.accept_len)
    assert (r2.selected == r.selected).all() and (r2.next_token == r.next_token).all()
