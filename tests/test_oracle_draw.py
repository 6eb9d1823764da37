"""Pins of the oracle's replacement and bonus draws.

* The inverse CDF equals numpy.searchsorted(cumsum(r), t, side="right") (a
  library routine) wherever t is below the total.
* With a one-hot drafter q = delta_x the residual max(0, p - q) is p with x
  removed and renormalised, the resampling that SpecDiff-2 appendix B.4
  describes for greedy acceptance; draws must follow it (chi-square).
* A residual without mass (p equal to q) falls back to p.
"""
import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chi2


@pytest.mark.parametrize("V", [1, 2, 5, 17, 64])
def test_inverse_cdf_matches_searchsorted(orc, V):
    rng = np.random.default_rng(V)
    for _ in range(50):
        r = rng.random(V)
        r[rng.random(V) < 0.3] = 0.0
        if r.sum() == 0:
            r[rng.integers(V)] = 1.0
        c = np.cumsum(r)  # sequential running sum, like the oracle's
        for t in np.concatenate([rng.random(20) * c[-1], [0.0]]):
            v, lo, hi = orc.inverse_cdf(r, float(t))
            want = int(np.searchsorted(c, t, side="right"))
            assert v == want
            assert r[v] > 0.0
            assert lo <= t < hi


def test_inverse_cdf_at_the_total_takes_last_massive_token(orc):
    r = np.array([0.2, 0.0, 0.5, 0.3, 0.0, 0.0])
    v, _, _ = orc.inverse_cdf(r, float(np.cumsum(r)[-1]))
    assert v == 3
    v, _, _ = orc.inverse_cdf(r, 10.0)
    assert v == 3


def test_inverse_cdf_never_picks_zero_mass(orc):
    r = np.array([0.0, 0.0, 1e-300, 0.0, 2.0])
    assert orc.inverse_cdf(r, 0.0)[0] == 2
    assert orc.inverse_cdf(r, 1e-300)[0] == 4


def test_residual_weights_and_fallback(orc):
    rng = np.random.default_rng(3)
    p = softmax(rng.standard_normal(40))
    q = softmax(rng.standard_normal(40))
    r, Z = orc.draw_weights(p, q)
    assert np.all(r >= 0) and abs(Z - 0.5 * np.abs(p - q).sum()) < 1e-15
    assert np.all(r[q >= p] == 0)
    r2, Z2 = orc.draw_weights(p, p)
    assert np.array_equal(r2, p) and abs(Z2 - 1) < 1e-15
    r3, Z3 = orc.draw_weights(p, None)
    assert np.array_equal(r3, p)


def test_one_hot_drafter_residual_is_p_without_x(orc):
    rng = np.random.default_rng(21)
    V, n = 12, 200_000
    zp = (rng.standard_normal((1, 1, 2, V)) * 1.5).astype(np.float32)
    x = 4
    zq = np.full((1, 1, 1, V), -np.inf, np.float32)
    zq[0, 0, 0, x] = 0.0
    P = softmax(zp[0, 0, 0].astype(np.float64))
    want = P.copy()
    want[x] = 0.0
    want /= want.sum()
    bp = np.ascontiguousarray(np.broadcast_to(zp, (n, 1, 2, V)))
    bq = np.ascontiguousarray(np.broadcast_to(zq, (n, 1, 1, V)))
    d = np.full((n, 1, 1), x, np.int32)
    # force a rejection at position 0 in every trial: the draw is then residual
    r = orc.select_and_verify(bp, bq, d, seed=11, force_L=np.zeros(n, np.int32))
    tok = r.next_token
    assert np.all(tok != x)
    counts = np.bincount(tok, minlength=V).astype(np.float64)
    exp = want * n
    m = exp > 0
    stat = ((counts[m] - exp[m]) ** 2 / exp[m]).sum()
    assert chi2.sf(stat, m.sum() - 1) > 1e-3
