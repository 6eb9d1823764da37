"""Pins of the oracle's adaptive draft length (DiffuSpec section 4.3: the
controller adjusts the next draft length from the EOS-aware generated length
and the accepted length, growing it while acceptance keeps pace with
generation on average and holding it once the generated length saturates;
section 6: it avoids over- and under-drafting).

* closed loop with every drafted token accepted: the window grows by `step`
  per call until k_max, and stays there;
* closed loop with the draft ending at EOS inside the window: the window
  holds, whatever is accepted;
* closed loop with a constant accepted streak c (L = min(c, window)): the
  window settles at c + 1, the streak plus the position that is rejected, from
  above and from below;
* the recent lengths are averages rounded down: under a constant input they
  reach 256 * L exactly from above and stop less than 2^shift below it from
  below;
* a longer accepted length never gives a shorter window; outputs stay in
  [k_min, k_max]; invalid prefixes keep their state; each prefix is
  independent of the others.
"""
import numpy as np
import pytest


def _loop(orc, n0, accepted, steps, eos_at=None, G=64, **kw):
    """Drive one prefix for `steps` calls: accepted(n) gives this step's L for
    a window of n; eos_at: the draft's EOS position (None: no EOS)."""
    n, st = n0, np.array([[256 * n0, 256 * n0]], np.int32)
    windows = [n]
    for _ in range(steps):
        d = np.full((1, 1, G), 7, np.int32)
        eos = -1
        if eos_at is not None:
            eos = 99
            if eos_at < n:
                d[0, 0, eos_at] = eos
        g = n if eos_at is None or eos_at >= n else eos_at + 1
        L = min(accepted(n), g)
        nxt, st = orc.adl_next(d, [0], [L], st, gamma_b=[n], eos=eos, **kw)
        n = int(nxt[0])
        windows.append(n)
    return windows, st


def test_expands_while_acceptance_keeps_pace(orc):
    for slack in (0, 64):
        w, _ = _loop(orc, 4, lambda n: n, 30, k_min=1, k_max=40, step=4, shift=2, slack=slack)
        assert w[:10] == [4, 8, 12, 16, 20, 24, 28, 32, 36, 40]
        assert all(x == 40 for x in w[9:])


def test_holds_once_generated_length_saturates(orc):
    # the drafter ends at EOS at position 5: with every token accepted the
    # window grows until it first holds the EOS, then stops growing
    w, _ = _loop(orc, 4, lambda n: n, 20, eos_at=5, k_min=1, k_max=60, step=4, shift=2, slack=64)
    assert w[0] == 4 and all(x == 8 for x in w[1:]), w
    # a window that already holds the EOS is kept, whatever is accepted
    for acc in (lambda n: n, lambda n: 2, lambda n: 0):
        w, _ = _loop(orc, 12, acc, 20, eos_at=5, k_min=1, k_max=60, step=4, shift=2, slack=64)
        assert all(x == 12 for x in w), w


def test_generated_length_is_the_eos_aware_one(orc):
    # ten steps in which the draft ends at EOS at position 5 and all of it is
    # accepted (accepted and generated lengths match), then drafts without EOS,
    # fully accepted: the averages still match, so the window grows at once
    n, st = 12, np.array([[256 * 12, 256 * 12]], np.int32)
    kw = dict(k_min=1, k_max=40, step=4, shift=2, slack=64)
    d = np.full((1, 1, 64), 7, np.int32)
    d[0, 0, 5] = 99
    for _ in range(10):
        nxt, st = orc.adl_next(d, [0], [6], st, gamma_b=[n], eos=99, **kw)
        assert nxt[0] == n
    d[0, 0, 5] = 7
    nxt, st = orc.adl_next(d, [0], [n], st, gamma_b=[n], eos=99, **kw)
    assert nxt[0] == n + 4


@pytest.mark.parametrize("c", [0, 1, 3, 7])
@pytest.mark.parametrize("n0", [2, 40])
def test_settles_at_the_streak_plus_one(orc, c, n0):
    w, st = _loop(orc, n0, lambda n: c, 200, k_min=1, k_max=48, step=4, shift=2, slack=64)
    assert all(x == c + 1 for x in w[-20:]), w[-30:]


def test_recent_lengths_are_averages_rounded_down(orc):
    for shift in (0, 1, 3, 6):
        # from above: exactly 256 * L in the end
        _, st = _loop(orc, 40, lambda n: 5, 400, k_min=40, k_max=40, step=0, shift=shift)
        assert st[0, 0] == 256 * 5
        # from below: stops within 2^shift below 256 * L, never above
        n, st = 8, np.array([[0, 0]], np.int32)
        d = np.full((1, 1, 8), 7, np.int32)
        trace = []
        for _ in range(400):
            _, st = orc.adl_next(d, [0], [8], st, gamma_b=[8], k_min=8, k_max=8, step=0,
                                 shift=shift)
            trace.append(int(st[0, 0]))
        assert all(b >= a for a, b in zip(trace, trace[1:]))
        assert 0 <= 256 * 8 - trace[-1] < (1 << shift)
        assert st[0, 1] == trace[-1]  # the generated length follows the same average


def test_longer_acceptance_never_gives_a_shorter_window(orc):
    rng = np.random.default_rng(5)
    for _ in range(300):
        G = 32
        n = int(rng.integers(1, G + 1))
        st = rng.integers(0, 256 * G, size=(1, 2)).astype(np.int32)
        d = rng.integers(0, 50, size=(1, 1, G)).astype(np.int32)
        eos = int(rng.integers(-1, 50))
        kw = dict(gamma_b=[n], eos=eos, k_min=int(rng.integers(1, 4)), k_max=G, step=3,
                  shift=int(rng.integers(0, 5)), slack=int(rng.integers(0, 300)))
        prev = None
        for L in range(0, n + 1):
            nxt, _ = orc.adl_next(d, [0], [L], st, **kw)
            if prev is not None:
                assert nxt[0] >= prev
            prev = nxt[0]


def test_bounds_invalid_prefixes_and_independence(orc):
    rng = np.random.default_rng(9)
    B, K, G = 400, 3, 24
    d = rng.integers(0, 30, size=(B, K, G)).astype(np.int32)
    gb = rng.integers(-1, G + 3, size=B).astype(np.int32)
    sel = rng.integers(-1, K, size=B).astype(np.int32)
    L = np.array([rng.integers(-1, max(int(n), 0) + 2) for n in gb], np.int32)
    st = rng.integers(-50, 256 * G + 50, size=(B, 2)).astype(np.int32)
    st[::7] = (1 << 20) + 1  # a state out of range
    kw = dict(gamma_b=gb, eos=5, k_min=2, k_max=20, step=5, shift=3, slack=32)
    nxt, st2 = orc.adl_next(d, sel, L, st, **kw)
    for b in range(B):
        n = gb[b]
        bad_n = not 1 <= n <= G
        bad_in = sel[b] < 0 or L[b] < 0 or L[b] > n
        bad_st = not (0 <= st[b, 0] <= 1 << 20 and 0 <= st[b, 1] <= 1 << 20)
        if bad_n:
            assert nxt[b] == -1 and np.array_equal(st2[b], st[b])
        elif bad_in:
            assert nxt[b] == n and np.array_equal(st2[b], st[b])
        elif bad_st:
            assert nxt[b] == -1 and np.array_equal(st2[b], st[b])
        else:
            assert 2 <= nxt[b] <= 20
        # one prefix alone gives the same
        one, st1 = orc.adl_next(d[b:b + 1], sel[b:b + 1], L[b:b + 1], st[b:b + 1],
                                gamma_b=gb[b:b + 1], eos=5, k_min=2, k_max=20, step=5, shift=3,
                                slack=32)
        assert one[0] == nxt[b] and np.array_equal(st1[0], st2[b])


def test_parameters_out_of_range_are_rejected(orc):
    d = np.zeros((1, 1, 4), np.int32)
    for kw in (dict(k_min=0), dict(k_min=5, k_max=4), dict(k_max=4097), dict(step=-1),
               dict(shift=17), dict(slack=-1)):
        with pytest.raises(ValueError):
            orc.adl_next(d, [0], [1], [[0, 0]], **kw)
