"""Pins of the oracle's counter-hash uniforms.

* The SplitMix64 output function against the published outputs of the
  generator started from state 0 (tests/golden/splitmix64_seed0.txt).
* The four-fold key composition and the 53-bit uniform against a third,
  independent big-integer implementation (tests/hash_ref.py).
"""
import os
import random

import numpy as np
import pytest

from hash_ref import GOLDEN, M64, key as _py_key

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_golden():
    rows = []
    with open(os.path.join(HERE, "golden", "splitmix64_seed0.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            n, h = line.split()
            rows.append((int(n), int(h, 16)))
    return rows


def test_published_splitmix64_sequence(orc):
    rows = _load_golden()
    assert len(rows) >= 3
    for n, want in rows:
        state = (n * GOLDEN) & M64
        assert orc.splitmix64(state) == want, n


def test_key_composition_matches_bigint(orc):
    rng = random.Random(12345)
    cases = [(0, 0, 0, 1), (1, 0, 0, 1), (1, 5, 2, 2), (M64, 1 << 40, 7, 2),
             (20261202, 123456, 31, 1)]
    cases += [(rng.getrandbits(64), rng.getrandbits(64), rng.randrange(0, 300), rng.randrange(1, 4))
              for _ in range(2000)]
    for c in cases:
        assert orc.key(*c) == _py_key(*c), c


def test_uniform_is_top_53_bits(orc):
    rng = random.Random(7)
    for _ in range(2000):
        c = (rng.getrandbits(64), rng.getrandbits(40), rng.randrange(0, 64), rng.randrange(1, 4))
        u = orc.uniform(*c)
        k = _py_key(*c)
        assert u == (k >> 11) / float(1 << 53)
        assert 0.0 <= u < 1.0


def test_uniforms_look_uniform(orc):
    # 20000 keys over distinct rows: mean and a 20-bin chi-square
    us = np.array([orc.uniform(3, r, 0, 1) for r in range(20000)])
    assert abs(us.mean() - 0.5) < 0.01
    counts, _ = np.histogram(us, bins=20, range=(0, 1))
    exp = len(us) / 20
    chi2 = ((counts - exp) ** 2 / exp).sum()
    from scipy.stats import chi2 as c2
    assert c2.sf(chi2, 19) > 1e-4


@pytest.mark.parametrize("purpose", [1, 2, 3])
def test_purposes_are_distinct_streams(orc, purpose):
    a = [orc.key(9, r, 4, purpose) for r in range(50)]
    b = [orc.key(9, r, 4, purpose % 3 + 1) for r in range(50)]
    assert not set(a) & set(b)
