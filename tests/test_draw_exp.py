"""Constants and steps of the draw's fp64 exp, checked on the CPU.

The draw kernels compute exp((z - m)/T) as 2^(x/256) with x = c z - M (the
argument in 1/256ths of an octave): a shifter add rounds x to n, r = x - n is
exact, a degree-4 Taylor polynomial gives 2^(r/256), a 256-entry table gives
2^((n mod 256)/256) and an ldexp applies n div 256.  These tests read the
table and the coefficients out of the kernel header and hold them to values
computed here with 50-digit decimal arithmetic, then emulate the steps with
exactly rounded fmas and bound the error against 2^x.
"""
import math
import os
import random
import re
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "lossless_draft_verification_verifier_amd", "csrc", "kr_draw.hpp")

getcontext().prec = 50
LN2 = Decimal(2).ln()


def _source():
    with open(HEADER) as f:
        return f.read()


def _table():
    s = _source()
    body = s[s.index("kExp2Frac[256] = {"):]
    body = body[:body.index("};")]
    return [float.fromhex(h) for h in re.findall(r"0x1\.[0-9a-f]+p[+-]0", body)]


def _exp2_function():
    s = _source()
    i = s.index("double exp2_256(")
    return s[i:s.index("\n}\n", i)]


def _coefficients():
    # the four polynomial constants, highest degree first, as they appear in the fmas
    body = _exp2_function()
    return [float.fromhex(h) for h in re.findall(r"0x1\.[0-9a-f]+p-\d+", body)]


def _nearest(d: Decimal) -> float:
    return float(d)  # Decimal -> float rounds correctly


def test_table_entries_are_correctly_rounded():
    tab = _table()
    assert len(tab) == 256
    for j, t in enumerate(tab):
        assert t == _nearest((Decimal(j) / 256 * LN2).exp()), j


def test_polynomial_coefficients_are_correctly_rounded():
    c = _coefficients()
    assert len(c) == 4
    expect = []
    f = Decimal(1)
    for k in range(1, 5):
        f *= k
        expect.append(_nearest((LN2 / 256) ** k / f))
    assert c == expect[::-1]  # degree 4, 3, 2, 1


def test_scale_constant_is_256_log2e():
    s = _source()
    m = re.search(r"kLog2e256 = (0x1\.[0-9a-f]+p\+8)", s)
    assert m
    assert float.fromhex(m.group(1)) == 256.0 * _nearest(1 / LN2)


def _fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _emulate(x, tab, coef):
    """The kernel's steps on x (in 1/256ths of an octave), each fma rounded once."""
    shift = float.fromhex("0x1.8p52")
    x = max(x, -281600.0)
    y = x + shift
    n = y - shift
    ni = struct.unpack("<Q", struct.pack("<d", y))[0] & 0xFFFFFFFF
    if ni >= 1 << 31:
        ni -= 1 << 32
    assert ni == int(n)
    r = x - n
    assert Fraction(r) == Fraction(x) - Fraction(n) and abs(r) <= 0.5  # exact remainder
    c4, c3, c2, c1 = coef
    p = _fma(c4, r, c3)
    p = _fma(p, r, c2)
    p = _fma(p, r, c1)
    p = _fma(p, r, 1.0)
    return math.ldexp(tab[ni & 255] * p, ni >> 8)


def test_emulated_exp_within_two_ulp():
    tab, coef = _table(), _coefficients()
    rng = random.Random(7)
    xs = [-rng.random() * s for s in (1e-6, 1e-3, 0.1, 1.0, 10.0, 60.0, 700.0, 1020.0)
          for _ in range(100)]
    xs += [0.0, -0.0, 2.0 ** -60, -1.0 / 512, -1.0 / 256, -1022.0]
    worst = 0.0
    for x2 in xs:  # x2: the exponent in octaves; the kernel sees 256 x2 (exact)
        got = _emulate(x2 * 256.0, tab, coef)
        want = (Decimal(x2) * LN2).exp()
        ulp = Decimal(math.ulp(float(want)))
        worst = max(worst, float(abs(Decimal(got) - want) / ulp))
    assert worst <= 2.0, worst


@pytest.mark.parametrize("x2", [-1080.0, -1100.0, -1e300, -math.inf])
def test_emulated_exp_underflows_to_zero(x2):
    assert _emulate(x2 * 256.0, _table(), _coefficients()) == 0.0
