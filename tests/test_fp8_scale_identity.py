"""The division-free arithmetic of the fp8 cache write, checked with exact
rational arithmetic (ATOM model operations guide, "KV cache operations":
per-token fp8 quantisation; the write rule is codes of x / s with the
stored scale s = absmax / 448, both correctly rounded float32).

The kernel stores the scale RN(m / 448) of a row maximum m (a bf16 value)
as q = RN(m r), e = RN(m - 448 q), RN(q + e r) with r = RN(1 / 448), and
forms each quotient x / s the same way with r = RN(1 / s); each step is
one float32 rounding (the last two fused multiply-adds).  Both must equal
the correctly rounded quotients."""
from fractions import Fraction

import numpy as np

F32 = np.float32


def _rn32(x: Fraction) -> Fraction:
    """Round a rational to the nearest float32, ties to even (subnormals
    included)."""
    f = F32(float(x))
    best = None
    for c in (f, np.nextafter(f, F32(np.inf)), np.nextafter(f, F32(-np.inf))):
        d = abs(Fraction(float(c)) - x)
        even = (int(np.array(c, dtype=F32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return Fraction(float(best[1]))


def test_rn32_rounds_ties_to_even():
    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    assert _rn32(one + ulp / 2) == one                       # tie, 1 is even
    assert _rn32(one + ulp + ulp / 2) == one + 2 * ulp       # tie, 1 + 2 ulp is even
    assert _rn32(one + ulp / 2 + Fraction(1, 2 ** 60)) == one + ulp


def test_scale_of_every_positive_bf16_maximum_is_the_rounded_quotient():
    r = _rn32(Fraction(1, 448))
    bad = []
    for bits in range(1, 0x7F80):          # positive finite bf16, subnormals included
        m = Fraction(float(np.array(bits << 16, dtype=np.uint32).view(F32)))
        q = _rn32(m * r)
        e = _rn32(m - 448 * q)
        s = _rn32(q + e * r)
        if s != _rn32(m / 448):
            bad.append(bits)
    assert not bad, f"{len(bad)} maxima, first bf16 bits {bad[:4]}"


def test_corrected_quotient_is_the_rounded_quotient_for_every_mantissa_pair():
    """Each code is the e4m3fn encoding of x / s for the stored scale s; the
    kernel forms the quotient as q = RN(x r), e = RN(x - s q),
    RN(q + e r) with r = RN(1 / s).  For every pair of bf16 mantissas of the
    row maximum a (which sets s = RN(a / 448)) and of the element x, at
    every magnitude ratio 2^-20 .. 1 of x to a, that equals RN(x / s)."""
    mantissas = [Fraction(128 + i, 128) for i in range(128)]
    bad = 0
    for am in mantissas:
        s = _rn32(am / 448)
        r = _rn32(1 / s)
        for k in range(0, 21):
            for xm in mantissas:
                x = min(xm / 2 ** k, am)
                q = _rn32(x * r)
                e = _rn32(x - s * q)
                if _rn32(q + e * r) != _rn32(x / s):
                    bad += 1
    assert bad == 0
