"""The fp8 cache write stores the scale RN(m / 448) of a row maximum m (a
bf16 value) without a division: q = RN(m r), e = RN(m - 448 q),
RN(q + e r) with r = RN(1 / 448), each step one float32 rounding (the last
two fused multiply-adds).  This checks that identity for every positive
finite bf16 m with exact rational arithmetic, so the kernel's stored scale
is the correctly rounded quotient the write rule names (ATOM model
operations guide, "KV cache operations": per-token fp8 quantisation)."""
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
