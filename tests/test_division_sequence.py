"""The division by a bias correction that the one- and two-element fused
steps and short AdamW launches use, checked with exact rational arithmetic
on the CPU.

For b = 1 - beta^t and the host's two-part reciprocal hi = RN(1/b),
lo = RN((1 - b hi) / b), the device computes
    q0 = fma(a, hi, a*lo);  r = fma(-b, q0, a);  q = fma(r, hi, q0)
and the claim is q = RN(a / b) (Markstein's theorem once q0 is faithful).
Here every fused multiply-add is evaluated exactly with fractions and
rounded once, as the hardware does, and q is compared with the correctly
rounded quotient on divisors from many betas and steps and on dividends
chosen to be hard: significands next to 1 and 2, widened fp32 values, and
dividends whose quotient lies next to a rounding midpoint.
"""

import random
import struct
from fractions import Fraction as Fr


def fma(x, y, z):
    return float(Fr(x) * Fr(y) + Fr(z))


def reciprocal_parts(b):
    hi = 1.0 / b
    e = fma(-b, hi, 1.0)
    assert Fr(e) == 1 - Fr(b) * Fr(hi), "1 - b*hi must be exact in one fma"
    return hi, e / b


def bias_division(a, b, hi, lo):
    q0 = fma(a, hi, a * lo)
    r = fma(-b, q0, a)
    return fma(r, hi, q0)


def divisors(rng):
    bs = set()
    for beta in (0.9, 0.95, 0.99, 0.5, 0.999, 0.98, 0.9999, 0.987654321):
        for t in list(range(1, 60)) + [rng.randrange(60, 10**6) for _ in range(10)]:
            bs.add(1.0 - beta ** t)
    for _ in range(40):
        bs.add(((rng.getrandbits(52) | (1 << 52)) * 2.0 ** -52) * 2.0 ** -rng.randrange(1, 53))
    bs.update((1.0, 0.5, 2.0 ** -53, 1.0 - 2.0 ** -53))
    return sorted(b for b in bs if 0 < b <= 1)


def dividend(rng, b):
    k = rng.randrange(5)
    if k == 0:   # an fp32 value, widened
        while True:
            x = struct.unpack("<f", struct.pack("<I", rng.getrandbits(32)))[0]
            if x == x and abs(x) != float("inf") and x != 0:
                return x
    if k == 1:   # significand next to 2
        return ((1 << 53) - 1 - rng.randrange(32)) * 2.0 ** (rng.randrange(-300, 200) - 52)
    if k == 2:   # significand next to 1
        return ((1 << 52) + rng.randrange(32)) * 2.0 ** (rng.randrange(-300, 200) - 52)
    if k == 3:   # quotient next to a midpoint between two doubles
        q = (rng.getrandbits(52) | (1 << 52)) * 2.0 ** (rng.randrange(-200, 100) - 52)
        return float((Fr(q) + Fr(q) * Fr(1, 2 ** 53)) * Fr(b))
    return (rng.getrandbits(53) | (1 << 52)) * 2.0 ** (rng.randrange(-400, 250) - 52)


def test_bias_division_is_correctly_rounded():
    rng = random.Random(20261203)
    bad, n = [], 0
    for b in divisors(rng):
        hi, lo = reciprocal_parts(b)
        for _ in range(40):
            a = dividend(rng, b) * rng.choice((1.0, -1.0))
            want = float(Fr(a) / Fr(b))
            got = bias_division(a, b, hi, lo)
            n += 1
            if got != want:
                bad.append((a.hex(), b.hex(), got.hex(), want.hex()))
    assert n > 20000
    assert not bad, bad[:5]


def test_a_planted_error_is_caught():
    """Without the correction step (q = q0 alone) the same cases find
    quotients that are not correctly rounded: the check can fail."""
    rng = random.Random(7)
    wrong = 0
    for b in divisors(rng)[:200]:
        hi, lo = reciprocal_parts(b)
        for _ in range(20):
            a = dividend(rng, b)
            wrong += float(Fr(a) / Fr(b)) != fma(a, hi, 0.0)
    assert wrong > 0
