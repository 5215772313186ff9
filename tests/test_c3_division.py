"""The C3 kernels' Lloyd means: the exact member sum over the count,
correctly rounded in fp64.  The oracle divides; the kernels take the
correctly rounded reciprocal y = 1/n once per count and, per column,
q = x*y, r = fma(-q, n, x), q' = fma(r, y, q) (a Newton correction with the
exact remainder, Markstein's theorem).  This checks on the CPU that q'
equals the IEEE quotient x/n over the values the method produces: sums of
keys on the 2^-24 grid below 2^29 in magnitude, counts up to 2^17.  The
fused multiply-add is emulated exactly (one rounding of the exact rational
result)."""
import random
from fractions import Fraction


def fma(a: float, b: float, c: float) -> float:
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def corrected_quotient(x: float, n: float) -> float:
    y = 1.0 / n
    q = x * y
    r = fma(-q, n, x)
    return fma(r, y, q)


def _cases(rng, counts, per):
    for n in counts:
        for t in range(per):
            bits = rng.randint(1, 53)
            k = rng.getrandbits(bits)
            if t % 3 == 0:                       # next to a multiple of n
                k = (k // n) * n + rng.randint(-1, 1)
            if rng.random() < 0.5:
                k = -k
            yield float(k) * 2.0 ** -24, float(n)


def test_corrected_quotient_is_the_ieee_quotient_for_local_counts():
    rng = random.Random(7)
    for x, n in _cases(rng, range(1, 97), 60):
        assert corrected_quotient(x, n) == x / n, (x, n)


def test_corrected_quotient_is_the_ieee_quotient_for_large_counts():
    rng = random.Random(11)
    counts = [97, 127, 128, 129, 1000, 4095, 4097, 65535, 65536, 131071, 131072]
    counts += [rng.randint(97, 1 << 17) for _ in range(40)]
    for x, n in _cases(rng, counts, 60):
        assert corrected_quotient(x, n) == x / n, (x, n)


def test_corrected_quotient_exact_and_extreme_values():
    for n in (1, 2, 3, 7, 96, 131072):
        for x in (0.0, 2.0 ** -24, -(2.0 ** -24), 2.0 ** 29 - 2.0 ** -24, float(n) * 3.0):
            assert corrected_quotient(x, float(n)) == x / n, (x, n)
