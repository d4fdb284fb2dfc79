"""A model of the encoder's division routine (floor(x / f) and x mod f for
x < 2^32 f without a hardware divider), run on the CPU with exact rationals
so that every fused multiply-add rounds once, as on the GPU: x as a double,
a hardware reciprocal of f with a relative error up to `rcp_rel_err`, one
Newton step, the quotient estimate plus one half converted with truncation
and saturation at 2^32 - 1 (so it is the true quotient or one above it),
then the remainder from the low 32 bits of x - q f read as signed, and a
one-sided fix.  Checked against exact integer division at the extremes of f
and x, with the reciprocal perturbed far beyond what the hardware's error
can be."""
from fractions import Fraction

import numpy as np
import pytest


def fma(a: float, b: float, c: float) -> float:
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def divmod_model(x: int, f: int, rcp_rel_err: float):
    xh, xl = x >> 32, x & 0xFFFFFFFF
    xd = fma(float(xh), 4294967296.0, float(xl))
    fd = float(f)
    r = (1.0 / fd) * (1.0 + rcp_rel_err)
    r = fma(r, fma(-fd, r, 1.0), r)
    est = fma(xd, r, 0.5)
    q = min(int(est), 2 ** 32 - 1)                 # truncation, saturating at 2^32 - 1
    exact = x - q * f
    assert -f <= exact < f                         # q is the quotient or one above it
    low = (x - q * f) & 0xFFFFFFFF                 # the low 32 bits of x - q f, as unsigned ...
    rem = low - 2 ** 32 if low >> 31 else low      # ... read as signed
    assert rem == exact                            # |x - q f| < 2^31: the low word is the value
    neg = 0xFFFFFFFF if rem < 0 else 0
    q = (q + neg) & 0xFFFFFFFF
    rem = (rem + (neg & f)) & 0xFFFFFFFF
    return q, rem


@pytest.mark.parametrize("err", [-2.0 ** -20, 0.0, 2.0 ** -20])
def test_division_model_is_exact(err):
    rng = np.random.default_rng(11)
    fs = [1, 2, 3, 40, 255, 256, 65535, 65536, 2 ** 24 + 1, 2 ** 31 - 65535, 2 ** 31 - 1] + \
         [int(v) for v in rng.integers(1, 2 ** 31, 24)]
    for f in fs:
        lo, hi = 2 ** 16 * f, min(2 ** 32 * f, 2 ** 63)        # the coder's range of x
        xs = [lo, lo + 1, hi - 1, hi - 2] + [int(v) for v in rng.integers(lo, hi, 200, dtype=np.uint64)]
        # exact multiples and one below them, where a quotient changes
        xs += [q * f for q in (2 ** 16, 2 ** 31, 2 ** 32 - 1) if lo <= q * f < hi]
        xs += [q * f - 1 for q in (2 ** 16 + 1, 2 ** 31, 2 ** 32 - 1) if lo <= q * f - 1 < hi]
        for x in xs:
            assert divmod_model(x, f, err) == divmod(x, f), (x, f)
