"""A float32 model of the encoder's division routine (floor(x / f) and
x mod f for x < 2^32 f without a hardware divider): a float estimate of the
quotient, one float correction from the remainder, and one integer
adjustment.  The model runs the same steps with NumPy float32 and checks
them against exact integer division at the extremes of f and x, with the
reciprocal perturbed by up to two ulps (the hardware reciprocal is not
correctly rounded)."""
import numpy as np
import pytest

f32 = np.float32


def divmod_model(x: int, f: int, ulps: int):
    rf = f32(1.0) / f32(f)
    for _ in range(abs(ulps)):
        rf = np.nextafter(rf, f32(np.inf if ulps > 0 else -np.inf))
    xh, xl = x >> 32, x & 0xFFFFFFFF
    fx = f32(float(f32(xh)) * 4294967296.0 + float(f32(xl)))          # one fma rounding
    q0 = int(min(max(f32(fx * rf), f32(0.0)), f32(4294967040.0)))
    r0 = x - q0 * f
    assert abs(r0) < 2 ** 42
    hi, lo = r0 >> 21, r0 & 0x1FFFFF                                    # both exact in float32
    fr0 = f32(float(f32(hi)) * 2097152.0 + float(f32(lo)))
    q1 = min(q0 + int(np.floor(f32(fr0 * rf))), 0xFFFFFFFF)
    r1 = x - q1 * f
    assert -f <= r1 < 2 * f
    if r1 < 0:
        q1, r1 = q1 - 1, r1 + f
    if r1 >= f:
        q1, r1 = q1 + 1, r1 - f
    return q1, r1


@pytest.mark.parametrize("ulps", [-2, 0, 2])
def test_division_model_is_exact(ulps):
    rng = np.random.default_rng(3 + ulps)
    fs = [1, 2, 3, 5, 40, 255, 256, 257, 65535, 65536, 2 ** 24 - 1, 2 ** 24 + 1, 2 ** 31 - 65535,
          2 ** 31 - 1] + [int(v) for v in rng.integers(1, 2 ** 31, 24)]
    for f in fs:
        lo, hi = 2 ** 16 * f, min(2 ** 32 * f, 2 ** 63)        # the coder's range of x
        xs = [lo, lo + 1, hi - 1, hi - 2] + [int(v) for v in rng.integers(lo, hi, 300, dtype=np.uint64)]
        for x in xs:
            assert divmod_model(x, f, ulps) == divmod(x, f), (x, f)


def divmod_f64_model(x: int, f: int, rcp_rel_err: float):
    """The fp64 variant: x as a double (one rounding), a hardware reciprocal
    with relative error up to `rcp_rel_err`, one Newton step, a truncated
    quotient within one of the truth, and a two-sided integer fix."""
    xh, xl = x >> 32, x & 0xFFFFFFFF
    xd = float(xh) * 4294967296.0 + float(xl)              # fma: exact product, one rounding
    fd = float(f)
    r = (1.0 / fd) * (1.0 + rcp_rel_err)
    e = 1.0 - fd * r                                         # fma
    r = r + r * e                                            # fma
    q = int(xd * r)                                          # truncation of a positive value
    q = min(q, 0xFFFFFFFF)
    rem = x - q * f
    assert -f <= rem < 2 * f
    if rem < 0:
        q, rem = q - 1, rem + f
    elif rem >= f:
        q, rem = q + 1, rem - f
    return q, rem


@pytest.mark.parametrize("err", [-2.0 ** -20, 0.0, 2.0 ** -20])
def test_division_f64_model_is_exact(err):
    rng = np.random.default_rng(11)
    fs = [1, 2, 3, 40, 255, 256, 65535, 65536, 2 ** 24 + 1, 2 ** 31 - 65535, 2 ** 31 - 1] + \
         [int(v) for v in rng.integers(1, 2 ** 31, 24)]
    for f in fs:
        lo, hi = 2 ** 16 * f, min(2 ** 32 * f, 2 ** 63)
        xs = [lo, lo + 1, hi - 1, hi - 2] + [int(v) for v in rng.integers(lo, hi, 300, dtype=np.uint64)]
        xs += [q * f for q in (2 ** 16, 2 ** 31, 2 ** 32 - 1) if lo <= q * f < hi]
        xs += [q * f - 1 for q in (2 ** 16 + 1, 2 ** 31, 2 ** 32 - 1) if lo <= q * f - 1 < hi]
        for x in xs:
            assert divmod_f64_model(x, f, err) == divmod(x, f), (x, f)
