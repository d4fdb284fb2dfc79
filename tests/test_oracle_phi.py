"""Pins of the integer mixture table (KVC-1 S-4) against scipy's ndtr (a
different implementation from the mpmath erfc the oracle uses) and against
closed-form properties of Phi."""
import numpy as np
import pytest
from scipy.special import ndtr

import oracle as O

TWO31 = 2 ** 31
Z = -24.0 + np.arange(12289) / 256.0


def test_base_tables_match_scipy_rounding():
    a, b = O.phi_tables()
    assert np.array_equal(a, np.floor(TWO31 * ndtr(Z) + 0.5).astype(np.int64))
    assert np.array_equal(b, np.floor(TWO31 * ndtr(Z / 3.0) + 0.5).astype(np.int64))


def test_base_tables_have_no_near_ties():
    # double-precision evaluation reproduces every entry only if no value
    # of 2^31 Phi sits close to a half-integer
    for x in (Z, Z / 3.0):
        frac = (TWO31 * ndtr(x)) % 1.0
        assert np.min(np.abs(frac - 0.5)) > 1e-6


def test_base_table_closed_forms():
    a, b = O.phi_tables()
    k = np.arange(12289)
    for t in (a, b):
        assert t[0] == 0 and t[6144] == 2 ** 30 and t[12288] == TWO31     # Phi(0) = 1/2
        assert np.all(t[k] + t[12288 - k] == TWO31)                      # Phi(x) + Phi(-x) = 1
        steps = np.diff(t)
        assert np.all(steps >= 0) and steps.max() < 2 ** 22
    # the narrow table saturates beyond |z| = 8 (Phi(-8) 2^31 ~ 1.3e-6)
    assert np.all(a[: 16 * 256 - 1] == 0) and np.all(a[32 * 256 + 1:] == TWO31)
    # the wide part is Phi(z/3): at z = 3x it equals the narrow part at x
    j = np.arange(0, 4097)
    assert np.array_equal(b[3 * j], a[4096 + j])


@pytest.mark.parametrize("w", [(9500, 300), (10000, 0), (7000, 2000), (0, 10000)])
def test_mixture_table(w, pages):
    for dtype in (O.BF16, O.E4M3):
        t_n, t_w, t_e = O.budgets(dtype, *w)
        h = O.mixture_table(t_n, t_w)
        assert h.size == 12290 and h[12289] == h[12288]
        assert h[0] == 0 and h[12288] == t_n + t_w
        assert np.all(np.diff(h) >= 0) and np.diff(h).max() < 2 ** 22
        cont = t_n * ndtr(Z) + t_w * ndtr(Z / 3.0)
        # two floors (< 1 each) and two table roundings (<= 1/2 each)
        assert np.max(np.abs(h[:12289] - cont)) <= 3.0


def test_pages_weights_give_the_budgets(pages):
    wts = pages["mixture_weights"]["value"]
    t_n, t_w, t_e = O.budgets(O.BF16, 9500, 300)
    t = O.M - 65536
    assert abs(t_n - t * wts["narrow"]) < 1 and abs(t_w - t * wts["wide"]) < 1
    assert abs(t_e - t * wts["escape"]) < 2


def test_h_fx_on_grid_and_between():
    t_n, t_w, _ = O.budgets(O.BF16, 9500, 300)
    h = O.mixture_table(t_n, t_w)
    q_grid = (np.arange(12289, dtype=np.int64) << 16) - (24 << 24)
    assert np.array_equal(O.h_fx(q_grid, h), h[:12289])
    rng = np.random.default_rng(1)
    q = rng.integers(-(24 << 24), (24 << 24) + 1, 300000)
    approx = O.h_fx(q, h).astype(np.float64)
    z = q / 2.0 ** 24
    exact = t_n * ndtr(z) + t_w * ndtr(z / 3.0)
    # linear interpolation at step 1/256 errs by at most h^2/8 max|H''|
    # (max |phi'| = 0.242, the wide part adds 1/27 of its weight) plus the
    # table's own rounding
    bound = (1 / 256) ** 2 / 8 * 0.2420 * (t_n + t_w / 27.0) + 3.0
    assert np.max(np.abs(approx - exact)) <= bound


def test_h_fx_monotone_and_symmetric():
    t_n, t_w, _ = O.budgets(O.BF16, 9500, 300)
    h = O.mixture_table(t_n, t_w)
    q = np.arange(-(24 << 24), (24 << 24) + 1, 4999, dtype=np.int64)
    p = O.h_fx(q, h)
    assert np.all(np.diff(p) >= 0)
    s = O.h_fx(q, h) + O.h_fx(-q, h)
    assert np.all(np.abs(s - (t_n + t_w)) <= 3)
