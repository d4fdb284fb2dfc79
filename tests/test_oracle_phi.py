"""Pins of the integer standard-normal CDF (KVC-1 S-4) against scipy's
ndtr (a different implementation from the mpmath erfc the oracle uses) and
against closed-form properties of Phi."""
import numpy as np
from scipy.special import ndtr

import oracle as O

TWO31 = 2 ** 31


def test_table_matches_scipy_rounding():
    tab = O.phi_table()
    k = np.arange(4097)
    x = -8.0 + k / 256.0
    ref = np.floor(TWO31 * ndtr(x) + 0.5).astype(np.int64)
    assert np.array_equal(tab[:4097], ref)
    assert tab[4097] == tab[4096]


def test_table_has_no_near_ties():
    # double-precision evaluation reproduces every entry only if no value
    # of 2^31 Phi sits close to a half-integer
    x = -8.0 + np.arange(4097) / 256.0
    frac = (TWO31 * ndtr(x)) % 1.0
    assert np.min(np.abs(frac - 0.5)) > 1e-6


def test_table_closed_form_values():
    tab = O.phi_table()
    assert tab[0] == 0                  # Phi(-8) * 2^31 ~ 1.3e-6
    assert tab[2048] == 2 ** 30         # Phi(0) = 1/2
    assert tab[4096] == TWO31           # Phi(8) rounds to 1
    k = np.arange(4097)
    assert np.all(tab[k] + tab[4096 - k] == TWO31)   # Phi(x) + Phi(-x) = 1
    steps = np.diff(tab[:4097])
    assert np.all(steps >= 0) and steps.max() < 2 ** 22


def test_phi_fx_on_grid_and_between():
    tab = O.phi_table()
    k = np.arange(4097)
    q_grid = (k.astype(np.int64) << 16) - (1 << 27)
    assert np.array_equal(O.phi_fx(q_grid), tab[:4097])
    rng = np.random.default_rng(1)
    q = rng.integers(-(1 << 27), (1 << 27) + 1, 200000)
    approx = O.phi_fx(q).astype(np.float64)
    exact = TWO31 * ndtr(q / 2.0 ** 24)
    # linear interpolation at step h = 1/256 errs by at most h^2/8 max|phi'|
    # (= 0.242) times 2^31 (~ 991), plus half a unit from the table rounding
    bound = (1 / 256) ** 2 / 8 * 0.2420 * TWO31 + 1.0
    assert np.max(np.abs(approx - exact)) <= bound


def test_phi_fx_monotone_and_symmetric():
    q = np.arange(-(1 << 27), (1 << 27) + 1, 997, dtype=np.int64)
    p = O.phi_fx(q)
    assert np.all(np.diff(p) >= 0)
    s = O.phi_fx(q) + O.phi_fx(-q)
    assert np.all(np.abs(s - TWO31) <= 1)
