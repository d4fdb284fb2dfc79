"""Pins of the oracle's rate-fitted sigma (S-12): the integer code length
against log2, the candidate chosen against a float64 brute force of the
exact code length, and the effect the fit exists for (an RMS inflated by
rare outliers costs bits that the fitted scale saves)."""
import math

import numpy as np
import pytest

import oracle as O
from entropy_coding_amd import workloads as W

W_MIX = (9500, 300)


def test_log2_table_and_code_length():
    tab = O.log2_table_q16()
    exact = 65536.0 * np.log2(1.0 + np.arange(256) / 256.0)
    assert np.all(np.abs(tab - exact) <= 0.5) and np.all(np.diff(tab) > 0)
    # every entry far from a rounding tie: any correctly rounded log2 gives the same table
    assert np.min(np.abs((exact % 1.0) - 0.5)) > 1e-4
    rng = np.random.default_rng(1)
    f = np.concatenate([np.int64(1) << np.arange(32), rng.integers(1, 1 << 31, 20000), [3, 5, 255, 257]])
    got = O.code_len_q16(f).astype(np.float64)
    ideal = 65536.0 * (31.0 - np.log2(f.astype(np.float64)))
    assert np.all(got - ideal >= -0.5) and np.all(got - ideal <= 65536.0 * math.log2(1 + 1 / 256) + 0.5)
    pw = np.int64(1) << np.arange(32)
    assert np.array_equal(O.code_len_q16(pw), (31 - np.arange(32)) * 65536)
    with pytest.raises(ValueError):
        O.code_len_q16(np.array([0]))


def outlier_case(seed=3, reps=2, planes=2, tokens=64, ch=64, frac=0.01, big=30.0):
    """Residual N(0, 0.01^2) with a fraction of 30x outliers: the RMS is
    about 3x the bulk's scale."""
    rng = np.random.default_rng(seed)
    mu = (rng.standard_normal((reps, planes, tokens, ch)) * 0.5).astype(np.float32)
    e = rng.standard_normal(mu.shape) * 0.01
    e = np.where(rng.random(mu.shape) < frac, e * big, e)
    kv = ((mu + e).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mub = (mu.view(np.uint32) >> 16).astype(np.uint16)
    return kv, mub


def test_choice_matches_brute_force_of_the_exact_code_length():
    kv, mu = outlier_case(planes=1, tokens=48)
    pref = O.build_marginal(kv.ravel(), O.BF16, *W_MIX)
    sig, costs = O.calibrate_sigma_rate(kv, mu, O.BF16, O.BF16, 2.0 ** -30, pref, *W_MIX, return_costs=True)
    base = O.calibrate_sigma(kv, mu, O.BF16, O.BF16, 2.0 ** -30)
    reps, planes, t, d = kv.shape
    n = reps * t
    exact = np.zeros((O.RATE_STEPS, planes, d))
    t_n, t_w, _ = O.budgets(O.BF16, *W_MIX)
    s = O.order_index(kv, O.BF16)
    m32 = O.mu_to_f32(mu, O.BF16)
    for j in range(O.RATE_STEPS):
        sj = np.maximum((base * np.float32(1 - j / 32)).astype(np.float32), np.float32(2.0 ** -30))
        inv = np.broadcast_to((np.float32(1) / sj)[:, None, :], (planes, t, d))
        for r in range(reps):
            f = O.cdf(s[r] + 1, m32[r], inv, O.BF16, t_n, t_w, pref) - O.cdf(s[r], m32[r], inv, O.BF16, t_n, t_w, pref)
            exact[j] += (31.0 - np.log2(f.astype(np.float64))).sum(axis=1)
    # the integer cost tracks the exact one within the table's resolution per symbol
    assert np.all(np.abs(costs[:, :, 0, :] / 65536.0 - exact) <= n * 0.0057)
    pick = np.argmin(costs[:, :, 0, :], axis=0)
    chosen = np.take_along_axis(exact, pick[None], 0)[0]
    assert np.all(chosen <= exact.min(axis=0) + n * 0.0114)
    # the result is that candidate
    want = np.maximum((base * (1 - pick / 32).astype(np.float32)).astype(np.float32), np.float32(2.0 ** -30))
    assert np.array_equal(sig, want)


def test_fit_saves_the_bits_an_inflated_rms_costs():
    kv, mu = outlier_case(planes=2, tokens=64)
    pref = O.build_marginal(kv.ravel(), O.BF16, *W_MIX)
    rms = O.calibrate_sigma(kv, mu, O.BF16, O.BF16, 2.0 ** -30)
    fit = O.calibrate_sigma_rate(kv, mu, O.BF16, O.BF16, 2.0 ** -30, pref, *W_MIX)
    assert np.all(fit <= rms) and np.median(fit / rms) < 0.6
    b_rms = O.model_bits_int(kv.reshape(-1, 64, 64), mu.reshape(-1, 64, 64), np.tile(rms, (2, 1)), pref,
                             O.BF16, O.BF16, *W_MIX)
    b_fit = O.model_bits_int(kv.reshape(-1, 64, 64), mu.reshape(-1, 64, 64), np.tile(fit, (2, 1)), pref,
                             O.BF16, O.BF16, *W_MIX)
    assert b_fit < b_rms - 0.5


def test_blocks_and_base_override():
    kv, mu = outlier_case(planes=2, tokens=40)
    pref = O.build_marginal(kv.ravel(), O.BF16, *W_MIX)
    blk = O.calibrate_sigma_rate(kv, mu, O.BF16, O.BF16, 2.0 ** -30, pref, *W_MIX, block_tokens=16)
    assert blk.shape == (2, 3, 64)
    base = O.calibrate_sigma(kv, mu, O.BF16, O.BF16, 2.0 ** -30, block_tokens=16)
    ratio = blk / base
    assert np.all(np.isin(np.round(32 * (1 - ratio)), np.arange(O.RATE_STEPS)))
    # a base given by the caller is used as is: twice the base, twice the result (exact in float32)
    two = O.calibrate_sigma_rate(kv, mu, O.BF16, O.BF16, 2.0 ** -30, pref, *W_MIX, block_tokens=16,
                                 base=base * np.float32(2))
    assert two.shape == blk.shape and np.all(two > 0)
