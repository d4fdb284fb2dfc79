"""Statistical pins of the oracle against closed forms the pages state:
the Gaussian cost at the optimum sigma, the cost of a perfect predictor, the
cost of an uninformative predictor, and the size of the escape component."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W


def bf16_bits(x: torch.Tensor):
    return W.to_numpy_bits(x.to(torch.bfloat16))


def gaussian_case(mu, sigma, n, seed):
    g = torch.Generator().manual_seed(seed)
    x = mu + sigma * torch.randn(n, generator=g)
    kv = bf16_bits(x).reshape(1, -1, 64)
    mub = bf16_bits(torch.full((n,), mu)).reshape(1, -1, 64)
    sig = np.full((1, 64), sigma, dtype=np.float32)
    return kv, mub, sig


@pytest.mark.parametrize("log2_sigma", [-6, -5, -4])
def test_single_gaussian_closed_form(log2_sigma, pages):
    """In [1, 2) every BF16 cell is 2^-7 wide; for sigma >> 2^-7 the cost of a
    discretised Gaussian is 1/2 log2(2 pi e sigma^2) - log2(width) bits."""
    sigma = 2.0 ** log2_sigma
    kv, mu, sig = gaussian_case(1.5, sigma, 1 << 17, seed=11 + log2_sigma)
    vals = O.symbol_value(O.order_index(kv, O.BF16), O.BF16)
    assert vals.min() >= 1.0 and vals.max() < 2.0
    closed = 0.5 * math.log2(2 * math.pi * math.e * sigma ** 2) - math.log2(2.0 ** -7)
    # exact entropy of the Gaussian discretised on the cells [v -+ 2^-8]
    from scipy.special import ndtr
    v = 1.0 + np.arange(128) / 128.0
    p = ndtr((v + 2.0 ** -8 - 1.5) / sigma) - ndtr((v - 2.0 ** -8 - 1.5) / sigma)
    p = p[p > 0]
    exact = float(-(p * np.log2(p)).sum())
    got = O.model_bits_int(kv, mu, sig, None, O.BF16, O.BF16, 10000, 0)
    fl = O.model_bits_float(kv, mu, sig, None, O.BF16, O.BF16, 10000, 0)
    se = 1.1 / math.sqrt(kv.size)          # per-scalar cost has sd ~ 1 bit
    assert abs(got - exact) < 4.5 * se
    assert abs(fl - exact) < 4.5 * se
    assert abs(got - fl) < 1e-3
    if sigma >= 2.0 ** -5:                 # cells narrow against sigma
        assert abs(exact - closed) < 0.005


def test_one_bit_per_doubling_of_sigma():
    a = O.model_bits_int(*gaussian_case(1.5, 2.0 ** -5, 1 << 17, 3), None, O.BF16, O.BF16, 10000, 0)
    b = O.model_bits_int(*gaussian_case(1.5, 2.0 ** -4, 1 << 17, 3), None, O.BF16, O.BF16, 10000, 0)
    assert abs((b - a) - 1.0) < 0.01


def test_calibrated_sigma_minimises_gaussian_cost():
    """sigma^2 = mean squared residual is the optimum of spread + miss cost."""
    g = torch.Generator().manual_seed(5)
    mu = torch.randn(1, 1, 2048, 64, generator=g).to(torch.bfloat16)
    kv = (mu.float() + 0.03 * torch.randn(1, 1, 2048, 64, generator=g)).to(torch.bfloat16)
    sig = O.calibrate_sigma(W.to_numpy_bits(kv), W.to_numpy_bits(mu), O.BF16, O.BF16, 2.0 ** -30)[0:1]
    kvn, mun = W.to_numpy_bits(kv)[0], W.to_numpy_bits(mu)[0]
    cost = {f: O.model_bits_float(kvn, mun, sig * np.float32(f), None, O.BF16, O.BF16, 10000, 0)
            for f in (0.8, 1.0, 1.25)}
    assert cost[1.0] < cost[0.8] and cost[1.0] < cost[1.25]


def test_perfect_predictor_costs_almost_nothing(pages):
    """mu = KV and sigma -> 0: the pages' zero-bit limit.  With the +1 floor
    the single Gaussian costs -log2((1+T)/M) per scalar; the mixture spends
    the 2% escape share, -log2(0.98) bits."""
    assert pages["target_as_predictor_bits"]["value"] == 0
    w = W.WORKLOADS[0]
    kv, _ = W.layer_data(w, 0, tokens=64)
    kvn = W.to_numpy_bits(kv)
    sig = np.full((kvn.shape[0], kvn.shape[2]), 2.0 ** -30, dtype=np.float32)
    single = O.model_bits_int(kvn, kvn, sig, None, O.BF16, O.BF16, 10000, 0)
    t = O.M - 65536
    floor_single = -math.log2((1 + t) / O.M)
    assert floor_single <= single < floor_single + 1e-4
    pref = O.build_marginal(W.to_numpy_bits(W.marginal_samples(w)), O.BF16, 9500, 300)
    mix = O.model_bits_int(kvn, kvn, sig, pref, O.BF16, O.BF16, 9500, 300)
    assert -math.log2(0.98 + 1e-3) < mix <= -math.log2(0.98) + 1e-4


def test_uninformative_predictor_costs_about_16_bits(pages):
    """An independent mu with a tiny sigma leaves only the escape part: the
    cost is -log2(w_e p_hat(x) + 1/M), about the 16 raw bits the pages give
    for a noise predictor."""
    w = W.WORKLOADS[0]
    kv, _ = W.layer_data(w, 0, tokens=128)
    kvn = W.to_numpy_bits(kv)
    mu = W.to_numpy_bits(W.noise_predictor(w, tuple(kv.shape)))
    sig = np.full((kvn.shape[0], kvn.shape[2]), 2.0 ** -30, dtype=np.float32)
    samples = W.to_numpy_bits(W.marginal_samples(w))
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    bits = O.model_bits_int(kvn, mu, sig, pref, O.BF16, O.BF16, 9500, 300)
    # closed form from the histogram itself
    counts = np.bincount(O.order_index(samples, O.BF16), minlength=65536) + 1
    p = counts[O.order_index(kvn, O.BF16)] / counts.sum()
    t_e = O.budgets(O.BF16, 9500, 300)[2]
    expect = float(np.mean(-np.log2((1 + t_e * p) / O.M)))
    assert abs(bits - expect) < 0.02
    assert abs(bits - pages["noise_predictor_bits"]["value"]) < 1.5


def test_escape_component_is_about_11_bits(pages):
    w = W.WORKLOADS[0]
    idx = O.order_index(W.to_numpy_bits(W.marginal_samples(w)), O.BF16)
    c = np.bincount(idx, minlength=65536)
    p = c[c > 0] / c.sum()
    h = float(-(p * np.log2(p)).sum())
    assert abs(h - pages["escape_component_bits"]["value"]) < 1.0


def test_wide_part_alone_is_a_gaussian_of_three_sigma():
    """Weights (0, 10000) leave only the N(mu, (3 sigma)^2) part: the float
    model must equal the single Gaussian at scale 3 sigma (3 sigma is exact
    in float32 here), and both the discretised entropy of that Gaussian and
    1/2 log2(2 pi e (3 sigma)^2) - log2(width) for cells narrow against it."""
    sigma = 2.0 ** -6                      # 3 sigma = 0.046875 exactly
    kv, mu, _ = gaussian_case(1.5, 3 * sigma, 1 << 17, seed=23)
    sig1 = np.full((1, 64), sigma, dtype=np.float32)
    sig3 = np.full((1, 64), 3 * sigma, dtype=np.float32)
    wide = O.model_bits_float(kv, mu, sig1, None, O.BF16, O.BF16, 0, 10000)
    single = O.model_bits_float(kv, mu, sig3, None, O.BF16, O.BF16, 10000, 0)
    assert wide == single
    from scipy.special import ndtr
    v = 1.0 + np.arange(128) / 128.0
    p = ndtr((v + 2.0 ** -8 - 1.5) / (3 * sigma)) - ndtr((v - 2.0 ** -8 - 1.5) / (3 * sigma))
    p = p[p > 0]
    exact = float(-(p * np.log2(p)).sum())
    closed = 0.5 * math.log2(2 * math.pi * math.e * (3 * sigma) ** 2) - math.log2(2.0 ** -7)
    se = 1.1 / math.sqrt(kv.size)
    assert abs(wide - exact) < 4.5 * se
    assert abs(exact - closed) < 0.005
    # the integer model of the same weights agrees with the float model
    assert abs(O.model_bits_int(kv, mu, sig1, None, O.BF16, O.BF16, 0, 10000) - wide) < 1e-3


def test_escape_part_alone_is_the_smoothed_histogram():
    """Weights (0, 0) leave only the escape part: every scalar costs
    -log2 p_hat(x).  Against the +1-smoothed histogram counted here pattern
    by pattern, p(x) = (1 + #{samples equal to x}) / (N + #samples), the
    integer prefix differs by at most one budget unit per symbol, so the mean
    cost differs by at most log2(1 + (N + #samples) / T_e)."""
    kv, mu, sig, samples = W.tiny_case(31, planes=2, tokens=40, channels=128)
    kvn, mun, sgn, smn = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(smn, O.BF16, 0, 0)
    got = O.model_bits_float(kvn, mun, sgn, pref, O.BF16, O.BF16, 0, 0)
    counts = {}
    for u in smn.ravel().tolist():
        counts[u] = counts.get(u, 0) + 1
    tot = 65536 + smn.size
    bits = [-math.log2((1 + counts.get(u, 0)) / tot) for u in kvn.ravel().tolist()]
    want = sum(bits) / len(bits)
    t_e = O.budgets(O.BF16, 0, 0)[2]
    assert t_e == O.M - 65536
    assert abs(got - want) <= math.log2(1 + tot / t_e)
    # the integer model codes (1 + dP) / M where the float model has dP / T_e
    # (dP >= T_e / tot - 1 units): the two differ by less than that bound too
    gi = O.model_bits_int(kvn, mun, sgn, pref, O.BF16, O.BF16, 0, 0)
    assert abs(got - gi) <= math.log2(1 + tot / t_e)
