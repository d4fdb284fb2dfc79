"""Pins of the mixture CDF (KVC-1 S-3, S-5): exact invariants on whole
alphabets, and closeness to the continuous mixture of the pages, with the
weights read from the pages' figures, within an error bound derived from
the fixed-point steps."""
import numpy as np
import pytest
from scipy.special import ndtr

import oracle as O

ADVERSARIAL = [
    # (mu, sigma)
    (0.0, 1e-3), (-0.0, 2.0 ** -30), (1e-40, 2.0 ** -30), (-1e-40, 2.0 ** -96),
    (3.0e38, 1.0), (-3.0e38, 2.0 ** 96), (1.5, 2.0 ** -4), (-2.75, 0.37),
    (0.001, 10.0), (1e4, 2.0 ** -7), (np.nan, 0.5), (np.inf, 0.5),
    (0.998046875, 2.0 ** -12), (448.0, 2.0), (-448.0, 0.01), (0.0, 1e4),
]


def marginal(dtype, seed=0, n=50000):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n).astype(np.float32)
    import torch
    if dtype == O.BF16:
        bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        bits = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return O.build_marginal(bits, dtype, 9500, 300)


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
@pytest.mark.parametrize("mode", ["single", "mixture"])
def test_whole_alphabet_invariants(dtype, mode):
    w = (10000, 0) if mode == "single" else (9500, 300)
    pref = marginal(dtype) if mode == "mixture" else None
    mus = np.array([m for m, _ in ADVERSARIAL], dtype=np.float32)
    sig = np.array([s for _, s in ADVERSARIAL], dtype=np.float32)
    tab = O.cdf_table(mus, sig, dtype, O.F32, *w, prefix=pref)
    assert np.all(tab[:, 0] == 0)
    assert np.all(tab[:, -1] == O.M)          # frequencies sum to the coder total
    f = np.diff(tab, axis=1)
    assert np.all(f >= 1)                     # every symbol stays codable


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
@pytest.mark.parametrize("mode", ["single", "mixture"])
def test_slot_ranges_tile_the_coder_range(dtype, mode):
    """The coder's slots: the Gaussian ranges [G(b), G(b+1)) tile
    [0, T_n + T_w) and the floor-and-escape ranges [Q(b), Q(b+1)) tile
    [0, N + T_e) (placed after them), and each symbol's two ranges add up to
    its mixture frequency C(b+1) - C(b): a bijection between slots and
    (symbol, rank) pairs with the mixture's frequencies."""
    w = (10000, 0) if mode == "single" else (9500, 300)
    t_n, t_w, t_e = O.budgets(dtype, *w)
    pref = marginal(dtype) if mode == "mixture" else None
    n = O.alphabet_size(dtype)
    b = np.arange(n + 1, dtype=np.int64)
    q = O.escape_cum(b, pref)
    assert q[0] == 0 and q[-1] == n + t_e and np.all(np.diff(q) >= 1)
    for mu, sg in ADVERSARIAL:
        mu32 = O.mu_to_f32(np.array([mu], dtype=np.float32), O.F32)[0]
        inv = (np.float32(1.0) / np.float32(sg)).astype(np.float32)
        g = O.gauss_cum(b, mu32, inv, dtype, t_n, t_w)
        assert g[0] == 0 and g[-1] == t_n + t_w and np.all(np.diff(g) >= 0)
        c = O.cdf(b, mu32, inv, dtype, t_n, t_w, pref)
        assert np.array_equal(np.diff(g) + np.diff(q), np.diff(c))


def test_single_gaussian_floor_symbol_costs_31_bits():
    tab = O.cdf_table(np.float32([1.0]), np.float32([0.01]), O.BF16, O.F32, 10000, 0)[0]
    nan_sym = int(O.order_index(0x7FC0, O.BF16))
    assert tab[nan_sym + 1] - tab[nan_sym] == 1          # -log2(1/M) = 31 bits


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
def test_close_to_continuous_mixture(dtype, pages):
    wts = pages["mixture_weights"]["value"]
    k = pages["wide_sigma_factor"]["value"]
    n = O.alphabet_size(dtype)
    t = O.M - n
    pref = marginal(dtype, seed=3)
    # the escape part as the pages describe it: the empirical marginal
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000).astype(np.float32)
    import torch
    if dtype == O.BF16:
        bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        bits = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    idx = O.order_index(bits, dtype)
    counts = np.bincount(idx, minlength=n) + 1
    cum = np.concatenate([[0], np.cumsum(counts)]) / counts.sum()
    pos = O.boundary_positions(dtype).astype(np.float64)
    cases = [(0.3, 0.05), (-1.2, 0.4), (0.0, 1e-3), (2.5, 2.0 ** -7), (-0.01, 0.2), (40.0, 3.0)]
    for mu, s in cases:
        tab = O.cdf_table(np.float32([mu]), np.float32([s]), dtype, O.F32, 9500, 300, prefix=pref)[0]
        mu64, s64 = float(np.float32(mu)), float(np.float32(s))
        with np.errstate(invalid="ignore"):
            zf = (pos - mu64) / s64
        ref = t * (wts["narrow"] * ndtr(zf) + wts["wide"] * ndtr(zf / k) + wts["escape"] * cum)
        err = np.abs(tab - np.arange(n + 1) - ref)
        # interpolation <= 992 units, float32 z within 3 roundings <= ~130
        # units, budget floors and weight rounding <= 4 units
        assert err.max() < 1300, (mu, s, err.max())


def test_nonfinite_mu_is_treated_as_zero():
    a = O.cdf_table(np.float32([np.nan, np.inf, -np.inf]), np.float32([0.3] * 3), O.BF16, O.F32, 10000, 0)
    b = O.cdf_table(np.float32([0.0]), np.float32([0.3]), O.BF16, O.F32, 10000, 0)
    assert np.array_equal(a, np.repeat(b, 3, axis=0))


@pytest.mark.parametrize("bad", [0.0, -1.0, np.inf, np.nan, 1e-45, 1e-30, 1e30])
def test_bad_sigma_rejected(bad):
    with pytest.raises(ValueError):
        O.cdf_table(np.float32([0.0]), np.float32([bad]), O.E4M3, O.F32, 10000, 0)
