"""Pins of the off-path helpers: the empirical marginal, sigma calibration
and the side-information checksum."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def test_marginal_brute_force_tiny():
    # e4m3 patterns: +1.0 is 0x38, -2.0 is 0xC0
    samples = np.array([0x38, 0x38, 0x38, 0xC0], dtype=np.uint8)
    pref = O.build_marginal(samples, O.E4M3, 9500, 300)
    t_e = O.budgets(O.E4M3, 9500, 300)[2]
    # counting by hand over values, not indices: the symbol of -2.0 sits
    # below the symbol of +1.0; every symbol carries weight 1 + its count
    vals = O.symbol_value(np.arange(256), O.E4M3)
    weight = [1 + (3 if v == 1.0 else 1 if v == -2.0 else 0) for v in vals]
    total = sum(weight)
    assert total == 260
    cum = 0
    for b in range(257):
        assert pref[b] == (Fraction(t_e) * cum / total).__floor__()
        if b < 256:
            cum += weight[b]
    assert pref[0] == 0 and pref[256] == t_e


def test_marginal_single_mode_is_zero():
    pref = O.build_marginal(np.array([1, 2, 3], dtype=np.uint16), O.BF16, 10000, 0)
    assert np.all(pref == 0)


def test_marginal_increments_follow_counts():
    rng = np.random.default_rng(2)
    samples = rng.integers(0, 65536, 300000).astype(np.uint16)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    t_e = O.budgets(O.BF16, 9500, 300)[2]
    c = np.bincount(O.order_index(samples, O.BF16), minlength=65536) + 1
    expect = t_e * c / c.sum()
    assert np.all(np.abs(np.diff(pref) - expect) < 1.0 + 1e-9)


def _bf16(x):
    import torch
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_calibrate_sigma_closed_form():
    # residuals +-0.5 and +-0.25 in equal numbers: RMS = sqrt(0.15625)
    mu = np.full((2, 1, 4, 64), 1.0, dtype=np.float32)
    res = np.array([0.5, -0.5, 0.25, -0.25], dtype=np.float32)[None, None, :, None]
    kv = mu + res
    s = O.calibrate_sigma(_bf16(kv), _bf16(mu), O.BF16, O.BF16, 2.0 ** -30)
    assert s.shape == (1, 64) and s.dtype == np.float32
    assert np.all(s == np.float32(np.sqrt(0.15625)))
    # RMS about mu, not about the residual mean: a constant offset counts
    s2 = O.calibrate_sigma(_bf16(mu + 0.5), _bf16(mu), O.BF16, O.BF16, 2.0 ** -30)
    assert np.all(s2 == np.float32(0.5))


def test_calibrate_sigma_floor_and_f32_mu():
    kv = np.zeros((1, 2, 3, 64), dtype=np.uint8)          # e4m3 +0
    mu = np.zeros((1, 2, 3, 64), dtype=np.float32)
    mu[0, 0, 0, 0] = np.nan                               # treated as 0
    s = O.calibrate_sigma(kv, mu, O.E4M3, O.F32, 2.0 ** -30)
    assert np.all(s == np.float32(2.0 ** -30))


# splitmix64 (Vigna): the state advances by 0x9E3779B97F4A7C15 per output
# and each output is the finaliser of the new state; seeded with 0, the
# generator's first three outputs are published values.
SPLITMIX64_SEED0 = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def _mix_scalar(z: int) -> int:
    """The splitmix64 finaliser on a Python int, reduced mod 2^64 by hand."""
    m = (1 << 64) - 1
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def test_side_hash_mixer_is_splitmix64():
    """The oracle's mixer reproduces splitmix64's published first outputs
    (seed 0), so a wrong shift or constant cannot pass."""
    from oracle import kvc_oracle as K
    golden = 0x9E3779B97F4A7C15
    for k, want in enumerate(SPLITMIX64_SEED0, start=1):
        state = (k * golden) % (1 << 64)
        assert _mix_scalar(state) == want
        with np.errstate(over="ignore"):
            assert int(K._mix64(np.uint64(state))) == want


def test_side_hash_small_case_by_hand():
    """Two sigma words and a three-entry prefix, summed word by word with
    Python ints: sum over (tag, index, word) of mix((index << 32 | word) +
    tag * golden) mod 2^64, sigma words tag 1, prefix words tag 2."""
    golden = 0x9E3779B97F4A7C15
    sig = np.array([[0.5, 3.0]], dtype=np.float32)          # words 0x3F000000, 0x40400000
    pref = np.array([0, 7, 1 << 30], dtype=np.int64)
    m = (1 << 64) - 1
    want = 0
    for i, w in enumerate([0x3F000000, 0x40400000]):
        want += _mix_scalar(((i << 32 | w) + 1 * golden) & m)
    for i, w in enumerate([0, 7, 1 << 30]):
        want += _mix_scalar(((i << 32 | w) + 2 * golden) & m)
    assert O.side_hash(sig, pref) == want & m
    assert O.side_hash(sig, None) == (_mix_scalar((0x3F000000 + golden) & m)
                                      + _mix_scalar(((1 << 32 | 0x40400000) + golden) & m)) & m


def test_side_hash_sensitivity():
    rng = np.random.default_rng(4)
    sig = rng.random((16, 128)).astype(np.float32)
    pref = np.sort(rng.integers(0, 1 << 26, 257))
    h0 = O.side_hash(sig, pref)
    assert 0 <= h0 < 2 ** 64
    assert O.side_hash(sig, pref) == h0
    for _ in range(100):
        s2 = sig.copy().view(np.uint32)
        i = int(rng.integers(0, s2.size))
        s2.flat[i] ^= np.uint32(1 << int(rng.integers(0, 32)))
        assert O.side_hash(s2.view(np.float32), pref) != h0
    p2 = pref.copy()
    p2[[3, 4]] = p2[[4, 3]]
    assert O.side_hash(sig, p2) != h0
    assert O.side_hash(sig, None) != h0


def test_scatter_to_pages_brute_force():
    """The paged placement against plain loops over every (plane, token)."""
    rng = np.random.default_rng(3)
    layers, batch, heads, t_len, d, pt = 2, 3, 2, 11, 64, 4
    g_n = layers * 2 * batch * heads
    kv = rng.integers(0, 1 << 16, size=(g_n, t_len, d)).astype(np.uint16)
    max_pages, num_pages = 3, 20
    table = rng.permutation(num_pages)[:batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    got = O.scatter_to_pages(kv, batch, heads, table, pt, num_pages, fill=0xABCD)
    want = np.full((layers * 2, num_pages, pt, heads, d), 0xABCD, dtype=np.uint16)
    for g in range(g_n):
        lk, rest = divmod(g, batch * heads)
        b, h = divmod(rest, heads)
        for t in range(t_len):
            want[lk, table[b, t // pt], t % pt, h, :] = kv[g, t, :]
    assert np.array_equal(got, want)
    # every token lands somewhere distinct: the pages hold all of kv
    assert np.sum(got != 0xABCD) == np.sum(kv != 0xABCD)
    with pytest.raises(ValueError):
        O.scatter_to_pages(kv, batch, heads, np.full((batch, max_pages), num_pages, np.int32), pt, num_pages)
