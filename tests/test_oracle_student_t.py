"""Pins of the oracle's Student-t narrow part (S-13, an optional residual
model: the pages name a better, heavier-tailed residual model as future work
without a form).  The t CDF against scipy's (another implementation) and the
closed forms for one and two degrees of freedom; the table's ends, symmetry,
rounding margin and step bound; the CDF invariants over whole alphabets; the
round trip; and the model's cost against the closed-form entropy of the
discretised t."""
import math

import numpy as np
import pytest
from scipy.special import beta, digamma, stdtr

import oracle as O
from entropy_coding_amd import workloads as W


@pytest.mark.parametrize("nu", list(range(1, 17)))
def test_t_cdf_matches_scipy(nu):
    import mpmath
    zs = [-24.0, -7.5, -3.0, -1.0, -0.3, 0.0, 0.01, 0.5, 2.0, 5.25, 12.0, 24.0]
    with mpmath.workdps(30):
        for z in zs:
            assert abs(float(O.student_t_cdf_mp(z, nu)) - stdtr(nu, z)) < 2e-15


def test_t_cdf_closed_forms():
    import mpmath
    with mpmath.workdps(40):
        for z in (-20.0, -1.5, 0.25, 3.0):
            assert abs(O.student_t_cdf_mp(z, 1) - (mpmath.mpf(1) / 2 + mpmath.atan(z) / mpmath.pi)) < 1e-35
            want2 = mpmath.mpf(1) / 2 + z / (2 * mpmath.sqrt(2 + mpmath.mpf(z) ** 2))
            assert abs(O.student_t_cdf_mp(z, 2) - want2) < 1e-35


@pytest.mark.parametrize("nu", [1, 2, 3, 5, 8, 16])
def test_narrow_table(nu):
    """Ends 0 and 2^31, symmetric, increasing, every step below 2^22, and
    equal to the float64 rounding of scipy's truncated t CDF (no entry lies
    near a rounding tie)."""
    a = O.narrow_table(nu)
    assert a.size == O.kvc_oracle.TABLE_POINTS and a[0] == 0 and a[-1] == 1 << 31
    assert np.all(a + a[::-1] == 1 << 31)
    assert np.all(np.diff(a) >= 0) and np.diff(a).max() < 1 << 22
    z = -24.0 + np.arange(O.kvc_oracle.TABLE_POINTS) / 256.0
    lo = stdtr(nu, -24.0)
    x = (stdtr(nu, z) - lo) / (1.0 - 2.0 * lo) * 2.0 ** 31
    frac = x - np.floor(x)
    assert np.min(np.abs(frac - 0.5)) > 1e-5
    assert np.array_equal(np.floor(x + 0.5).astype(np.int64), a)


def test_large_dof_approaches_the_gaussian():
    g = O.phi_tables()[0].astype(np.float64)
    d16 = np.abs(O.narrow_table(16) - g).max() / 2.0 ** 31
    d3 = np.abs(O.narrow_table(3) - g).max() / 2.0 ** 31
    assert d16 < d3 / 3 and d16 < 0.02


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
@pytest.mark.parametrize("nu", [1, 3, 7])
def test_cdf_invariants_with_a_t_narrow_part(dtype, nu):
    n = O.alphabet_size(dtype)
    samples = (np.random.default_rng(1).standard_normal(5000)).astype(np.float32)
    import torch
    bits = W.to_numpy_bits(torch.from_numpy(samples).to(torch.bfloat16 if dtype == O.BF16 else torch.float8_e4m3fn)
                           .view(torch.int16 if dtype == O.BF16 else torch.uint8)) if dtype == O.E4M3 else \
        W.to_numpy_bits(torch.from_numpy(samples).to(torch.bfloat16))
    pref = O.build_marginal(bits, dtype, 9500, 300)
    mu_dtype = O.BF16 if dtype == O.BF16 else O.F32
    mus = np.array([0x3FC0, 0x0000, 0xC2C8, 0x0001], dtype=np.uint16) if dtype == O.BF16 else \
        np.array([1.5, 0.0, -100.0, 1e-7], dtype=np.float32)
    for sg in (2.0 ** -96, 2.0 ** -9, 0.5, 2.0 ** 96):
        c = O.cdf_table(mus, np.full(mus.size, sg, dtype=np.float32), dtype, mu_dtype, 9500, 300, pref, narrow_dof=nu)
        assert np.all(c[:, 0] == 0) and np.all(c[:, n] == O.M)
        assert np.all(np.diff(c, axis=1) >= 1)


@pytest.mark.parametrize("nu", [3, 5])
@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
def test_round_trip_and_header_field(nu, kv_dtype):
    kv, mu, sig, samples = W.tiny_case(7, 3, 45, 128, kv_dtype)
    kv, mu, sig, samples = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(samples, kv_dtype, 9500, 300)
    st = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, 16, narrow_dof=nu)
    assert O.parse_header(st)["narrow_dof"] == nu and st[14] == nu
    assert np.array_equal(O.decode(st, mu, sig, pref), kv)
    # a different narrow part is a different stream
    assert O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, 16) != st
    bad = bytearray(st)
    bad[14] = 17
    import zlib
    bad[92:96] = zlib.crc32(bytes(bad[:92])).to_bytes(4, "little")
    with pytest.raises(O.StreamError):
        O.parse_header(bytes(bad))
    with pytest.raises(ValueError):
        O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, 16, narrow_dof=17)


def t_entropy_bits(nu):
    """Differential entropy of the standard t_nu in bits:
    (nu+1)/2 [psi((nu+1)/2) - psi(nu/2)] + ln(sqrt(nu) B(nu/2, 1/2)) nats."""
    h = (nu + 1) / 2 * (digamma((nu + 1) / 2) - digamma(nu / 2)) + math.log(math.sqrt(nu) * beta(nu / 2, 0.5))
    return h / math.log(2)


def test_t_model_cost_closed_form():
    """Data drawn from the model itself (t_3 truncated at 24 scale units, scale
    2^-5 around 1.5, where every BF16 cell is 2^-7 wide): the mean cost of the
    float model is the entropy of the discretised t, which for cells narrow
    against the scale is h(t_3) + log2(scale / width)."""
    nu, scale = 3, 2.0 ** -5
    rng = np.random.default_rng(13)
    t = rng.standard_t(nu, 1 << 18)
    t = t[np.abs(t) < 24.0][: 1 << 17]
    import torch
    x = torch.from_numpy(1.5 + scale * t).to(torch.float32)
    kv = W.to_numpy_bits(x.to(torch.bfloat16)).reshape(1, -1, 64)
    mu = W.to_numpy_bits(torch.full((kv.size,), 1.5).to(torch.bfloat16)).reshape(1, -1, 64)
    sig = np.full((1, 64), scale, dtype=np.float32)
    fl = O.model_bits_float(kv, mu, sig, None, O.BF16, O.BF16, 10000, 0, narrow_dof=nu)
    ib = O.model_bits_int(kv, mu, sig, None, O.BF16, O.BF16, 10000, 0, narrow_dof=nu)
    closed = t_entropy_bits(nu) + math.log2(scale / 2.0 ** -7)
    # exact entropy of the discretised, truncated t over the cells in [1, 2)
    # and their mirror images beyond (cells of 2^-7 up to 2, 2^-6 above)
    v = 1.0 + np.arange(128) / 128.0
    edges = np.concatenate([v - 2.0 ** -8, [2.0 - 2.0 ** -8]])
    p = stdtr(nu, (edges[1:] - 1.5) / scale) - stdtr(nu, (edges[:-1] - 1.5) / scale)
    inside = p.sum()
    exact_inside = float(-(p * np.log2(p)).sum())
    se = 2.0 / math.sqrt(kv.size)
    assert inside > 0.999
    assert abs(fl - closed) < 0.02 and abs(exact_inside - closed) < 0.02
    assert abs(ib - fl) < 2e-3


def test_t_narrow_part_fits_a_heavy_tailed_residual_better():
    """On the heavy-tailed synthetic residual of the 8B-shaped workload (85%
    t_3, 14.5% normal, 0.5% outliers at 20 sigma), each model at the scale the
    rate fit picks: the t_3 narrow part costs fewer bits than the Gaussian."""
    w = W.WORKLOADS[2]
    kv, mu = W.layer_data(w, 0, tokens=256)
    ck, cm = W.layer_calibration(w, 0, reps=2, tokens=256)
    kvn, mun = W.to_numpy_bits(kv[:8]), W.to_numpy_bits(mu[:8])
    ckn, cmn = W.to_numpy_bits(ck[:, :8]), W.to_numpy_bits(cm[:, :8])
    pref = O.build_marginal(W.to_numpy_bits(W.marginal_samples(w)), O.BF16, 9500, 300)
    bits = {}
    for nu in (0, 3):
        sg = O.calibrate_sigma_rate(ckn, cmn, O.BF16, O.BF16, 2.0 ** -30, pref, 9500, 300, narrow_dof=nu)
        bits[nu] = O.model_bits_int(kvn, mun, sg, pref, O.BF16, O.BF16, 9500, 300, narrow_dof=nu)
    assert bits[3] < bits[0] - 0.01, bits
