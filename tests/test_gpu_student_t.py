"""GPU parity of the Student-t narrow part (an optional residual model):
streams byte-identical to the oracle's for several degrees of freedom,
dtypes and weights, the CDF for every symbol, the bits estimates, and the
rate-fitted sigma under the t model."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bits(x, dev):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def case(kv_dtype, seed=7, planes=3, tokens=45, channels=128):
    kv, mu, sig, samples = W.tiny_case(seed, planes, tokens, channels, kv_dtype)
    return W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)


@pytest.mark.parametrize("nu", [1, 3, 4, 16])
@pytest.mark.parametrize("kv_dtype,w", [(O.BF16, (9500, 300)), (O.BF16, (10000, 0)), (O.E4M3, (9500, 300))])
def test_stream_matches_oracle(kvc, cuda, nu, kv_dtype, w):
    kv, mu, sig, samples = case(kv_dtype)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(samples, kv_dtype, *w) if w[0] + w[1] < 10000 else None
    want = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, *w, 16, narrow_dof=nu)
    pref_d = None if pref is None else torch.from_numpy(pref.astype(np.int32)).to(cuda)
    kv_d, mu_d, sig_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, w, 16, narrow_dof=nu)
    assert st.cpu().numpy().tobytes() == want
    out = kvc.kvc_decode(st, mu_d, sig_d, pref_d)
    assert torch.equal(out, kv_d.view(out.dtype))


@pytest.mark.parametrize("nu", [2, 3, 9])
@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
def test_cdf_table_matches_oracle(kvc, cuda, nu, kv_dtype):
    rng = np.random.default_rng(nu)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    n = 12
    if kv_dtype == O.BF16:
        mu = W.to_numpy_bits(torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 3).to(torch.bfloat16))
    else:
        mu = (rng.standard_normal(n) * 30).astype(np.float32)
    sig = (2.0 ** rng.uniform(-12, 4, n)).astype(np.float32)
    samples = W.to_numpy_bits(W.tiny_case(3, kv_dtype=kv_dtype)[3])
    pref = O.build_marginal(samples, kv_dtype, 9500, 300)
    want = O.cdf_table(mu, sig, kv_dtype, mu_dtype, 9500, 300, pref, narrow_dof=nu)
    got = kvc.kvc_cdf_table(kv_dtype, dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda),
                            torch.from_numpy(pref.astype(np.int32)).to(cuda), (9500, 300), narrow_dof=nu)
    assert np.array_equal(got.cpu().numpy().view(np.uint32).astype(np.int64), want)


def test_estimate_bits_match_oracle(kvc, cuda):
    kv, mu, sig, samples = case(O.BF16, planes=2, tokens=64)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    for nu in (3, 6):
        bi = O.model_bits_int(kv, mu, sig, pref, O.BF16, O.BF16, 9500, 300, narrow_dof=nu)
        bf = O.model_bits_float(kv, mu, sig, pref, O.BF16, O.BF16, 9500, 300, narrow_dof=nu)
        gi, gf = kvc.kvc_estimate_bits(dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda),
                                       torch.from_numpy(pref.astype(np.int32)).to(cuda), narrow_dof=nu)
        assert abs(gi - bi) <= 1e-9 * bi and abs(gf - bf) < 1e-3


def test_rate_sigma_matches_oracle(kvc, cuda):
    w = W.WORKLOADS[2]
    ck, cm = W.layer_calibration(w, 0, reps=2, tokens=64)
    ck, cm = ck[:, :4].contiguous(), cm[:, :4].contiguous()
    pref = O.build_marginal(W.to_numpy_bits(W.marginal_samples(w)), O.BF16, 9500, 300)
    pref_d = torch.from_numpy(pref.astype(np.int32)).to(cuda)
    got = kvc.kvc_calibrate_sigma_rate(ck.to(cuda), cm.to(cuda), pref_d, (9500, 300), narrow_dof=3)
    base = kvc.kvc_calibrate_sigma(ck.to(cuda), cm.to(cuda)).cpu().numpy()
    want = O.calibrate_sigma_rate(W.to_numpy_bits(ck), W.to_numpy_bits(cm), O.BF16, O.BF16, 2.0 ** -30, pref,
                                  9500, 300, base=base, narrow_dof=3)
    assert np.array_equal(got.cpu().numpy(), want)
