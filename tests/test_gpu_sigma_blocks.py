"""GPU parity of position-aware sigma (one sigma per block of B tokens):
streams byte-identical to the oracle's and decoded exactly, per-block
calibration within one float32 ulp of the oracle, the bits estimate, and
the error statuses of the new field."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bits(x: np.ndarray, dev):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def dev_prefix(pref, dev):
    return None if pref is None else torch.from_numpy(np.asarray(pref, dtype=np.int64).astype(np.int32)).to(dev)


def block_sigma(sig, nb, seed):
    rng = np.random.default_rng(seed)
    return (sig[:, None, :] * rng.uniform(0.25, 4.0, size=(sig.shape[0], nb, sig.shape[1]))).astype(np.float32)


CASES = [
    # kv dtype, weights, chunk tokens, block tokens, planes, tokens, channels
    (O.BF16, (9500, 300), 8, 16, 3, 45, 128),      # ragged last block (13 tokens) and chunk (5)
    (O.BF16, (9500, 300), 5, 15, 2, 45, 128),      # three chunks per block
    (O.BF16, (10000, 0), 9, 9, 2, 40, 192),        # block = chunk, three channel groups
    (O.BF16, (9500, 300), 16, 100, 2, 45, 64),     # one block covers every token
    (O.E4M3, (9500, 300), 7, 14, 3, 45, 128),
]


@pytest.mark.parametrize("kv_dtype,w,tc,blk,g,t,d", CASES)
def test_block_sigma_stream_matches_oracle(kvc, cuda, kv_dtype, w, tc, blk, g, t, d):
    say(f"case kv={kv_dtype} w={w} tc={tc} block={blk} shape={g}x{t}x{d}")
    kv, mu, sig, samples = W.tiny_case(13, g, t, d, kv_dtype)
    kv, mu, sig, samples = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    nb = -(-t // blk)
    sig3 = block_sigma(sig, nb, tc * 31 + blk)
    pref = O.build_marginal(samples, kv_dtype, *w) if w[0] + w[1] < 10000 else None
    expect = O.encode(kv, mu, sig3, pref, kv_dtype, mu_dtype, *w, tc, sigma_block_tokens=blk)
    kv_d, mu_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), dev_prefix(pref, cuda)
    sig_d = torch.from_numpy(sig3).to(cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, w, tc, sigma_block_tokens=blk)
    got = st.cpu().numpy().tobytes()
    assert len(got) == len(expect)
    if got != expect:
        diff = np.flatnonzero(np.frombuffer(got, np.uint8) != np.frombuffer(expect, np.uint8))
        pytest.fail(f"stream differs at {diff[:8]} of {len(got)}")
    out = kvc.kvc_decode(st, mu_d, sig_d, pref_d)
    assert np.array_equal(out.cpu().numpy().view(kv.dtype), kv)
    # the bits estimate uses the same per-block sigma
    if kv_dtype == O.BF16:
        bi, _ = kvc.kvc_estimate_bits(kv_d, mu_d, sig_d, pref_d, w, sigma_block_tokens=blk, chunk_tokens=tc)
        ei = O.model_bits_int(kv, mu, sig3, pref, kv_dtype, mu_dtype, *w, sigma_block_tokens=blk)
        assert abs(bi - ei) <= 1e-9 * ei


def test_block_sigma_errors(kvc, cuda):
    kv, mu, sig, samples = W.tiny_case(5, 2, 45, 128, O.BF16)
    kv, mu, sig, samples = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    sig3 = block_sigma(sig, 3, 1)
    kv_d, mu_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), dev_prefix(pref, cuda)
    sig_d = torch.from_numpy(sig3).to(cuda)
    # a block length that is not a multiple of the chunk length
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 2, 45, 128, (9500, 300), 8, 20)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_encode_sizes(p)
    assert e.value.status == kvc.KVC_ERR_INVALID
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, (9500, 300), 8, sigma_block_tokens=16)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    out = torch.empty(kv.shape, dtype=torch.int16, device=cuda)
    assert kvc.kvc_decode_into(st, mu_d, sig_d, pref_d, out, ws) == kvc.KVC_OK
    # one sigma of the last block changed: the checksum covers every block
    s2 = sig_d.clone()
    s2[1, 2, 77] *= 2
    assert kvc.kvc_decode_into(st, mu_d, s2, pref_d, out, ws) == kvc.KVC_ERR_MISMATCH
    # the per-plane sigma of the same planes is smaller than the blocks the
    # header describes: refused before anything runs
    assert kvc.kvc_decode_into(st, mu_d, torch.from_numpy(sig).to(cuda), pref_d, out, ws) == kvc.KVC_ERR_INVALID


@pytest.mark.parametrize("reps,planes,tokens,channels,blk", [
    (2, 3, 45, 128, 16),      # ragged last block
    (5, 2, 33, 64, 1),        # one token per block
    (3, 1, 300, 192, 128),    # many splits per block
    (2, 2, 40, 64, 64),       # one block covering every token
])
def test_block_calibration_matches_oracle(kvc, cuda, reps, planes, tokens, channels, blk):
    g = torch.Generator(device="cpu").manual_seed(reps * 100 + tokens + blk)
    mu = (torch.randn((reps, planes, tokens, channels), generator=g) * 0.5).to(torch.bfloat16)
    scale = 0.02 + 0.2 * torch.rand((1, 1, tokens, 1), generator=g)        # residual scale by position
    kv = (mu.float() + scale * torch.randn(mu.shape, generator=g)).to(torch.bfloat16)
    got = kvc.kvc_calibrate_sigma(kv.to(cuda), mu.to(cuda), block_tokens=blk).cpu().numpy()
    expect = O.calibrate_sigma(W.to_numpy_bits(kv), W.to_numpy_bits(mu), O.BF16, O.BF16, 2.0 ** -30,
                               block_tokens=blk)
    assert got.shape == expect.shape == (planes, -(-tokens // blk), channels)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - expect.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
