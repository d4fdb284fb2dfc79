"""Pins of the oracle's position-aware sigma (S-11: sigma per block of B
tokens; [blog] § limitations and future directions).  Special cases reduce
to the per-plane sigma, the calibration has a closed form per block, a
block's sigma reaches only its own chunks, and the model with matched
per-block sigma costs less than one sigma per plane when the residual
scale changes with position."""
import numpy as np
import pytest

import oracle as O
from entropy_coding_amd import workloads as W

W_MIX = (9500, 300)


def case(seed=11, planes=2, tokens=45, channels=128):
    kv, mu, sig, samples = W.tiny_case(seed, planes, tokens, channels, O.BF16)
    return W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)


def body(stream: bytes) -> bytes:
    """Directory and payloads: everything after the header."""
    return stream[O.HEADER_BYTES:]


def test_one_block_covering_every_token_is_the_per_plane_sigma():
    kv, mu, sig, samples = case()
    pref = O.build_marginal(samples, O.BF16, *W_MIX)
    a = O.encode(kv, mu, sig, pref, O.BF16, O.BF16, *W_MIX, 16)
    b = O.encode(kv, mu, sig[:, None, :], pref, O.BF16, O.BF16, *W_MIX, 16, sigma_block_tokens=45)
    c = O.encode(kv, mu, sig[:, None, :], pref, O.BF16, O.BF16, *W_MIX, 16, sigma_block_tokens=1000)
    assert body(a) == body(b) == body(c)
    # the same sigma words: the same side hash; only the block field differs
    assert a[:88] == b[:88] and O.parse_header(b)["sigma_block_tokens"] == 45
    assert np.array_equal(O.decode(b, mu, sig[:, None, :], pref), kv)


def test_equal_blocks_give_the_per_plane_payloads():
    kv, mu, sig, samples = case()
    pref = O.build_marginal(samples, O.BF16, *W_MIX)
    a = O.encode(kv, mu, sig, pref, O.BF16, O.BF16, *W_MIX, 8)
    rep = np.repeat(sig[:, None, :], 3, axis=1)            # B = 16: blocks of 16, 16, 13 tokens
    b = O.encode(kv, mu, rep, pref, O.BF16, O.BF16, *W_MIX, 8, sigma_block_tokens=16)
    ha, hb = O.parse_header(a), O.parse_header(b)
    assert ha["side_hash"] != hb["side_hash"]              # 3x the sigma words
    assert body(a) == body(b)


@pytest.mark.parametrize("tc,blk", [(8, 16), (5, 15), (9, 9), (1, 4)])
def test_round_trip_with_varying_block_sigma(tc, blk):
    kv, mu, sig, samples = case(tokens=45)
    nb = -(-45 // blk)
    rng = np.random.default_rng(tc * 100 + blk)
    sig3 = (sig[:, None, :] * rng.uniform(0.25, 4.0, size=(sig.shape[0], nb, sig.shape[1]))).astype(np.float32)
    pref = O.build_marginal(samples, O.BF16, *W_MIX)
    st = O.encode(kv, mu, sig3, pref, O.BF16, O.BF16, *W_MIX, tc, sigma_block_tokens=blk)
    assert np.array_equal(O.decode(st, mu, sig3, pref), kv)
    with pytest.raises(O.StreamError):
        O.decode(st, mu, sig3[:, :1, :], pref)             # wrong shape for the stream's blocks
    with pytest.raises(O.StreamError):
        O.decode(st, mu, sig3 * np.float32(2), pref)       # other sigma: side hash


def test_a_blocks_sigma_reaches_only_its_chunks():
    kv, mu, sig, samples = case(tokens=48)
    pref = O.build_marginal(samples, O.BF16, *W_MIX)
    tc, blk = 8, 16
    sig3 = np.repeat(sig[:, None, :], 3, axis=1)
    a = O.encode(kv, mu, sig3, pref, O.BF16, O.BF16, *W_MIX, tc, sigma_block_tokens=blk)
    sig3b = sig3.copy()
    sig3b[1, 1, 70] *= np.float32(3.0)                    # plane 1, tokens 16..31, channel 70
    b = O.encode(kv, mu, sig3b, pref, O.BF16, O.BF16, *W_MIX, tc, sigma_block_tokens=blk)
    g_of, tc_of, k_of, _ = O.chunk_layout(2, 48, 128, tc)
    for cid in range(g_of.size):
        same = O.chunk_payload(a, cid) == O.chunk_payload(b, cid)
        hit = g_of[cid] == 1 and tc_of[cid] * tc // blk == 1 and k_of[cid] == 1
        assert same != hit, cid


def test_block_length_must_tile_the_chunks():
    kv, mu, sig, samples = case(tokens=45)
    pref = O.build_marginal(samples, O.BF16, *W_MIX)
    sig3 = np.repeat(sig[:, None, :], 3, axis=1)
    with pytest.raises(ValueError):
        O.encode(kv, mu, sig3, pref, O.BF16, O.BF16, *W_MIX, 8, sigma_block_tokens=20)
    with pytest.raises(ValueError):
        O.encode(kv, mu, sig, pref, O.BF16, O.BF16, *W_MIX, 8, sigma_block_tokens=16)   # sigma [G, D]


def test_calibration_per_block_closed_form():
    """Residual c_j (a constant) in block j: sigma[p, j, d] = |c_j| exactly;
    B = 0 gives the RMS over every token; B >= T gives that same value as a
    single block."""
    reps, planes, tokens, ch = 2, 1, 10, 64
    mu = np.zeros((reps, planes, tokens, ch), dtype=np.float32)
    c = np.array([0.5] * 4 + [2.0] * 4 + [0.125] * 2, dtype=np.float32)   # blocks of 4: 4, 4, 2 tokens
    kv32 = np.broadcast_to(c[None, None, :, None], mu.shape).astype(np.float32)
    kv = (kv32.view(np.uint32) >> 16).astype(np.uint16)                    # exact in bf16
    s = O.calibrate_sigma(kv, mu, O.BF16, O.F32, 2.0 ** -30, block_tokens=4)
    assert s.shape == (planes, 3, ch)
    assert np.all(s[0, 0] == 0.5) and np.all(s[0, 1] == 2.0) and np.all(s[0, 2] == 0.125)
    whole = O.calibrate_sigma(kv, mu, O.BF16, O.F32, 2.0 ** -30)
    expect = np.float32(np.sqrt(np.mean(c.astype(np.float64) ** 2)))
    assert whole.shape == (planes, ch) and np.all(whole == expect)
    one = O.calibrate_sigma(kv, mu, O.BF16, O.F32, 2.0 ** -30, block_tokens=64)
    assert one.shape == (planes, 1, ch) and np.array_equal(one[:, 0, :], whole)


def test_matched_block_sigma_costs_fewer_bits():
    """Residual N(0, s_j^2) with s_j differing 8x between blocks: the model
    with the per-block RMS costs less than the model with the RMS over every
    token (cross-entropy is least at the matched scale), by about
    log2 of the ratio of the scales' geometric and RMS means."""
    rng = np.random.default_rng(5)
    planes, tokens, ch, blk = 2, 64, 64, 16
    scale = np.array([0.4, 0.05, 0.05, 0.05], dtype=np.float64).repeat(blk)[:tokens]
    mu = rng.standard_normal((planes, tokens, ch)).astype(np.float32)
    x = mu + rng.standard_normal((planes, tokens, ch)) * scale[None, :, None]
    kv = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mub = (mu.view(np.uint32) >> 16).astype(np.uint16)
    per_plane = O.calibrate_sigma(kv[None], mub[None], O.BF16, O.BF16, 2.0 ** -30)
    per_block = O.calibrate_sigma(kv[None], mub[None], O.BF16, O.BF16, 2.0 ** -30, block_tokens=blk)
    pref = O.build_marginal(kv.ravel(), O.BF16, *W_MIX)
    b_plane = O.model_bits_int(kv, mub, per_plane, pref, O.BF16, O.BF16, *W_MIX)
    b_block = O.model_bits_int(kv, mub, per_block, pref, O.BF16, O.BF16, *W_MIX, sigma_block_tokens=blk)
    gain = np.log2(np.sqrt(np.mean(scale ** 2)) / np.exp(np.mean(np.log(scale))))
    assert b_block < b_plane
    assert abs((b_plane - b_block) - gain) < 0.25
    st = O.encode(kv, mub, per_block, pref, O.BF16, O.BF16, *W_MIX, 16, sigma_block_tokens=blk)
    assert np.array_equal(O.decode(st, mub, per_block, pref), kv)
