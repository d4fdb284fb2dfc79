"""Pins of the per-channel split of the Gaussian budget (KVC-1 S-14): each
(plane, channel) moves weight between the narrow and the wide Gaussian while
the escape weight stays the call's.

- Where every lane of a chunk has the same narrow weight, and the weights are
  multiples of 625 bp so that every floor is exact, a chunk must be the same
  bytes as the chunk coded with that weight as the call's (already pinned)
  global weights.
- Where every lane has its own weight, each lane's final state and word
  count must be those of a one-lane rANS written out in the test over that
  lane's frequencies, taken from a one-channel, global-weight model of that
  lane alone (a lane given another lane's split changes its state).
- Code lengths per channel, round trips, the header flag, the side hash and
  the calibration against a float64 brute force."""
import numpy as np
import pytest

import oracle as O
from entropy_coding_amd import workloads as W

W_N, W_W = 8750, 625                 # T w / 10^4 is an integer for multiples of 625 bp
W_ALL = W_N + W_W


def case(kv_dtype=O.BF16, seed=11, planes=2, tokens=40, channels=128):
    kv, mu, sig, samples = W.tiny_case(seed, planes, tokens, channels, kv_dtype)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    return (W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(),
            W.to_numpy_bits(samples), mu_dtype)


def _exact(kv_dtype, w):
    t = O.M - O.alphabet_size(kv_dtype)
    return (t * w) % 10000 == 0


def test_budgets_give_back_the_call_weights_and_stay_in_range():
    for kv_dtype in (O.BF16, O.E4M3):
        t_n, t_w, t_e = O.budgets(kv_dtype, 9500, 300)
        tn, tw = O.split_budgets(kv_dtype, 9500, 300, np.array([9500, 0, 9800, 4321]))
        assert (tn[0], tw[0]) == (t_n, t_w)               # w_c = w_n: the call's budgets
        assert tn[1] == 0 and tw[1] == t_n + t_w           # all Gaussian weight on the wide part
        assert tw[2] == 0 and tn[2] == t_n + t_w           # floor(T W / 10^4) > T_n + T_w is capped
        assert np.all(tn + tw == t_n + t_w) and np.all(tn >= 0) and np.all(tw >= 0)
        with pytest.raises(ValueError):
            O.split_budgets(kv_dtype, 9500, 300, np.array([9801]))
        with pytest.raises(ValueError):
            O.split_budgets(kv_dtype, 9500, 300, np.array([-1]))


@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
@pytest.mark.parametrize("sigma_block,dof", [(0, 0), (20, 0), (0, 5)])
def test_chunks_with_one_weight_equal_the_global_weight_chunks(kv_dtype, sigma_block, dof):
    planes, tokens, channels, tc = 2, 40, 192, 20
    kv, mu, sig, samples, mu_dtype = case(kv_dtype, planes=planes, tokens=tokens, channels=channels)
    if sigma_block:
        sig = np.stack([sig, sig * np.float32(0.75)], axis=1)
    values = [9375, 8750, 8125, 5000, 625, 0]
    assert all(_exact(kv_dtype, v) and _exact(kv_dtype, W_ALL - v) for v in values)
    split = np.zeros((planes, channels), dtype=np.int64)
    for g in range(planes):
        for k in range(channels // 64):
            split[g, 64 * k:64 * k + 64] = values[(3 * g + k) % len(values)]
    pref = O.build_marginal(samples, kv_dtype, W_N, W_W)
    st = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, W_N, W_W, tc, sigma_block_tokens=sigma_block,
                  narrow_dof=dof, channel_split=split)
    g_of, _, k_of, _ = O.chunk_layout(planes, tokens, channels, tc)
    for cid in range(len(g_of)):
        v = int(split[g_of[cid], 64 * k_of[cid]])
        ref = O.encode_chunks(kv, mu, sig, pref, kv_dtype, mu_dtype, v, W_ALL - v, tc, [cid],
                              sigma_block_tokens=sigma_block, narrow_dof=dof)[cid]
        assert O.chunk_payload(st, cid) == ref, (cid, v)
    assert np.array_equal(O.decode(st, mu, sig, pref, channel_split=split), kv)


@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
def test_each_lane_codes_under_its_own_weight(kv_dtype):
    """Each lane's final state and word count, from a one-lane rANS written
    out here with Python ints (S-8: emit while x >> 32 >= f, then
    x = (x // f) M + slot, slot = G(s) + r in the Gaussian range or T_n + T_w
    + Q(s) + r - f_G in the escape range) over that lane's own global-weight
    model."""
    kv, mu, sig, samples, mu_dtype = case(kv_dtype, planes=1, tokens=30, channels=64)
    pref = O.build_marginal(samples, kv_dtype, W_N, W_W)
    split = (625 * ((np.arange(64) * 5) % 16)).astype(np.int64)[None, :]     # 0 .. 9375 across lanes
    st = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, W_N, W_W, 30, channel_split=split)
    s = O.order_index(kv, kv_dtype)
    m = O.mu_to_f32(mu, mu_dtype)
    inv = (np.float32(1) / sig).astype(np.float32)
    states, n_words = [], 0
    for lane in range(64):
        v = int(split[0, lane])
        t_n, t_w, _ = O.budgets(kv_dtype, v, W_ALL - v)
        sl = s[0, :, lane]
        g0 = O.gauss_cum(sl, m[0, :, lane], inv[0, lane], kv_dtype, t_n, t_w)
        g1 = O.gauss_cum(sl + 1, m[0, :, lane], inv[0, lane], kv_dtype, t_n, t_w)
        x = O.L
        for t in range(29, -1, -1):
            fg = int(g1[t] - g0[t])
            q0 = int(sl[t]) + int(pref[sl[t]])
            f = fg + int(sl[t]) + 1 + int(pref[sl[t] + 1]) - q0
            while (x >> 32) >= f:
                x >>= 16
                n_words += 1
            r = x % f
            slot = int(g0[t]) + r if r < fg else t_n + t_w + q0 + (r - fg)
            x = (x // f) * O.M + slot
        states.append(x)
    body = O.chunk_payload(st, 0)
    assert list(np.frombuffer(body[:O.STATE_BYTES], dtype="<u8")) == states
    assert len(body) == O.STATE_BYTES + -(-2 * n_words // 8) * 8
    assert np.array_equal(O.decode(st, mu, sig, pref, channel_split=split), kv)
    assert all(_exact(kv_dtype, v) for v in range(0, W_ALL + 1, 625))      # the global models are exact


def test_code_length_is_the_sum_over_channels():
    """model_bits_int / _float with a split equal the per-channel models with
    that channel's weight as the call's."""
    kv, mu, sig, samples, mu_dtype = case(planes=2, tokens=24, channels=64)
    pref = O.build_marginal(samples, O.BF16, W_N, W_W)
    split = (625 * ((np.arange(128) * 7) % 16)).astype(np.int64).reshape(2, 64)
    got_i = O.model_bits_int(kv, mu, sig, pref, O.BF16, mu_dtype, W_N, W_W, channel_split=split)
    got_f = O.model_bits_float(kv, mu, sig, pref, O.BF16, mu_dtype, W_N, W_W, channel_split=split)
    ref_i = ref_f = 0.0
    for g in range(2):
        for c in range(64):
            v = int(split[g, c])
            sl = (slice(g, g + 1), slice(None), slice(c, c + 1))
            ref_i += O.model_bits_int(kv[sl], mu[sl], sig[g:g + 1, c:c + 1], pref, O.BF16, mu_dtype, v, W_ALL - v)
            ref_f += O.model_bits_float(kv[sl], mu[sl], sig[g:g + 1, c:c + 1], pref, O.BF16, mu_dtype, v,
                                        W_ALL - v)
    assert got_i == pytest.approx(ref_i / 128, rel=1e-12)
    assert got_f == pytest.approx(ref_f / 128, rel=1e-12)


@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
def test_round_trip_with_uneven_weights(kv_dtype):
    kv, mu, sig, samples, mu_dtype = case(kv_dtype, planes=3, tokens=33, channels=128)
    rng = np.random.default_rng(3)
    split = rng.integers(0, 9801, size=(3, 128))
    pref = O.build_marginal(samples, kv_dtype, 9500, 300)
    st = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, 8, channel_split=split)
    h = O.parse_header(st)
    assert h["channel_split"] == 1 and st[15] == 1
    assert np.array_equal(O.decode(st, mu, sig, pref, channel_split=split), kv)
    with pytest.raises(ValueError):                         # the split is needed
        O.decode(st, mu, sig, pref)
    other = split.copy()
    other[2, 100] ^= 1
    with pytest.raises(O.StreamError):                      # a different split: side hash
        O.decode(st, mu, sig, pref, channel_split=other)
    plain = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, 8)
    assert plain[15] == 0
    # a split where every channel has the call's weight codes the same chunks
    same = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, 8,
                    channel_split=np.full((3, 128), 9500))
    n = O.parse_header(plain)["n_chunks"]
    assert all(O.chunk_payload(same, c) == O.chunk_payload(plain, c) for c in range(n))


def test_split_flag_in_the_header():
    kv, mu, sig, samples, mu_dtype = case()
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    split = np.full((2, 128), 9000)
    st = O.encode(kv, mu, sig, pref, O.BF16, mu_dtype, 9500, 300, 16, channel_split=split)
    bad = bytearray(st)
    bad[15] = 0                                             # flag damaged: header checksum
    with pytest.raises(O.StreamError):
        O.parse_header(bytes(bad))
    bad[15] = 2                                             # an unknown value, checksum fixed
    bad[92:96] = O.crc32(bytes(bad[:92])).to_bytes(4, "little")
    with pytest.raises(O.StreamError, match="unsupported"):
        O.parse_header(bytes(bad))
    with pytest.raises(ValueError):                         # wrong shape of the split
        O.encode(kv, mu, sig, pref, O.BF16, mu_dtype, 9500, 300, 16, channel_split=split[:, :64])


def test_side_hash_with_a_split_by_hand():
    """Two sigma words and one split word, written out: the split words
    follow the sigma words in the tag-1 sequence."""
    sig = np.array([[1.0, 2.0]], dtype=np.float32)
    split = np.array([[9000, 7]])
    words = [0x3F800000, 0x40000000, 9000, 7]
    gold = 0x9E3779B97F4A7C15
    mask = (1 << 64) - 1

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        return z ^ (z >> 31)
    ref = sum(mix((((i << 32) | w) + gold) & mask) for i, w in enumerate(words)) & mask
    assert O.side_hash(sig, None, split) == ref
    assert O.side_hash(sig, None, None) != ref


@pytest.mark.parametrize("outlier_rate", [0.0, 0.04])
def test_calibration_matches_a_float64_brute_force(outlier_rate):
    """Per channel, the chosen weight's continuous code length is within the
    integer model's error of the best candidate's (float64 mixture mass per
    cell, each candidate as the call's weights of a one-channel model)."""
    reps, planes, tokens, channels = 2, 1, 48, 64
    rng = np.random.default_rng(21)
    import torch
    mu_f = torch.tensor(rng.normal(0, 1, (reps, planes, tokens, channels)), dtype=torch.float32)
    scale = torch.tensor(rng.uniform(0.02, 0.2, (1, 1, 1, channels)), dtype=torch.float32)
    res = torch.tensor(rng.normal(0, 1, mu_f.shape), dtype=torch.float32) * scale
    hit = torch.tensor(rng.random(mu_f.shape) < outlier_rate * (np.arange(channels) % 2))
    res = torch.where(hit, res * 12, res)
    kv = W.to_numpy_bits((mu_f + res).to(torch.bfloat16))
    mu = W.to_numpy_bits(mu_f.to(torch.bfloat16))
    sig = O.calibrate_sigma(kv, mu, O.BF16, O.BF16, 1e-3)
    pref = O.build_marginal(kv.reshape(-1), O.BF16, 9500, 300)
    pick, costs = O.calibrate_split(kv, mu, sig, pref, O.BF16, O.BF16, 9500, 300, return_costs=True)
    cands = O.split_candidates(9500, 300)
    assert pick.shape == (planes, channels) and np.all(np.isin(pick, cands))
    n_sym = reps * tokens
    for c in range(channels):
        fl = []
        for v in cands:
            bits = 0.0
            for r in range(reps):
                sl = (slice(0, 1), slice(None), slice(c, c + 1))
                bits += O.model_bits_float(kv[r][sl], mu[r][sl], sig[:, c:c + 1], pref, O.BF16, O.BF16,
                                           int(v), 9800 - int(v)) * tokens
            fl.append(bits)
        fl = np.array(fl)
        got = fl[list(cands).index(pick[0, c])]
        # code_len_q16 reads high by < 0.0056 bits, the integer model differs
        # from the float one by far less than 0.01 bits per symbol
        assert got <= fl.min() + 2 * 0.016 * n_sym, (c, got, fl.min())
        # and the integer costs are the code lengths of that channel alone
        assert costs[:, 0, c].argmin() == list(cands).index(pick[0, c])
    # a channel with outliers moves weight to the wide part; a clean one keeps it narrow
    if outlier_rate:
        assert np.mean(pick[0, 1::2]) < np.mean(pick[0, 0::2])
