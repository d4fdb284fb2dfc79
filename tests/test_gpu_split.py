"""GPU parity of per-channel mixture weights (a per-(plane, channel) split of
the Gaussian weight between the narrow and the wide part, carried after
sigma in the side buffer): streams byte-identical to the oracle's for both
dtypes, sigma blocks and the Student-t narrow part; exact round trips
through the plain, allocation-free, paged and host-offload decoders; a
changed weight refused by the side-information check and a weight above
the Gaussian weight refused by the encoder; the bits estimates; the
calibration bit for bit; and a full-size layer checked on sampled chunks."""
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


def random_split(planes, channels, w_gauss, seed):
    """Weights over the whole range, with the two ends present."""
    rng = np.random.default_rng(seed)
    s = rng.integers(0, w_gauss + 1, size=(planes, channels))
    s[0, :3] = [0, w_gauss, w_gauss // 2]
    return s.astype(np.int64)


CASES = [
    # kv dtype, weights, chunk tokens, sigma block, narrow dof
    (O.BF16, (9500, 300), 16, 0, 0),
    (O.BF16, (8750, 625), 7, 14, 0),
    (O.BF16, (10000, 0), 16, 0, 0),
    (O.BF16, (9500, 300), 45, 0, 4),
    (O.E4M3, (9500, 300), 16, 0, 0),
    (O.E4M3, (7000, 2000), 9, 0, 3),
]


@pytest.mark.parametrize("kv_dtype,w,tc,block,dof", CASES)
def test_stream_matches_oracle_and_decodes(kvc, cuda, kv_dtype, w, tc, block, dof):
    say(f"case kv={kv_dtype} w={w} tc={tc} block={block} dof={dof}")
    planes, tokens, channels = 3, 45, 192
    kv, mu, sig, samples = case(kv_dtype, planes=planes, tokens=tokens, channels=channels)
    if block:
        sig = np.stack([sig * np.float32(1.5 ** j) for j in range(-(-tokens // block))], axis=1)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(samples, kv_dtype, *w) if w[0] + w[1] < 10000 else None
    split = random_split(planes, channels, w[0] + w[1], tc)
    want = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, *w, tc, sigma_block_tokens=block, narrow_dof=dof,
                    channel_split=split)
    pref_d = None if pref is None else torch.from_numpy(pref.astype(np.int32)).to(cuda)
    kv_d, mu_d, sig_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda)
    split_d = torch.from_numpy(split.astype(np.int32)).to(cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, w, tc, sigma_block_tokens=block, narrow_dof=dof,
                        channel_split=split_d)
    assert st.cpu().numpy().tobytes() == want
    side = kvc.side_info(sig_d, split_d)
    out = kvc.kvc_decode(st, mu_d, side, pref_d)
    assert torch.equal(out, kv_d.view(out.dtype))
    out2 = torch.zeros_like(out)
    assert kvc.kvc_decode_noalloc(st, mu_d, side, pref_d, out2) == kvc.KVC_OK
    assert torch.equal(out2, out)


def test_changed_or_missing_weights_are_refused(kvc, cuda):
    kv, mu, sig, samples = case(O.BF16, planes=2, tokens=40)
    kv_d, mu_d, sig_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda)
    pref_d = kvc.kvc_build_marginal(dev_bits(samples, cuda))
    split = torch.from_numpy(random_split(2, 128, 9800, 1).astype(np.int32)).to(cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, (9500, 300), 16, channel_split=split)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    out = torch.zeros(kv_d.shape, dtype=torch.int16, device=cuda)
    other = split.clone()
    other[1, 77] += 1
    assert kvc.kvc_decode_into(st, mu_d, kvc.side_info(sig_d, other), pref_d, out, ws) == kvc.KVC_ERR_MISMATCH
    assert not out.any()                                                      # nothing decoded
    # sigma alone: the side buffer is shorter than the header needs
    assert kvc.kvc_decode_into(st, mu_d, sig_d, pref_d, out, ws) == kvc.KVC_ERR_INVALID
    assert kvc.kvc_decode_into(st, mu_d, kvc.side_info(sig_d, split), pref_d, out, ws) == kvc.KVC_OK
    assert torch.equal(out, kv_d.view(torch.int16))
    # damaged payloads are reported, as without the weights
    h = O.parse_header(st.cpu().numpy().tobytes())
    pay = 128 + 8 * (h["n_chunks"] + 1)
    rng = np.random.default_rng(4)
    side = kvc.side_info(sig_d, split)
    for _ in range(8):
        bad = st.clone()
        i = int(rng.integers(pay, st.numel()))
        bad[i] ^= 1 << int(rng.integers(0, 8))
        assert kvc.kvc_decode_into(bad, mu_d, side, pref_d, out, ws) == kvc.KVC_ERR_CORRUPT
    # a stream without the split decoded with a side buffer that has it: the
    # extra words are outside the checksum's range, sigma decides
    plain = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, (9500, 300), 16)
    assert kvc.kvc_decode_into(plain, mu_d, kvc.side_info(sig_d, split), pref_d, out, ws) == kvc.KVC_OK


def test_weight_above_the_gaussian_weight_is_refused(kvc, cuda):
    kv, mu, sig, samples = case(O.BF16, planes=2, tokens=40)
    kv_d, mu_d, sig_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda)
    pref_d = kvc.kvc_build_marginal(dev_bits(samples, cuda))
    split = torch.full((2, 128), 9800, dtype=torch.int32, device=cuda)
    split[1, 5] = 9801
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, (9500, 300), 16, channel_split=split)
    assert e.value.status == kvc.KVC_ERR_INVALID
    with pytest.raises(kvc.KvcError):
        kvc.kvc_estimate_bits(kv_d, mu_d, sig_d, pref_d, channel_split=split)


@pytest.mark.parametrize("kv_dtype,tc,pt", [(O.BF16, 16, 8), (O.E4M3, 7, 5)])
def test_paged_decode_places_rows_as_the_oracle(kvc, cuda, kv_dtype, tc, pt):
    layers, batch, heads, t, d = 2, 2, 2, 45, 128
    g_n = layers * 2 * batch * heads
    kv, mu, sig, samples = case(kv_dtype, seed=23, planes=g_n, tokens=t, channels=d)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(samples, kv_dtype, 9500, 300)
    split = random_split(g_n, d, 9800, 5)
    st = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, tc, channel_split=split)
    max_pages = -(-t // pt) + 1
    num_pages = batch * max_pages + 3
    table = np.random.default_rng(pt).permutation(num_pages)[:batch * max_pages].reshape(batch, max_pages)
    table = table.astype(np.int32)
    fill = 0x5A5A if kv_dtype == O.BF16 else 0x5A
    want = O.scatter_to_pages(kv, batch, heads, table, pt, num_pages, fill=fill)
    dt = torch.int16 if kv_dtype == O.BF16 else torch.uint8
    pools = [torch.full((num_pages, pt, heads, d), fill, dtype=dt, device=cuda) for _ in range(layers * 2)]
    paged = kvc.PagedKV(pools, torch.from_numpy(table).to(cuda), pt)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    side = kvc.side_info(torch.from_numpy(sig).to(cuda), torch.from_numpy(split.astype(np.int32)).to(cuda))
    rc = kvc.kvc_decode_paged(torch.from_numpy(np.frombuffer(st, np.uint8).copy()).to(cuda), dev_bits(mu, cuda),
                              side, torch.from_numpy(pref.astype(np.int32)).to(cuda), paged, ws)
    assert rc == kvc.KVC_OK
    got = np.stack([p.cpu().numpy() for p in pools])
    if kv_dtype == O.BF16:
        got = got.view(np.uint16)
    assert np.array_equal(got, want)


def test_reload_decodes_split_layers(kvc, cuda):
    """Three layers, each with its own weights, through the host-offload
    reload: the side buffers are stacked per layer (sigma, then weights)."""
    w = W.WORKLOADS[1]
    layers = 3
    prefix = kvc.kvc_build_marginal(W.marginal_samples(w, device=cuda), (w.w_narrow_bp, w.w_wide_bp))
    kvs, mus, sides, host = [], [], [], []
    for l in range(layers):
        kv, mu = W.layer_data(w, l, device=cuda, tokens=256)
        ck, cm = W.layer_calibration(w, l, reps=2, device=cuda, tokens=256)
        sig_kvh = kvc.kvc_calibrate_sigma(ck, cm)
        split_kvh = kvc.kvc_calibrate_split(ck, cm, sig_kvh, prefix)
        sig, split = W.expand_sigma(w, sig_kvh), W.expand_sigma(w, split_kvh)
        st = kvc.kvc_encode(kv, mu, sig, prefix, (w.w_narrow_bp, w.w_wide_bp), 64, channel_split=split)
        h = torch.empty(st.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(st)
        kvs.append(kv)
        mus.append(mu)
        sides.append(kvc.side_info(sig, split))
        host.append(h)
    kv, mu, side = torch.stack(kvs), torch.stack(mus), torch.stack(sides)
    out = torch.zeros(kv.shape, dtype=torch.int16, device=cuda)
    st, failed = kvc.kvc_reload(host, mu, side, prefix, out)
    assert st == kvc.KVC_OK and failed == -1
    assert torch.equal(out, kv.view(torch.int16))


@pytest.mark.parametrize("kv_dtype,dof", [(O.BF16, 0), (O.E4M3, 0), (O.BF16, 5)])
def test_estimate_bits_match_oracle(kvc, cuda, kv_dtype, dof):
    kv, mu, sig, samples = case(kv_dtype, planes=2, tokens=64)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(samples, kv_dtype, 9500, 300)
    split = random_split(2, 128, 9800, 9)
    bi = O.model_bits_int(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, narrow_dof=dof, channel_split=split)
    bf = O.model_bits_float(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, narrow_dof=dof, channel_split=split)
    gi, gf = kvc.kvc_estimate_bits(dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda),
                                   torch.from_numpy(pref.astype(np.int32)).to(cuda), narrow_dof=dof,
                                   channel_split=torch.from_numpy(split.astype(np.int32)).to(cuda))
    assert abs(gi - bi) <= 1e-9 * bi and abs(gf - bf) < 1e-3


@pytest.mark.parametrize("kv_dtype,block,w,dof", [(O.BF16, 0, (9500, 300), 0), (O.BF16, 32, (9500, 300), 0),
                                                  (O.E4M3, 0, (9500, 300), 0), (O.BF16, 0, (10000, 0), 3)])
def test_calibration_matches_oracle(kvc, cuda, kv_dtype, block, w, dof):
    wl = W.WORKLOADS[2] if kv_dtype == O.BF16 else W.WORKLOADS[3]
    ck, cm = W.layer_calibration(wl, 0, reps=2, tokens=96)
    ck, cm = ck[:, :4].contiguous(), cm[:, :4].contiguous()
    pref = O.build_marginal(W.to_numpy_bits(W.marginal_samples(wl, 1 << 16)), kv_dtype, *w) \
        if w[0] + w[1] < 10000 else None
    pref_d = None if pref is None else torch.from_numpy(pref.astype(np.int32)).to(cuda)
    ckd, cmd = ck.to(cuda), cm.to(cuda)
    sig = kvc.kvc_calibrate_sigma(ckd, cmd, block_tokens=block)
    got = kvc.kvc_calibrate_split(ckd, cmd, sig, pref_d, w, block_tokens=block, narrow_dof=dof)
    want = O.calibrate_split(W.to_numpy_bits(ck), W.to_numpy_bits(cm), sig.cpu().numpy(), pref, kv_dtype,
                             wl.mu_dtype, *w, sigma_block_tokens=block, narrow_dof=dof)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), want)


def test_full_size_layer_on_sampled_chunks(kvc, cuda):
    """One layer of the Qwen3-8B-shaped cache (64 planes x 4096 tokens x 128
    channels) at the library's default chunk length, weights calibrated on
    held-out draws: sampled chunks byte-identical to the oracle's, the whole
    layer decoded exactly, and the bits against the same layer without the
    split."""
    w = W.WORKLOADS[2]
    wts = (w.w_narrow_bp, w.w_wide_bp)
    kv, mu = W.layer_data(w, 0, device=cuda)
    ck, cm = W.layer_calibration(w, 0, reps=8, device=cuda)
    prefix = kvc.kvc_build_marginal(W.marginal_samples(w, device=cuda), wts)
    sig_kvh = kvc.kvc_calibrate_sigma(ck, cm)
    split_kvh = kvc.kvc_calibrate_split(ck, cm, sig_kvh, prefix, wts)
    sig, split = W.expand_sigma(w, sig_kvh), W.expand_sigma(w, split_kvh)
    st = kvc.kvc_encode(kv, mu, sig, prefix, wts, 0, channel_split=split)
    plain = kvc.kvc_encode(kv, mu, sig, prefix, wts, 0)
    say(f"layer: split {st.numel()} bytes, without {plain.numel()} bytes; "
        f"weights used {sorted(set(split_kvh.cpu().numpy().ravel().tolist()))}")
    host = st.cpu().numpy().tobytes()
    h = O.parse_header(host)
    assert h["channel_split"] == 1
    rng = np.random.default_rng(2)
    ids = sorted(set([0, h["n_chunks"] - 1] + rng.integers(0, h["n_chunks"], 10).tolist()))
    kvn, mun = W.to_numpy_bits(kv), W.to_numpy_bits(mu)
    want = O.encode_chunks(kvn, mun, sig.cpu().numpy(), prefix.cpu().numpy().astype(np.int64), O.BF16, O.BF16,
                           *wts, h["chunk_tokens"], ids, channel_split=split.cpu().numpy().astype(np.int64))
    for c in ids:
        assert O.chunk_payload(host, c) == want[c], c
    out = kvc.kvc_decode(st, mu, kvc.side_info(sig, split), prefix)
    assert torch.equal(out, kv.view(torch.int16))
