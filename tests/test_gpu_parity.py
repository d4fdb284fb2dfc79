"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer and byte results must match bit for bit: CDF tables, whole streams,
chunk payloads, decoded KV, marginal prefixes.  sigma (float64 sums rounded
once to float32) may differ by one float32 ulp; bits estimates by 1e-9
(integer model) and 1e-3 (float model) per the method's own tolerance.
"""
import hashlib
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bits(x: np.ndarray, dev):
    """Host patterns -> device tensor the binding accepts."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def dev_prefix(pref, dev):
    return None if pref is None else torch.from_numpy(np.asarray(pref, dtype=np.int64).astype(np.int32)).to(dev)


def host_bytes(t: torch.Tensor) -> bytes:
    return t.cpu().numpy().tobytes()


def tiny(kv_dtype, seed=7, planes=3, tokens=45, channels=128):
    kv, mu, sig, samples = W.tiny_case(seed, planes, tokens, channels, kv_dtype)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    return (W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples), mu_dtype)


# ---------------------------------------------------------------------------
# the CDF
# ---------------------------------------------------------------------------
def adversarial_pairs(rng, n_random):
    # the last four put z * 2^24 at subnormal magnitudes of either sign for the edges next to mu
    # (floor of a negative subnormal is -1)
    mus = [0.0, -0.0, 1e-40, -1e-40, 3.0e38, -3.0e38, 1.5, -2.75, 0.001, 1e4, np.nan, np.inf, -np.inf,
           0.998046875, 448.0, -448.0, 0.0, 2.0 ** -133, 0.5 * (1 + 2 ** -8),
           2.0 ** -60, -2.0 ** -60, 1e-20, -3e-20]
    sig = [1e-3, 2.0 ** -30, 2.0 ** -30, 2.0 ** -96, 1.0, 2.0 ** 96, 2.0 ** -4, 0.37, 10.0, 2.0 ** -7, 0.5, 0.5, 0.5,
           2.0 ** -12, 2.0, 0.01, 1e4, 2.0 ** -20, 2.0 ** -9,
           2.0 ** 96, 2.0 ** 96, 2.0 ** 96, 2.0 ** 90]
    m = np.concatenate([np.float32(mus), (rng.standard_normal(n_random) * np.exp(rng.normal(0, 2, n_random))).astype(np.float32)])
    s = np.concatenate([np.float32(sig), np.exp2(rng.uniform(-30, 8, n_random)).astype(np.float32)])
    return m.astype(np.float32), s.astype(np.float32)


@pytest.mark.parametrize("kv_dtype,n_random", [(O.E4M3, 2000), (O.BF16, 40)])
@pytest.mark.parametrize("w", [(10000, 0), (9500, 300)])
def test_cdf_table_matches_oracle(kvc, cuda, kv_dtype, n_random, w):
    rng = np.random.default_rng(100 + kv_dtype)
    mus, sig = adversarial_pairs(rng, n_random)
    samples = rng.standard_normal(30000).astype(np.float32)
    bits = torch.from_numpy(samples)
    bits = W.to_numpy_bits(bits.to(torch.bfloat16)) if kv_dtype == O.BF16 else \
        W.to_numpy_bits(bits.to(torch.float8_e4m3fn).view(torch.uint8))
    pref = O.build_marginal(bits, kv_dtype, *w) if w[1] else None
    expect = O.cdf_table(mus, sig, kv_dtype, O.F32, *w, prefix=pref)
    got = kvc.kvc_cdf_table(kv_dtype, torch.from_numpy(mus).to(cuda), torch.from_numpy(sig).to(cuda),
                            dev_prefix(pref, cuda), w).cpu().numpy().view(np.uint32).astype(np.int64)
    bad = np.argwhere(got != expect)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], expect[tuple(bad[0])])


def test_cdf_table_bf16_mu(kvc, cuda):
    rng = np.random.default_rng(5)
    mu_f = (rng.standard_normal(64) * 3).astype(np.float32)
    mu_b = W.to_numpy_bits(torch.from_numpy(mu_f).to(torch.bfloat16))
    sig = np.exp2(rng.uniform(-12, 2, 64)).astype(np.float32)
    expect = O.cdf_table(mu_b, sig, O.BF16, O.BF16, 10000, 0)
    got = kvc.kvc_cdf_table(kvc.KVC_BF16, dev_bits(mu_b, cuda), torch.from_numpy(sig).to(cuda), None,
                            (10000, 0)).cpu().numpy().view(np.uint32).astype(np.int64)
    assert np.array_equal(got, expect)


def test_cdf_table_rejects_bad_sigma(kvc, cuda):
    for bad in [0.0, -1.0, float("inf"), float("nan"), 1e-45, 1e-30, 1e30]:
        with pytest.raises(kvc.KvcError) as e:
            kvc.kvc_cdf_table(kvc.KVC_E4M3, torch.zeros(2, device=cuda), torch.tensor([1.0, bad], device=cuda),
                              None, (10000, 0))
        assert e.value.status == kvc.KVC_ERR_INVALID


# ---------------------------------------------------------------------------
# whole streams on small irregular cases
# ---------------------------------------------------------------------------
CASES = [
    (O.BF16, (9500, 300), 16, 3, 45, 128),
    (O.BF16, (10000, 0), 64, 3, 45, 128),
    (O.BF16, (9500, 300), 1, 2, 9, 128),
    (O.BF16, (7000, 2000), 7, 2, 45, 192),
    (O.BF16, (9500, 300), 1024, 2, 1, 64),
    (O.E4M3, (9500, 300), 7, 3, 45, 128),
    (O.E4M3, (10000, 0), 16, 2, 33, 64),
]


@pytest.mark.parametrize("kv_dtype,w,tc,g,t,d", CASES)
def test_stream_matches_oracle_and_round_trips(kvc, cuda, kv_dtype, w, tc, g, t, d):
    kv, mu, sig, samples, mu_dtype = tiny(kv_dtype, planes=g, tokens=t, channels=d)
    pref = O.build_marginal(samples, kv_dtype, *w) if w[0] + w[1] < 10000 else None
    expect = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, *w, tc)
    kv_d, mu_d, sig_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda), dev_prefix(pref, cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, w, tc)
    got = host_bytes(st)
    assert len(got) == len(expect)
    if got != expect:
        diff = np.flatnonzero(np.frombuffer(got, np.uint8) != np.frombuffer(expect, np.uint8))
        pytest.fail(f"stream differs at {diff[:8]} of {len(got)}")
    out = kvc.kvc_decode(st, mu_d, sig_d, pref_d)
    assert np.array_equal(out.cpu().numpy().view(kv.dtype), kv)
    # the decoder also reads the oracle's own stream
    out2 = kvc.kvc_decode(torch.from_numpy(np.frombuffer(expect, np.uint8).copy()).to(cuda), mu_d, sig_d, pref_d)
    assert np.array_equal(out2.cpu().numpy().view(kv.dtype), kv)


@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
@pytest.mark.parametrize("w", [(0, 0), (0, 10000), (5000, 0), (9999, 0)])
@pytest.mark.parametrize("marg", ["data", "peaked"])
def test_escape_heavy_and_escape_free_mixtures(kvc, cuda, kv_dtype, w, marg):
    """Weights that put every slot in the floor-and-escape range (0, 0), none
    there but the floor (0, 10000), half of them (5000, 0) or a sliver
    (9999, 0), with the marginal of the data or one concentrated on a single
    symbol: streams identical to the oracle's, and they decode."""
    kv, mu, sig, samples, mu_dtype = tiny(kv_dtype, planes=2, tokens=40, channels=128)
    if marg == "peaked":
        samples = np.full_like(samples, samples[0])
    pref = O.build_marginal(samples, kv_dtype, *w) if w[0] + w[1] < 10000 else None
    expect = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, *w, 16)
    kv_d, mu_d, sig_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda), dev_prefix(pref, cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, w, 16)
    assert host_bytes(st) == expect
    out = kvc.kvc_decode(st, mu_d, sig_d, pref_d)
    assert np.array_equal(out.cpu().numpy().view(kv.dtype), kv)


def test_golden_streams(kvc, cuda):
    with open(os.path.join(ROOT, "tests", "golden", "tiny_streams.txt")) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for name, kv_dtype, w_n, w_w, tc, size, digest in lines:
        kv_dtype, w_n, w_w, tc = int(kv_dtype), int(w_n), int(w_w), int(tc)
        kv, mu, sig, samples, mu_dtype = tiny(kv_dtype)
        pref = O.build_marginal(samples, kv_dtype, w_n, w_w)
        st = kvc.kvc_encode(dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda),
                            dev_prefix(pref, cuda), (w_n, w_w), tc)
        b = host_bytes(st)
        assert len(b) == int(size) and hashlib.sha256(b).hexdigest() == digest, name


# ---------------------------------------------------------------------------
# the tiny workload in full: single and mixture
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def cfg0(cuda):
    w = W.WORKLOADS[0]
    kv, mu = W.layer_data(w, 0, device=cuda)
    sig = W.layer_sigma_true(w, 0, device=cuda)
    samples = W.marginal_samples(w, device=cuda)
    return w, kv, mu, sig, samples


@pytest.mark.parametrize("weights", [(10000, 0), (9500, 300)])
def test_tiny_workload_full_parity(kvc, cfg0, weights):
    w, kv, mu, sig, samples = cfg0
    kvn, mun, sgn = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.cpu().numpy()
    pref = O.build_marginal(W.to_numpy_bits(samples), O.BF16, *weights) if weights[1] else None
    pref_d = dev_prefix(pref, kv.device)
    st = kvc.kvc_encode(kv, mu, sig, pref_d, weights, w.chunk_tokens)
    expect = O.encode(kvn, mun, sgn, pref, O.BF16, O.BF16, *weights, w.chunk_tokens)
    assert host_bytes(st) == expect
    out = kvc.kvc_decode(st, mu, sig, pref_d)
    assert torch.equal(out, kv.view(torch.int16))
    assert np.array_equal(O.decode(expect, mun, sgn, pref), kvn)


def test_marginal_matches_oracle(kvc, cfg0, cuda):
    _, _, _, _, samples = cfg0
    for weights in [(9500, 300), (10000, 0), (5000, 0)]:
        got = kvc.kvc_build_marginal(samples, weights).cpu().numpy().astype(np.int64)
        assert np.array_equal(got, O.build_marginal(W.to_numpy_bits(samples), O.BF16, *weights))
    e = W.tiny_case(3, kv_dtype=O.E4M3)[3]
    got = kvc.kvc_build_marginal(e.to(cuda)).cpu().numpy().astype(np.int64)
    assert np.array_equal(got, O.build_marginal(W.to_numpy_bits(e), O.E4M3, 9500, 300))


def test_estimate_bits_matches_oracle(kvc, cfg0):
    w, kv, mu, sig, samples = cfg0
    kvn, mun, sgn = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.cpu().numpy()
    for weights in [(10000, 0), (9500, 300)]:
        pref = O.build_marginal(W.to_numpy_bits(samples), O.BF16, *weights) if weights[1] else None
        bi, bf = kvc.kvc_estimate_bits(kv, mu, sig, dev_prefix(pref, kv.device), weights)
        ei = O.model_bits_int(kvn, mun, sgn, pref, O.BF16, O.BF16, *weights)
        ef = O.model_bits_float(kvn, mun, sgn, pref, O.BF16, O.BF16, *weights)
        say(f"bits weights={weights}: int gpu {bi:.9f} oracle {ei:.9f}; float gpu {bf:.9f} oracle {ef:.9f}")
        assert abs(bi - ei) <= 1e-9 * ei
        assert abs(bf - ef) <= 1e-3


def test_calibrate_matches_oracle(kvc, cuda):
    w = W.WORKLOADS[1]
    kv, mu = W.layer_calibration(w, 3, reps=8, device=cuda)
    got = kvc.kvc_calibrate_sigma(kv, mu).cpu().numpy()
    expect = O.calibrate_sigma(W.to_numpy_bits(kv), W.to_numpy_bits(mu), O.BF16, O.BF16, 2.0 ** -30)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - expect.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1 and np.mean(ulp == 0) > 0.99
    # e4m3 KV with float32 mu, and non-finite residuals skipped
    w3 = W.WORKLOADS[3]
    kv3, mu3 = W.layer_calibration(w3, 0, reps=2, device=cuda, tokens=256)
    mu3[0, 0, 0, :5] = float("nan")
    kv3[1, 1, 3, 7] = 0x7F
    got3 = kvc.kvc_calibrate_sigma(kv3, mu3).cpu().numpy()
    exp3 = O.calibrate_sigma(W.to_numpy_bits(kv3), mu3.cpu().numpy(), O.E4M3, O.F32, 2.0 ** -30)
    ulp3 = np.abs(got3.view(np.int32).astype(np.int64) - exp3.view(np.int32).astype(np.int64))
    assert ulp3.max() <= 1


@pytest.mark.parametrize("reps,planes,tokens,channels", [
    (1, 1, 1, 64),          # one row: one split
    (3, 2, 1, 128),         # rows step over several reps at once (tokens < waves per block)
    (5, 3, 3, 64),          # 15 rows in 15 splits, ragged carries
    (7, 1, 333, 192),       # many splits of uneven length, three channel groups
])
def test_calibrate_odd_shapes(kvc, cuda, reps, planes, tokens, channels):
    g = torch.Generator(device="cpu").manual_seed(reps * 1000 + tokens)
    mu = (torch.randn((reps, planes, tokens, channels), generator=g) * 0.5).to(torch.bfloat16)
    kv = (mu.float() + 0.05 * torch.randn(mu.shape, generator=g)).to(torch.bfloat16)
    got = kvc.kvc_calibrate_sigma(kv.to(cuda), mu.to(cuda)).cpu().numpy()
    expect = O.calibrate_sigma(W.to_numpy_bits(kv), W.to_numpy_bits(mu), O.BF16, O.BF16, 2.0 ** -30)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - expect.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1


def test_calibrate_rejects_short_workspace(kvc, cuda):
    kv = torch.zeros((2, 3, 8, 64), dtype=torch.bfloat16, device=cuda)
    ws = torch.empty(kvc.calibrate_workspace_bytes(3, 64) - 1, dtype=torch.uint8, device=cuda)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_calibrate_sigma(kv, kv, workspace=ws)
    assert e.value.status == kvc.KVC_ERR_INVALID


# ---------------------------------------------------------------------------
# error paths
# ---------------------------------------------------------------------------
def test_error_statuses(kvc, cuda):
    kv, mu, sig, samples, mu_dtype = tiny(O.BF16)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    kv_d, mu_d, sig_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda), dev_prefix(pref, cuda)
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, (9500, 300), 16)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    out = torch.empty(kv.shape, dtype=torch.int16, device=cuda)

    def dec(stream, s=sig_d, p=pref_d):
        return kvc.kvc_decode_into(stream, mu_d, s, p, out, ws)

    assert dec(st) == kvc.KVC_OK
    # wrong side information
    s2 = sig_d.clone()
    s2[0, 0] = torch.nextafter(s2[0, 0], torch.tensor(1.0, device=cuda))
    assert dec(st, s=s2) == kvc.KVC_ERR_MISMATCH
    p2 = pref_d.clone()
    p2[1000] += 1
    assert dec(st, p=p2) == kvc.KVC_ERR_MISMATCH
    # damaged payload, directory, header; truncation
    h = O.parse_header(host_bytes(st))
    pay = 128 + 8 * (h["n_chunks"] + 1)
    rng = np.random.default_rng(9)
    for _ in range(8):
        bad = st.clone()
        i = int(rng.integers(pay, st.numel()))
        bad[i] ^= 1 << int(rng.integers(0, 8))
        assert dec(bad) == kvc.KVC_ERR_CORRUPT
    bad = st.clone()
    bad[pay + 7] ^= 0x80                    # top bit of lane 0's state
    assert dec(bad) == kvc.KVC_ERR_CORRUPT
    bad = st.clone()
    bad[128 + 8 * 2] ^= 8
    assert dec(bad) == kvc.KVC_ERR_CORRUPT
    bad = st.clone()
    bad[0] ^= 1
    assert dec(bad) == kvc.KVC_ERR_CORRUPT
    assert dec(st[:-8]) == kvc.KVC_ERR_CORRUPT
    assert dec(st[:100]) == kvc.KVC_ERR_CORRUPT
    # bad sigma on encode
    for v in [0.0, float("nan"), float("inf"), -1.0, 1e-30, 1e30]:
        s3 = sig_d.clone()
        s3[1, 5] = v
        with pytest.raises(kvc.KvcError) as e:
            kvc.kvc_encode(kv_d, mu_d, s3, pref_d, (9500, 300), 16)
        assert e.value.status == kvc.KVC_ERR_INVALID
    # capacity too small, and the size it needed
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, *kv.shape, (9500, 300), 16)
    enc = kvc.Encoder(p, cuda, out_capacity=st.numel() - 1)
    with pytest.raises(kvc.KvcError) as e:
        enc(kv_d, mu_d, sig_d, pref_d)
    assert e.value.status == kvc.KVC_ERR_CAPACITY
    enc = kvc.Encoder(p, cuda, out_capacity=st.numel())
    assert torch.equal(enc(kv_d, mu_d, sig_d, pref_d), st)
    # missing prefix for a mixture
    with pytest.raises(kvc.KvcError):
        kvc.kvc_encode(kv_d, mu_d, sig_d, None, (9500, 300), 16)


def test_decode_checks_the_header_and_the_buffers(kvc, cuda):
    """kvc_decode takes the header from the host: it must be valid (CRC),
    its length must be the stream's, the device stream's header must equal
    it, and every caller buffer must hold what it describes; otherwise
    nothing runs (or nothing is decoded) and the status says why."""
    kv, mu, sig, samples, mu_dtype = tiny(O.BF16)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    kv_d, mu_d, sig_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda), dev_prefix(pref, cuda)
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, *kv.shape, (9500, 300), 16)
    enc = kvc.Encoder(p, cuda)
    st = enc(kv_d, mu_d, sig_d, pref_d).clone()
    head = enc.header.copy()
    assert head.tobytes() == host_bytes(st)[:128]
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    out = torch.empty(kv.shape, dtype=torch.int16, device=cuda)

    def dec(h=head, m=mu_d, s=sig_d, pr=pref_d, o=out, stream=st):
        o.fill_(0)
        return kvc.kvc_decode_into(stream, m, s, pr, o, ws, header=h)

    assert dec() == kvc.KVC_OK and torch.equal(out, kv_d)
    # header fields damaged on the host copy: refused by the CRC
    for off in (9, 48, 88):
        bad = head.copy()
        bad[off] ^= 1
        assert dec(h=bad) == kvc.KVC_ERR_CORRUPT
    # a valid header (CRC recomputed) that is not the device stream's
    import zlib
    other = head.copy()
    other[80] ^= 1                                        # the side-information checksum
    other[92:96] = np.frombuffer(zlib.crc32(other[:92].tobytes()).to_bytes(4, "little"), np.uint8)
    assert dec(h=other) == kvc.KVC_ERR_CORRUPT
    assert int(out.abs().sum()) == 0                      # nothing decoded
    # buffers shorter than the header describes
    assert dec(m=mu_d.flatten()[:-1]) == kvc.KVC_ERR_INVALID
    assert dec(s=sig_d.flatten()[:-1]) == kvc.KVC_ERR_INVALID
    assert dec(pr=pref_d[:-1]) == kvc.KVC_ERR_INVALID
    assert dec(o=out.flatten()[:-1]) == kvc.KVC_ERR_INVALID
    # a stream one word longer than its header says
    longer = torch.cat([st, torch.zeros(8, dtype=torch.uint8, device=cuda)])
    assert dec(stream=longer) == kvc.KVC_ERR_CORRUPT


def test_asynchronous_calls(kvc, cuda):
    """Encodes and decodes queued without waiting, their outcomes read
    afterwards, give what the synchronous calls give."""
    kv, mu, sig, samples, mu_dtype = tiny(O.BF16)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    kv_d, mu_d, sig_d, pref_d = dev_bits(kv, cuda), dev_bits(mu, cuda), torch.from_numpy(sig).to(cuda), dev_prefix(pref, cuda)
    want = kvc.kvc_encode(kv_d, mu_d, sig_d, pref_d, (9500, 300), 16)
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, *kv.shape, (9500, 300), 16)
    encs = [kvc.Encoder(p, cuda) for _ in range(2)]
    s2 = torch.cuda.Stream()
    encs[0].enqueue(kv_d, mu_d, sig_d, pref_d)
    with torch.cuda.stream(s2):
        encs[1].enqueue(kv_d, mu_d, sig_d, pref_d, stream=s2)
    a = encs[0].result()
    b = encs[1].result(stream=s2)
    assert torch.equal(a, want) and torch.equal(b, want)
    assert encs[1].header.tobytes() == host_bytes(want)[:128]
    ws = [torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda) for _ in range(2)]
    outs = [torch.empty(kv.shape, dtype=torch.int16, device=cuda) for _ in range(2)]
    for i in range(2):
        assert kvc.kvc_decode_async(want, mu_d, sig_d, pref_d, outs[i], ws[i], encs[0].header) == kvc.KVC_OK
    assert kvc.kvc_decode_result(ws[0]) == kvc.KVC_OK and kvc.kvc_decode_result(ws[1]) == kvc.KVC_OK
    assert torch.equal(outs[0], kv_d) and torch.equal(outs[1], kv_d)
    # a damaged stream queued asynchronously reports through the result call
    bad = want.clone()
    bad[-9] ^= 4
    assert kvc.kvc_decode_async(bad, mu_d, sig_d, pref_d, outs[0], ws[0], encs[0].header) == kvc.KVC_OK
    assert kvc.kvc_decode_result(ws[0]) == kvc.KVC_ERR_CORRUPT
