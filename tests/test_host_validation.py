"""The C ABI's host-side checks, called with no GPU: every entry point
refuses bad arguments, damaged or mismatched headers and buffers smaller
than the header describes, with the status its declaration states, before
it touches the device.  Device pointers here are stand-in addresses that the
host code must never dereference (only their alignment and whether they are
null are looked at), so the module stays off machines with a GPU: there a
check that wrongly passed would launch on them.  The same tests run under
the sanitizer build (test_host_sanitizers.py)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="stand-in device pointers: host-only checks, kept off GPUs")

FAKE = 1 << 40                 # a 256-byte-aligned stand-in device address, never dereferenced
W_MIX = (9500, 300)


@pytest.fixture(scope="module")
def case():
    """A small oracle stream (bf16, mixture, ragged chunks) and its sizes."""
    kv, mu, sig, samples = W.tiny_case(11, planes=2, tokens=40)
    kvn, mun, sgn, smn = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(smn, O.BF16, *W_MIX)
    st = O.encode(kvn, mun, sgn, pref, O.BF16, O.BF16, *W_MIX, 16)
    n = kv.numel()
    return dict(stream=np.frombuffer(st, dtype=np.uint8).copy(), n=n, planes=2, tokens=40, channels=128,
                mu_bytes=2 * n, sigma_bytes=4 * 2 * 128, prefix_bytes=4 * 65537, kv_bytes=2 * n)


def _decode(kvc, c, header=None, in_bytes=None, d_in=FAKE, mu_bytes=None, sigma_bytes=None, prefix=FAKE,
            prefix_bytes=None, kv_out=FAKE, kv_bytes=None, ws=FAKE, ws_bytes=None, fn="decode"):
    h = c["stream"] if header is None else header
    args = [h.ctypes.data if h is not False else None, d_in,
            len(c["stream"]) if in_bytes is None else in_bytes,
            FAKE, c["mu_bytes"] if mu_bytes is None else mu_bytes,
            FAKE, c["sigma_bytes"] if sigma_bytes is None else sigma_bytes,
            prefix, c["prefix_bytes"] if prefix_bytes is None else prefix_bytes,
            kv_out, c["kv_bytes"] if kv_bytes is None else kv_bytes,
            ws, kvc.DECODE_WORKSPACE_BYTES if ws_bytes is None else ws_bytes, None]
    if fn == "decode":
        return kvc._lib_decode(*args, None)
    return kvc._lib_decode_async(*args)


def test_decode_refuses_bad_arguments_before_the_device(kvc, case):
    c = case
    assert _decode(kvc, c, header=False) == kvc.KVC_ERR_INVALID
    assert _decode(kvc, c, d_in=None) == kvc.KVC_ERR_INVALID
    assert _decode(kvc, c, kv_out=None) == kvc.KVC_ERR_INVALID
    assert _decode(kvc, c, d_in=FAKE + 4) == kvc.KVC_ERR_INVALID          # stream not 8-byte aligned
    assert _decode(kvc, c, ws=FAKE + 128) == kvc.KVC_ERR_INVALID         # workspace not 256-byte aligned
    assert _decode(kvc, c, ws_bytes=kvc.DECODE_WORKSPACE_BYTES - 1) == kvc.KVC_ERR_CAPACITY
    assert _decode(kvc, c, in_bytes=len(c["stream"]) - 8) == kvc.KVC_ERR_CORRUPT
    assert _decode(kvc, c, in_bytes=len(c["stream"]) + 8) == kvc.KVC_ERR_CORRUPT
    assert _decode(kvc, c, in_bytes=64) == kvc.KVC_ERR_CORRUPT
    assert _decode(kvc, c, mu_bytes=c["mu_bytes"] - 2) == kvc.KVC_ERR_INVALID
    assert _decode(kvc, c, sigma_bytes=c["sigma_bytes"] - 4) == kvc.KVC_ERR_INVALID
    assert _decode(kvc, c, prefix=None) == kvc.KVC_ERR_INVALID           # the mixture has an escape part
    assert _decode(kvc, c, prefix_bytes=c["prefix_bytes"] - 4) == kvc.KVC_ERR_INVALID
    assert _decode(kvc, c, kv_bytes=c["kv_bytes"] - 2) == kvc.KVC_ERR_INVALID
    for fn in ("decode", "async"):
        assert _decode(kvc, c, mu_bytes=0, fn=fn) == kvc.KVC_ERR_INVALID


@pytest.mark.parametrize("offset", [0, 4, 8, 9, 14, 15, 24, 40, 48, 64, 72, 80, 88, 92, 100, 127])
def test_decode_refuses_a_damaged_header(kvc, case, offset):
    h = case["stream"][:128].copy()
    h[offset] ^= 0x01
    assert _decode(kvc, case, header=h) == kvc.KVC_ERR_CORRUPT


def test_decode_refuses_a_header_with_a_recomputed_crc_but_bad_fields(kvc, case):
    import zlib
    for off, val in [(8, 7), (9, 1), (14, 17), (15, 2), (13, 32)]:
        h = case["stream"][:128].copy()
        h[off] = val
        h[92:96] = np.frombuffer(zlib.crc32(h[:92].tobytes()).to_bytes(4, "little"), dtype=np.uint8)
        assert _decode(kvc, case, header=h) == kvc.KVC_ERR_CORRUPT, off


def test_decode_of_a_split_stream_needs_the_weights_in_the_side_buffer(kvc, case):
    """A stream with per-channel weights: the side buffer holds sigma, then
    planes x channels weights; a buffer that holds sigma alone is refused."""
    kv, mu, sig, samples = W.tiny_case(11, planes=2, tokens=40)
    kvn, mun, sgn, smn = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(smn, O.BF16, *W_MIX)
    split = np.full((2, 128), 9000)
    st = O.encode(kvn, mun, sgn, pref, O.BF16, O.BF16, *W_MIX, 16, channel_split=split)
    c = dict(case, stream=np.frombuffer(st, dtype=np.uint8).copy())
    assert _decode(kvc, c) == kvc.KVC_ERR_INVALID                         # sigma words only
    assert _decode(kvc, c, sigma_bytes=c["sigma_bytes"] + 4 * 256 - 4) == kvc.KVC_ERR_INVALID
    p, total = kvc.kvc_stream_info(st[:128])
    assert p.channel_split == 1 and total == len(st)


def _paged(kvc, c, **kw):
    p = kvc.kvc_paged_kv(d_pools=FAKE, d_block_table=FAKE, n_pools=2, pool_bytes=8 * 8 * 128 * 2 * 100,
                         batch=1, heads=1, max_pages=5, num_pages=100, page_tokens=8, reserved=0)
    for k, v in kw.items():
        setattr(p, k, v)
    return kvc._lib_decode_paged(c["stream"].ctypes.data, FAKE, len(c["stream"]), FAKE, c["mu_bytes"], FAKE,
                                 c["sigma_bytes"], FAKE, c["prefix_bytes"], ctypes.byref(p), FAKE,
                                 kvc.DECODE_WORKSPACE_BYTES, None, None)


def test_paged_decode_refuses_a_descriptor_that_does_not_match(kvc, case):
    # the 2 planes are (layer 0, K and V) of batch 1 x 1 head: two pools of 8-token pages of 1 x 128 channels
    bad = [dict(n_pools=1), dict(n_pools=3), dict(pool_bytes=8 * 128 * 2 * 100 - 1), dict(page_tokens=0),
           dict(max_pages=4), dict(batch=0), dict(heads=2), dict(num_pages=0), dict(reserved=1),
           dict(d_pools=None), dict(d_block_table=None), dict(d_pools=FAKE + 4), dict(d_block_table=FAKE + 2)]
    for kw in bad:
        assert _paged(kvc, case, **kw) == kvc.KVC_ERR_INVALID, kw
    assert kvc._lib_decode_paged(case["stream"].ctypes.data, FAKE, len(case["stream"]), FAKE, case["mu_bytes"],
                                 FAKE, case["sigma_bytes"], FAKE, case["prefix_bytes"], None, FAKE,
                                 kvc.DECODE_WORKSPACE_BYTES, None, None) == kvc.KVC_ERR_INVALID


def _reload(kvc, c, streams, mu_stride=None, staging_bytes=None, ws_bytes=None, n=None, failed=True):
    arr = [s.ctypes.data for s in streams]
    ptrs = (ctypes.c_void_p * len(arr))(*arr)
    sizes = (ctypes.c_uint64 * len(arr))(*[len(s) for s in streams])
    n = len(streams) if n is None else n
    f = ctypes.c_int64(7)
    st = kvc._lib_reload(n, ptrs, sizes, FAKE, c["mu_bytes"] if mu_stride is None else mu_stride, FAKE,
                         c["sigma_bytes"], FAKE, c["prefix_bytes"], FAKE, c["kv_bytes"], FAKE,
                         1 << 20 if staging_bytes is None else staging_bytes, FAKE,
                         kvc.DECODE_WORKSPACE_BYTES * max(n, 1) if ws_bytes is None else ws_bytes, None, None,
                         ctypes.byref(f) if failed else None)
    return st, f.value


def test_reload_checks_every_layer_before_copying(kvc, case):
    good = case["stream"]
    damaged = good.copy()
    damaged[50] ^= 0x10                                   # a header byte: the CRC no longer matches
    short = good[:-8].copy()                              # a truncated stream
    assert _reload(kvc, case, [good, damaged, good]) == (kvc.KVC_ERR_CORRUPT, 1)
    assert _reload(kvc, case, [good, good, short]) == (kvc.KVC_ERR_CORRUPT, 2)
    assert _reload(kvc, case, [good, good], mu_stride=case["mu_bytes"] - 2) == (kvc.KVC_ERR_INVALID, 0)
    assert _reload(kvc, case, [good, good], staging_bytes=2 * 256) == (kvc.KVC_ERR_CAPACITY, 0)
    assert _reload(kvc, case, [good, good], ws_bytes=kvc.DECODE_WORKSPACE_BYTES)[0] == kvc.KVC_ERR_CAPACITY
    assert _reload(kvc, case, [good], n=0)[0] == kvc.KVC_ERR_INVALID
    assert _reload(kvc, case, [good, damaged], failed=False)[0] == kvc.KVC_ERR_CORRUPT


def test_encode_refuses_bad_arguments_before_the_device(kvc):
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 2, 40, 128, W_MIX, 16)
    _, ws = kvc.kvc_encode_sizes(p)
    out = ctypes.c_uint64(0)
    hdr = np.zeros(128, dtype=np.uint8)

    def enc(q=p, kv=FAKE, prefix=FAKE, out_bytes=True, header=None, wsp=FAKE, ws_bytes=ws):
        return kvc._lib_encode(ctypes.byref(q), kv, FAKE, FAKE, prefix, FAKE, 1 << 20,
                               ctypes.byref(out) if out_bytes else None, header, wsp, ws_bytes, None, None)
    assert enc(kv=None) == kvc.KVC_ERR_INVALID
    assert enc(prefix=None) == kvc.KVC_ERR_INVALID                         # mixture without its prefix
    assert enc(out_bytes=False, header=hdr.ctypes.data) == kvc.KVC_ERR_INVALID   # host output needs the sync
    assert enc(ws_bytes=ws - 1) == kvc.KVC_ERR_CAPACITY
    assert enc(wsp=FAKE + 64) == kvc.KVC_ERR_INVALID
    q = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 2, 40, 96, W_MIX, 16)   # channels not a multiple of 64
    assert enc(q=q) == kvc.KVC_ERR_INVALID
    q = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 2, 40, 128, W_MIX, 16)
    q.narrow_dof = 17
    assert enc(q=q) == kvc.KVC_ERR_INVALID
    q = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 2, 40, 128, W_MIX, 16, channel_split=2)
    assert enc(q=q) == kvc.KVC_ERR_INVALID
    assert kvc._lib_encode_sizes(ctypes.byref(q), None, None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_encode_result(None, None, ctypes.byref(out), None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_encode_result(FAKE + 8, None, ctypes.byref(out), None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_decode_result(FAKE + 8, None, None) == kvc.KVC_ERR_INVALID


def test_other_calls_refuse_bad_arguments(kvc):
    f = ctypes.c_float(2.0 ** -30)
    # calibration: 64-channel groups, positive sizes, an accepted floor
    assert kvc._lib_calibrate(FAKE, FAKE, kvc.KVC_BF16, kvc.KVC_BF16, 1, 1, 16, 96, f, FAKE, FAKE, 1 << 20,
                              None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_calibrate(FAKE, FAKE, 5, kvc.KVC_BF16, 1, 1, 16, 128, f, FAKE, FAKE, 1 << 20,
                              None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_calibrate_blocks(FAKE, FAKE, kvc.KVC_BF16, kvc.KVC_BF16, 1, 1, 16, 128, -1, f, FAKE, FAKE,
                                     1 << 20, None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_calibrate_rate(FAKE, FAKE, kvc.KVC_BF16, kvc.KVC_BF16, 1, 1, 16, 128, 0, f, 9500, 300, 17,
                                   FAKE, FAKE, FAKE, 1 << 20, None) == kvc.KVC_ERR_INVALID
    # per-channel split: 64-channel groups, positive sizes, known dtypes, a
    # prefix with an escape part, a workspace of the stated size
    ws = 2 * 128 * 8192

    def split(**kw):
        a = dict(kv=FAKE, mu=FAKE, kvd=kvc.KVC_BF16, mud=kvc.KVC_BF16, reps=1, planes=2, tokens=16, channels=128,
                 block=0, sigma=FAKE, wn=9500, ww=300, dof=0, prefix=FAKE, out=FAKE, wsp=FAKE, ws_bytes=ws)
        a.update(kw)
        return kvc._lib_calibrate_split(a["kv"], a["mu"], a["kvd"], a["mud"], a["reps"], a["planes"], a["tokens"],
                                        a["channels"], a["block"], a["sigma"], a["wn"], a["ww"], a["dof"],
                                        a["prefix"], a["out"], a["wsp"], a["ws_bytes"], None)
    for kw in (dict(channels=96), dict(reps=0), dict(tokens=0), dict(planes=0), dict(block=-1), dict(dof=17),
               dict(kvd=5), dict(mud=1), dict(wn=9800, ww=300), dict(prefix=None), dict(sigma=None),
               dict(out=None), dict(out=FAKE + 2), dict(wsp=FAKE + 64), dict(ws_bytes=ws - 1),
               dict(planes=1 << 26, tokens=1, ws_bytes=1 << 62)):               # the workspace formula would overflow
        assert split(**kw) == kvc.KVC_ERR_INVALID, kw
    # marginal: a known dtype, weights within 10000 basis points
    assert kvc._lib_marginal(FAKE, 3, 10, 9500, 300, FAKE, None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_marginal(FAKE, kvc.KVC_BF16, 10, 9500, 600, FAKE, None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_marginal(None, kvc.KVC_BF16, 10, 9500, 300, FAKE, None) == kvc.KVC_ERR_INVALID
    # CDF table: pairs in [1, 2^24], narrow part up to 16 degrees of freedom
    assert kvc._lib_cdf_table(kvc.KVC_BF16, kvc.KVC_BF16, 9500, 300, 0, FAKE, FAKE, 0, FAKE, FAKE,
                              None) == kvc.KVC_ERR_INVALID
    assert kvc._lib_cdf_table(kvc.KVC_BF16, kvc.KVC_BF16, 9500, 300, 17, FAKE, FAKE, 1, FAKE, FAKE,
                              None) == kvc.KVC_ERR_INVALID
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 2, 40, 128, W_MIX, 16)
    bits = (ctypes.c_double * 2)()
    assert kvc._lib_estimate(ctypes.byref(p), FAKE, FAKE, FAKE, None, bits, FAKE, 1 << 20,
                             None) == kvc.KVC_ERR_INVALID                     # mixture without its prefix
    assert kvc._lib_estimate(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, bits, FAKE, 8,
                             None) == kvc.KVC_ERR_CAPACITY
    assert kvc._lib_narrow_table(17, bits) == kvc.KVC_ERR_INVALID
    assert kvc._lib_phi_tables(None, None) == kvc.KVC_ERR_INVALID
