"""The C ABI library without a GPU: it loads, exports every call declared
in include/kvc.h, and its host-side logic (Phi table, sizes, header
parsing, argument validation) behaves."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from entropy_coding_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_calls():
    with open(os.path.join(ROOT, "include", "kvc.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(kvc_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_call_is_exported(kvc):
    names = declared_calls()
    assert len(names) >= 11
    lib = ctypes.CDLL(kvc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(kvc.EXPORTS) == names


def test_binding_constants_match_header(kvc):
    with open(os.path.join(ROOT, "include", "kvc.h")) as f:
        text = f.read()
    ws = int(re.search(r"#define KVC_DECODE_WORKSPACE_BYTES (\d+)", text).group(1))
    hb = int(re.search(r"#define KVC_HEADER_BYTES (\d+)", text).group(1))
    assert kvc.DECODE_WORKSPACE_BYTES == ws and ws % 256 == 0
    na = int(re.search(r"#define KVC_NOALLOC_SCRATCH_BYTES (\d+)", text).group(1))
    assert kvc.NOALLOC_SCRATCH_BYTES == na and na >= ws
    assert kvc.HEADER_BYTES == hb


def test_version_and_status_strings(kvc):
    assert kvc.kvc_version() == O.VERSION == 4
    assert kvc.kvc_status_string(0) == "ok"
    assert "corrupt" in kvc.kvc_status_string(-3)


def test_host_phi_tables_equal_oracle(kvc):
    # libm erfc in double on the library side, mpmath at 50 digits in the oracle
    a, b = kvc.kvc_phi_tables()
    oa, ob = O.phi_tables()
    assert np.array_equal(a.astype(np.int64), oa) and np.array_equal(b.astype(np.int64), ob)


def test_encode_sizes(kvc):
    w = W.WORKLOADS[2]
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, w.planes, w.tokens, w.channels, (9500, 300), 1024)
    max_stream, ws = kvc.kvc_encode_sizes(p)
    n_chunks = w.planes * 4 * 2
    assert max_stream == 128 + 8 * (n_chunks + 1) + n_chunks * (512 + 2 * 2 * 64 * 1024)
    # a look-back entry and a worst-case word slot (two words per scalar) per chunk
    assert n_chunks * (8 + 4 * 64 * 1024) <= ws <= n_chunks * (8 + 4 * 64 * 1024) + (1 << 20)
    for bad in [dict(channels=96), dict(planes=0), dict(tokens=0), dict(sigma_block_tokens=30, chunk_tokens=20),
                dict(sigma_block_tokens=1, chunk_tokens=0, planes=1 << 30, tokens=1 << 10), dict(kv_dtype=2),
                dict(mu_dtype=1), dict(w_narrow_bp=9000, w_wide_bp=1001), dict(chunk_tokens=1 << 21),
                dict(channels=1 << 21, chunk_tokens=1024)]:
        q = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 4, 100, 128)
        for k, v in bad.items():
            setattr(q, k, v)
        with pytest.raises(kvc.KvcError) as e:
            kvc.kvc_encode_sizes(q)
        assert e.value.status == kvc.KVC_ERR_INVALID


@pytest.mark.parametrize("planes,tokens,channels,expect", [
    (2304, 4096, 128, 586),      # 7 chunks per plane and group: 32,256 chunks, 3.94 rounds of 8,192
                                 # (1024 tokens: 18,432 chunks in 3 rounds, the last a quarter full)
    (448, 1024, 128, 256),       # 3,584 chunks: one round at any length, so the floor
    (16, 32768, 128, 256),       # one 32K-token layer: 4,096 chunks at the floor
    (576, 8192, 128, 586),       # 16,128 chunks, 1.97 rounds (1024 tokens: 9,216 chunks, 2 rounds)
    (64, 4096, 128, 256),        # 2,048 chunks
    (512, 4096, 128, 512),       # exactly one round of 8,192 chunks
    (3, 45, 128, 45),            # short sequences keep one chunk per plane and group
])
def test_default_chunk_length(kvc, planes, tokens, channels, expect):
    """chunk_tokens = 0 picks, among lengths from 1024 down to 256 tokens,
    the one with the least (rounds of 8,192 chunks) x (length + 9)."""
    auto = kvc.kvc_encode_sizes(kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, planes, tokens, channels, (9500, 300), 0))
    fixed = kvc.kvc_encode_sizes(kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, planes, tokens, channels, (9500, 300),
                                                 expect))
    assert auto == fixed
    if expect > 256:
        other = kvc.kvc_encode_sizes(kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, planes, tokens, channels,
                                                     (9500, 300), expect // 2))
        assert other != auto


@pytest.mark.parametrize("planes,tokens,block,expect", [
    (2304, 4096, 1024, 256),     # divisors 1024, 512, 256: 3, 5, 9 rounds of 1033, 521, 265
    (448, 1024, 300, 300),       # the only divisor of 300 in [256, 1024]
    (3, 45, 16, 16),             # blocks shorter than the floor: the block itself
    (3, 45, 100, 45),            # one block covers every token: the rule without blocks
    (4, 2000, 1031, 1),          # a prime block length above 1024: its divisor 1
])
def test_default_chunk_length_with_sigma_blocks(kvc, planes, tokens, block, expect):
    """With sigma blocks shorter than the tokens, the default chunk length is
    the best divisor of the block length (no chunk straddles two blocks)."""
    mk = lambda tc: kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, planes, tokens, 128, (9500, 300), tc, block)
    assert kvc.kvc_encode_sizes(mk(0)) == kvc.kvc_encode_sizes(mk(expect))


def oracle_stream(kv_dtype=O.BF16, w=(9500, 300), tc=16):
    kv, mu, sig, samples = W.tiny_case(7, kv_dtype=kv_dtype)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(W.to_numpy_bits(samples), kv_dtype, *w)
    return O.encode(W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), pref, kv_dtype, mu_dtype, *w, tc)


def test_stream_info_reads_oracle_headers(kvc):
    for kv_dtype, w, tc in [(O.BF16, (9500, 300), 16), (O.E4M3, (9500, 300), 7), (O.BF16, (10000, 0), 64)]:
        st = oracle_stream(kv_dtype, w, tc)
        p, total = kvc.kvc_stream_info(st[:128])
        h = O.parse_header(st)
        assert total == len(st)
        assert (p.kv_dtype, p.mu_dtype, p.w_narrow_bp, p.w_wide_bp, p.chunk_tokens) == \
               (h["kv_dtype"], h["mu_dtype"], h["w_narrow_bp"], h["w_wide_bp"], h["chunk_tokens"])
        assert (p.planes, p.tokens, p.channels) == (h["planes"], h["tokens"], h["channels"])


def test_stream_info_reads_the_sigma_block_field(kvc):
    kv, mu, sig, samples = W.tiny_case(3, 2, 45, 128, O.BF16)
    kv, mu, sig, samples = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    sig3 = np.repeat(sig[:, None, :], 3, axis=1)
    st = O.encode(kv, mu, sig3, pref, O.BF16, O.BF16, 9500, 300, 8, sigma_block_tokens=16)
    p, total = kvc.kvc_stream_info(st[:128])
    assert p.sigma_block_tokens == 16 and p.chunk_tokens == 8 and total == len(st)
    bad = bytearray(st[:128])
    bad[88] = 20                                       # 20 is not a multiple of the 8-token chunks
    with pytest.raises(kvc.KvcError):
        kvc.kvc_stream_info(bytes(bad))


@pytest.mark.parametrize("offset", [0, 4, 8, 10, 13, 16, 24, 36, 56, 64, 92, 100])
def test_stream_info_rejects_damaged_headers(kvc, offset):
    st = bytearray(oracle_stream()[:128])
    st[offset] ^= 0x41
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_stream_info(bytes(st))
    assert e.value.status == kvc.KVC_ERR_CORRUPT


@pytest.mark.parametrize("offset,bit", [(9, 1), (9, 2), (48, 0), (48, 1), (64, 0), (72, 3), (80, 5), (88, 0), (88, 4)])
def test_stream_info_rejects_single_bit_flips_that_keep_the_fields_valid(kvc, offset, bit):
    """Flips that leave every field plausible on its own (mu dtype bf16 ->
    f32, a token count with the same chunk count, the payload size, the side
    checksum, the sigma block length) are caught by the header CRC."""
    st = bytearray(oracle_stream()[:128])
    st[offset] ^= 1 << bit
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_stream_info(bytes(st))
    assert e.value.status == kvc.KVC_ERR_CORRUPT


def test_stream_info_accepts_a_recomputed_crc(kvc):
    """The library's CRC is zlib's: a field changed together with a
    recomputed CRC parses (so the check is the CRC, not a byte compare)."""
    import zlib
    st = bytearray(oracle_stream()[:128])
    st[80] ^= 0xFF                                          # the side checksum: any value is valid
    st[92:96] = zlib.crc32(bytes(st[:92])).to_bytes(4, "little")
    p, total = kvc.kvc_stream_info(bytes(st))
    assert total == len(oracle_stream())


@pytest.mark.parametrize("nu", list(range(0, 17)))
def test_library_narrow_tables_equal_the_oracle(kvc, nu):
    """The library's double-precision Student-t series (and libm's erfc for
    nu = 0) round to the oracle's 50-digit tables."""
    assert np.array_equal(kvc.kvc_narrow_table(nu).astype(np.int64), O.narrow_table(nu))


def test_stream_info_reads_the_narrow_part(kvc):
    kv, mu, sig, samples = W.tiny_case(7)
    kv, mu, sig, samples = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(samples, O.BF16, 9500, 300)
    st = O.encode(kv, mu, sig, pref, O.BF16, O.BF16, 9500, 300, 16, narrow_dof=5)
    p, total = kvc.kvc_stream_info(st[:128])
    assert p.narrow_dof == 5 and total == len(st)
    import zlib
    bad = bytearray(st[:128])
    bad[14] = 17
    bad[92:96] = zlib.crc32(bytes(bad[:92])).to_bytes(4, "little")
    with pytest.raises(kvc.KvcError):
        kvc.kvc_stream_info(bytes(bad))
    with pytest.raises(kvc.KvcError):
        kvc.kvc_narrow_table(17)
    q = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, 4, 100, 128, narrow_dof=17)
    with pytest.raises(kvc.KvcError):
        kvc.kvc_encode_sizes(q)
