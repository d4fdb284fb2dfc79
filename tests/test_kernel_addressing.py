"""A host replay of the coding kernels' index arithmetic for small shapes,
asserting that every access stays inside its buffer.  It follows the
kernels' own steps: a wave's chunk from its index (chunk_pos: channel group
fastest, then the token chunk, then the plane), the rows it reads (KV, mu)
or writes (decoded KV) through buffer ranges that start at the chunk's first
row, its sigma row (one sigma block per chunk), its word slot in the encode
workspace (filled from the slot's end, at most two words per lane and
token), the placement copy (16-byte reads that run a few dwords past the
words) and the chunk's place in the stream.  The chunk order is checked
against the oracle's chunk layout (S-10), and the workspace and stream
sizes against what kvc_encode_sizes returns."""
import numpy as np
import pytest

import oracle as O
from entropy_coding_amd import workloads as W

LANES = 64
STATE_BYTES = 8 * LANES
HEADER_BYTES = 128


def geometry(planes, tokens, channels, tc, block):
    """The library's chunk geometry for a call (the same integer steps)."""
    n_tok = -(-tokens // tc)
    groups = channels // 64
    sigma_blocks = -(-tokens // block) if block else 1
    sigma_tc = block // tc if block else 0
    return dict(planes=planes, tokens=tokens, channels=channels, tc=tc, n_tok=n_tok, groups=groups,
                n_chunks=planes * n_tok * groups, sigma_blocks=sigma_blocks, sigma_tc=sigma_tc)


def chunk_pos(geo, c):
    """A wave's chunk from its index, as the kernels derive it."""
    k = c % geo["groups"]
    rest = c // geo["groups"]
    tci = rest % geo["n_tok"]
    g = rest // geo["n_tok"]
    srow = g * geo["sigma_blocks"] + (tci // geo["sigma_tc"] if geo["sigma_tc"] else 0)
    t0 = tci * geo["tc"]
    ln = min(geo["tc"], geo["tokens"] - t0)
    return g, srow, t0, ln, k


def slot_words(tc):
    return -(-2 * LANES * tc // 4) * 4           # two words per lane and token, a multiple of 4


SHAPES = [  # planes, tokens, channels, chunk tokens, sigma block
    (1, 1, 64, 1, 0), (2, 45, 128, 16, 0), (3, 100, 192, 33, 0), (4, 64, 128, 64, 0),
    (2, 45, 128, 16, 32), (5, 130, 256, 20, 40), (1, 300, 64, 256, 0), (2, 17, 128, 5, 15),
]


@pytest.mark.parametrize("planes,tokens,channels,tc,block", SHAPES)
def test_every_scalar_is_read_and_written_once_inside_its_buffers(planes, tokens, channels, tc, block):
    geo = geometry(planes, tokens, channels, tc, block)
    total = planes * tokens * channels
    hits = np.zeros(total, dtype=np.int64)
    sigma_words = planes * geo["sigma_blocks"] * channels
    lane = np.arange(LANES)
    for c in range(geo["n_chunks"]):
        g, srow, t0, ln, k = chunk_pos(geo, c)
        assert 0 <= g < planes and 1 <= ln <= tc and t0 + ln <= tokens
        # the chunk's buffer range: len rows from its first row (the KV, mu and output buffers)
        row0 = (g * tokens + t0) * channels + 64 * k
        rng_end = row0 + ln * channels
        t = np.arange(ln)[:, None]
        idx = row0 + t * channels + lane[None, :]
        assert idx.min() >= row0 and idx.max() < rng_end          # inside the buffer range ...
        assert idx.max() < total                                   # ... and inside the tensor
        np.add.at(hits, idx.ravel(), 1)
        # sigma: one row per chunk, every token of the chunk in that block
        s_idx = srow * channels + 64 * k + lane
        assert s_idx.min() >= 0 and s_idx.max() < sigma_words
        if block:
            assert (t0 // block) == ((t0 + ln - 1) // block) == srow - g * geo["sigma_blocks"]
    assert np.all(hits == 1)


@pytest.mark.parametrize("planes,tokens,channels,tc,block", SHAPES)
def test_chunk_order_is_the_oracle_layout(planes, tokens, channels, tc, block):
    geo = geometry(planes, tokens, channels, tc, block)
    g_of, tc_of, k_of, len_of = O.kvc_oracle.chunk_layout(planes, tokens, channels, tc)
    assert len(g_of) == geo["n_chunks"]
    for c in range(geo["n_chunks"]):
        g, _, t0, ln, k = chunk_pos(geo, c)
        assert (g, t0, k, ln) == (g_of[c], tc_of[c] * tc, k_of[c], len_of[c])


@pytest.mark.parametrize("planes,tokens,channels,tc,block", SHAPES)
def test_encode_workspace_and_stream_hold_the_worst_case(kvc, planes, tokens, channels, tc, block):
    geo = geometry(planes, tokens, channels, tc, block)
    p = kvc.make_params(kvc.KVC_BF16, kvc.KVC_BF16, planes, tokens, channels, (9500, 300), tc)
    p.sigma_block_tokens = block
    max_stream, ws = kvc.kvc_encode_sizes(p)
    n = geo["n_chunks"]
    sw = slot_words(tc)
    status = 256
    slots = -(-(status + 8 * n) // 256) * 256
    # look-back entries before the slots; the last slot, plus the copy's
    # read-ahead (4 dwords), inside the workspace
    assert status + 8 * n <= slots
    assert slots + 2 * n * sw + 16 <= ws
    worst = HEADER_BYTES + 8 * (n + 1)
    for c in range(n):
        _, _, _, ln, _ = chunk_pos(geo, c)
        words = 2 * LANES * ln                                     # every symbol at two words
        assert words <= sw
        worst += -(-(STATE_BYTES + 2 * words) // 8) * 8
    assert worst <= max_stream


def copy_ranges(nw, sw):
    """The placement copy of a chunk with nw words left in its slot of sw
    words: (first, last) dword read relative to the slot's start, and the
    dwords written after the chunk's states."""
    wp = sw - nw
    size = -(-(STATE_BYTES + 2 * nw) // 8) * 8
    out_dw = (size - STATE_BYTES) // 4
    src = wp >> 1
    last = -1
    for base in range(0, out_dw, 256 * 4):
        for b in range(4):
            j = base + 256 * b + 4 * np.arange(LANES)
            j = j[j < out_dw]
            if len(j):
                last = max(last, int(src + j.max() + 4))              # the uint4 and the dword after it
    return src, last, out_dw, size


@pytest.mark.parametrize("seed,planes,tokens,tc,weights", [
    (3, 2, 45, 16, (9500, 300)), (4, 1, 70, 64, (10000, 0)), (5, 3, 33, 8, (0, 0))])
def test_placement_copy_of_real_chunks_stays_in_the_workspace(seed, planes, tokens, tc, weights):
    kv, mu, sig, samples = W.tiny_case(seed, planes=planes, tokens=tokens)
    kvn, mun, sgn, smn = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    pref = O.build_marginal(smn, O.BF16, *weights)
    st = O.encode(kvn, mun, sgn, pref, O.BF16, O.BF16, *weights, tc)
    geo = geometry(planes, tokens, 128, tc, 0)
    n = geo["n_chunks"]
    d = np.frombuffer(st[HEADER_BYTES:HEADER_BYTES + 8 * (n + 1)], dtype="<u8")
    sw = slot_words(tc)
    slots = -(-(256 + 8 * n) // 256) * 256
    for c in range(n):
        size = int(d[c + 1] - d[c])
        nw_max = (size - STATE_BYTES) // 2
        # the words actually emitted: the chunk size is the states plus the words, padded to 8 bytes
        for nw in range(max(0, nw_max - 3), nw_max + 1):
            if -(-(STATE_BYTES + 2 * nw) // 8) * 8 != size:
                continue
            src, last, out_dw, sz = copy_ranges(nw, sw)
            assert sz == size and 2 * out_dw * 2 >= 2 * nw
            assert src >= 0
            # reads stay within this slot and 4 dwords past it; past the last
            # slot, inside the workspace (slots are followed by the tables)
            assert last < sw // 2 + 4
            assert slots + 2 * (c * sw) + 4 * (last + 1) <= slots + 2 * n * sw + 16
        # the chunk's place in the stream: states then words, inside the payload
        assert d[c] % 8 == 0 and d[c + 1] <= len(st) - HEADER_BYTES - 8 * (n + 1)
