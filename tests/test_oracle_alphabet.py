"""Pins of the oracle's ordered alphabet and cell edges (KVC-1 S-1, S-2).

Values come from torch's own bf16 / float8_e4m3fn decoders, not from the
oracle, so a wrong bit trick in the oracle fails here."""
import numpy as np
import pytest
import torch

import oracle as O


def torch_values(dtype):
    if dtype == O.BF16:
        u = torch.arange(65536, dtype=torch.int32).to(torch.int16)
        return u.view(torch.bfloat16).to(torch.float64).numpy()
    u = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return u.view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
def test_order_index_is_a_bijection(dtype):
    n = O.alphabet_size(dtype)
    bits = np.arange(n)
    idx = O.order_index(bits, dtype)
    assert np.array_equal(np.sort(idx), np.arange(n))
    assert np.array_equal(O.bits_of_order(idx, dtype), bits)


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
def test_order_index_sorts_values(dtype):
    vals = torch_values(dtype)
    n = vals.size
    order = O.bits_of_order(np.arange(n), dtype)
    v = vals[order]
    fin = np.isfinite(v) | np.isinf(v)
    vv = v[fin]
    assert np.all(np.diff(vv) >= 0)
    # NaNs sit only at the two ends
    nan_pos = np.flatnonzero(np.isnan(v))
    lo_block = nan_pos[nan_pos < n // 2]
    hi_block = nan_pos[nan_pos >= n // 2]
    assert np.array_equal(lo_block, np.arange(lo_block.size))
    assert np.array_equal(hi_block, np.arange(n - hi_block.size, n))


def test_bf16_landmarks():
    b = O.order_index(np.array([0xFFFF, 0xFF80, 0xFF7F, 0x8000, 0x0000, 0x7F7F, 0x7F80, 0x7FC0, 0x7FFF]), O.BF16)
    assert b.tolist() == [0, 127, 128, 32767, 32768, 65407, 65408, 65472, 65535]


def test_e4m3_landmarks():
    b = O.order_index(np.array([0xFF, 0xFE, 0x80, 0x00, 0x7E, 0x7F]), O.E4M3)
    assert b.tolist() == [0, 1, 127, 128, 254, 255]


def test_e4m3_decoder_matches_torch():
    mine = O.symbol_value(O.order_index(np.arange(256), O.E4M3), O.E4M3)
    ref = torch_values(O.E4M3)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.nanmax(ref) == 448.0


@pytest.mark.parametrize("dtype", [O.BF16, O.E4M3])
def test_boundary_positions(dtype):
    pos = O.boundary_positions(dtype).astype(np.float64)
    n = O.alphabet_size(dtype)
    vals = torch_values(dtype)[O.bits_of_order(np.arange(n), dtype)]
    finite = np.isfinite(vals)
    lo, hi = np.flatnonzero(finite)[[0, -1]]
    zero = int(O.order_index(0, dtype))
    b = np.arange(n + 1)
    inner = (b > lo) & (b <= hi) & (b != zero)
    bi = b[inner]
    # the edge is exactly the midpoint of its two neighbours
    assert np.array_equal(2.0 * pos[inner], vals[bi - 1] + vals[bi])
    assert pos[zero] == 0.0
    assert np.all(np.isneginf(pos[: lo + 1])) and np.all(np.isposinf(pos[hi + 1:]))
    # strictly increasing over the finite range, and never a symbol value
    fin = pos[lo + 1: hi + 1]
    assert np.all(np.diff(fin) > 0)
    assert not np.any(np.isin(fin[fin != 0], vals[finite]))


def test_bf16_edge_examples():
    pos = O.boundary_positions(O.BF16)
    # between 0.99609375 (0x3F7F) and 1.0 (0x3F80)
    b = int(O.order_index(0x3F80, O.BF16))
    assert pos[b] == np.float32(0.998046875)
    # the -max cell is open to -inf, +max cell to +inf
    assert pos[128] == -np.inf and pos[129] < -3.3e38
    assert pos[65408] == np.inf and pos[65407] > 3.3e38
