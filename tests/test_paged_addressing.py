"""A host model of the paged decoder's address arithmetic (the PAGED
variant of the decoding kernel), run over every paged parity case and the
full-size configurations.  Per wave (chunk) it follows the kernel's own
incremental steps: the pool chosen from the plane, the page base of the
chunk's 64 channels of one head, the 32-entry window of its block-table row
staged per wave (refilled every 32 pages), the countdown to the next page
boundary, and the row address advanced by one token row per step.  Every
table read must fall inside the entries the call checks ([0, used) of the
sequence's row), every row store must be the intended row of the intended
page (page block_table[b][t / page_tokens], row t % page_tokens, head h,
channels 64k .. 64k + 63) and inside its pool."""
import numpy as np
import pytest

from entropy_coding_amd import workloads as W

WINDOW = 32          # block-table entries a wave stages in LDS


def chunk_layout(planes, tokens, channels, tc):
    n_tc = -(-tokens // tc)
    groups = channels // 64
    c = np.arange(planes * n_tc * groups, dtype=np.int64)
    k = c % groups
    tci = (c // groups) % n_tc
    g = c // (groups * n_tc)
    t0 = tci * tc
    length = np.minimum(tc, tokens - t0)
    return g, t0, k, length


def check_paged(planes, tokens, channels, tc, esize, batch, heads, page_tokens, table, num_pages, mutate=None):
    """Replays the kernel's paged addressing for every chunk; raises on the
    first out-of-range table read or misplaced store.  Returns the number of
    row stores checked."""
    table = np.asarray(table, dtype=np.int64)
    max_pages = table.shape[1]
    per_kv = batch * heads
    assert planes % (2 * per_kv) == 0
    n_pools = planes // per_kv
    used = -(-tokens // page_tokens)                    # columns the pre-check covers
    assert np.all((table[:, :used] >= 0) & (table[:, :used] < num_pages))
    tok_bytes = heads * channels * esize
    page_bytes = page_tokens * tok_bytes
    pool_bytes = num_pages * page_bytes
    assert tok_bytes < 2 ** 32 and page_bytes < 2 ** 32
    g, t0, k, length = chunk_layout(planes, tokens, channels, tc)
    lk = g // per_kv
    assert np.all(lk < n_pools)                         # pools[lk] inside the pool array
    bh = g - lk * per_kv
    b = bh // heads
    h = bh - b * heads
    # pool bases as distinct far-apart addresses, so a store landing in the
    # wrong pool or outside its pool shows up
    pool_base = (np.arange(n_pools, dtype=np.int64) + 1) * (1 << 40)
    page_base = pool_base[lk] + (h * channels + k * 64) * esize
    page_i = t0 // page_tokens
    in_page = t0 - page_i * page_tokens
    if mutate == "row":                                 # a planted mistake: the chunk's first row
        in_page = np.minimum(in_page + 1, page_tokens - 1)
    entry0 = b * max_pages + page_i                     # flat index of the window's first entry
    cols_left = used - page_i
    n_chunks = g.size
    window = np.full((n_chunks, WINDOW), -1, dtype=np.int64)

    def fill(mask):
        n = np.minimum(cols_left, WINDOW)
        for lane in range(WINDOW):
            m = mask & (lane < n)
            idx = entry0[m] + lane
            row, col = idx // max_pages, idx % max_pages
            assert np.all(row == b[m]) and np.all(col < used), "table read outside the checked entries"
            window[m, lane] = table[row, col]

    fill(np.ones(n_chunks, dtype=bool))
    slot = np.zeros(n_chunks, dtype=np.int64)
    page_left = page_tokens - in_page
    assert np.all(window[np.arange(n_chunks), slot] >= 0)
    page_row = page_base + window[np.arange(n_chunks), slot] * page_bytes + in_page * tok_bytes
    stores = 0
    for t in range(int(length.max())):
        live = t < length
        tok = t0 + t
        want_page = table[b, np.minimum(tok // page_tokens, used - 1)]
        want = pool_base[lk] + want_page * page_bytes + (tok % page_tokens) * tok_bytes \
            + (h * channels + k * 64) * esize
        bad = live & (page_row != want)
        assert not np.any(bad), f"misplaced row store at step {t} in chunk {int(np.argmax(bad))}"
        lo = page_row - pool_base[lk]
        assert np.all(~live | ((lo >= 0) & (lo + 64 * esize <= pool_bytes))), "store outside its pool"
        stores += int(live.sum())
        # the kernel's step: a token row further, a new page at a boundary
        page_row = page_row + tok_bytes
        page_left = page_left - (2 if mutate == "boundary" else 1)
        nxt = live & (page_left == 0) & (t + 1 < length)
        if np.any(nxt):
            slot = np.where(nxt, slot + 1, slot)
            refill = nxt & (slot == WINDOW)
            if np.any(refill):
                entry0 = np.where(refill, entry0 + WINDOW, entry0)
                cols_left = np.where(refill, cols_left - WINDOW, cols_left)
                assert np.all(cols_left[refill] >= 1)
                window[refill] = -1
                fill(refill)
                slot = np.where(refill, 0, slot)
            page_left = np.where(nxt, page_tokens, page_left)
            e = window[np.arange(n_chunks), slot]
            assert np.all(e[nxt] >= 0), "page entry read from an unfilled window slot"
            page_row = np.where(nxt, page_base + e * page_bytes, page_row)
    return stores


# the paged parity cases: kv dtype size, chunk tokens, page tokens, layers,
# batch, heads, tokens, channels (the table has one spare column and spare
# pages, shuffled)
CASES = [
    (2, 16, 8, 2, 2, 2, 45, 128),
    (2, 7, 5, 1, 3, 2, 45, 64),
    (2, 45, 1, 1, 1, 2, 45, 128),
    (1, 7, 16, 2, 1, 2, 33, 128),
    (2, 586, 1, 1, 1, 1, 1300, 64),          # a page per token over more than one window
    (2, 100, 3, 1, 2, 1, 1000, 128),         # pages straddling chunks, many windows
]


@pytest.mark.parametrize("esize,tc,pt,layers,batch,heads,t,d", CASES)
def test_paged_addressing_of_the_parity_cases(esize, tc, pt, layers, batch, heads, t, d):
    max_pages = -(-t // pt) + 1
    num_pages = batch * max_pages + 5
    rng = np.random.default_rng(pt * 7 + tc)
    table = rng.permutation(num_pages)[:batch * max_pages].reshape(batch, max_pages)
    planes = layers * 2 * batch * heads
    n = check_paged(planes, t, d, tc, esize, batch, heads, pt, table, num_pages)
    assert n == planes * t * (d // 64)


@pytest.mark.parametrize("pt", [16, 1024])
def test_paged_addressing_full_size(pt):
    """The Qwen3-8B-shaped cache at its benchmark chunk length in shuffled
    pages, as the full-size paged test and the benchmark lay it out."""
    w = W.WORKLOADS[2]
    max_pages = w.tokens // pt
    num_pages = w.batch * max_pages
    table = np.random.default_rng(5).permutation(num_pages).reshape(w.batch, max_pages)
    n = check_paged(w.planes, w.tokens, w.channels, w.chunk_tokens, 2, w.batch, w.heads, pt, table, num_pages)
    assert n == w.planes * w.tokens * (w.channels // 64)


@pytest.mark.parametrize("mutate", ["row", "boundary"])
def test_model_catches_planted_mistakes(mutate):
    """The model notices a misplaced store: a chunk that starts one row off
    within its page, or a page boundary counted twice as fast."""
    rng = np.random.default_rng(3)
    table = rng.permutation(20)[:14].reshape(2, 7)
    check_paged(8, 45, 64, 16, 2, 2, 2, 8, table, 20)
    with pytest.raises(AssertionError):
        check_paged(8, 45, 64, 16, 2, 2, 2, 8, table, 20, mutate=mutate)
