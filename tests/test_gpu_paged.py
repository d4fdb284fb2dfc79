"""GPU parity of the decoder fused into a paged KV cache: every decoded row
lands in its page exactly where the oracle places it (other pages keep
their contents), a full-size cache round-trips through the pages, and bad
descriptors or table entries are rejected."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bits(x: np.ndarray, dev):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def make_pools(kvc, n_pools, num_pages, pt, heads, d, dtype, dev, fill):
    return [torch.full((num_pages, pt, heads, d), fill, dtype=dtype, device=dev) for _ in range(n_pools)]


CASES = [
    # kv dtype, chunk tokens, page tokens, layers, batch, heads, tokens, channels
    (O.BF16, 16, 8, 2, 2, 2, 45, 128),      # two pages per chunk, ragged last page
    (O.BF16, 7, 5, 1, 3, 2, 45, 64),        # pages straddle chunks
    (O.BF16, 45, 1, 1, 1, 2, 45, 128),      # a page per token
    (O.E4M3, 7, 16, 2, 1, 2, 33, 128),
]


@pytest.mark.parametrize("kv_dtype,tc,pt,layers,batch,heads,t,d", CASES)
def test_paged_decode_matches_oracle_placement(kvc, cuda, kv_dtype, tc, pt, layers, batch, heads, t, d):
    say(f"case kv={kv_dtype} tc={tc} page={pt} layers={layers} batch={batch} heads={heads} tokens={t}")
    g_n = layers * 2 * batch * heads
    kv, mu, sig, samples = W.tiny_case(17, g_n, t, d, kv_dtype)
    kv, mu, sig, samples = W.to_numpy_bits(kv), W.to_numpy_bits(mu), sig.numpy(), W.to_numpy_bits(samples)
    mu_dtype = O.BF16 if kv_dtype == O.BF16 else O.F32
    pref = O.build_marginal(samples, kv_dtype, 9500, 300)
    st = O.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, 9500, 300, tc)
    max_pages = -(-t // pt) + 1                       # one spare column
    num_pages = batch * max_pages + 5                 # pages no token maps to
    rng = np.random.default_rng(pt * 7 + tc)
    table = rng.permutation(num_pages)[:batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    fill = SENTINEL if kv_dtype == O.BF16 else 0x5A
    want = O.scatter_to_pages(O.decode(st, mu, sig, pref), batch, heads, table, pt, num_pages, fill=fill)

    dt = torch.int16 if kv_dtype == O.BF16 else torch.uint8
    pools = make_pools(kvc, layers * 2, num_pages, pt, heads, d, dt, cuda, fill)
    paged = kvc.PagedKV(pools, torch.from_numpy(table).to(cuda), pt)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    rc = kvc.kvc_decode_paged(torch.from_numpy(np.frombuffer(st, np.uint8).copy()).to(cuda), dev_bits(mu, cuda),
                              torch.from_numpy(sig).to(cuda), torch.from_numpy(pref.astype(np.int32)).to(cuda),
                              paged, ws)
    assert rc == kvc.KVC_OK
    got = np.stack([p.cpu().numpy() for p in pools])
    if kv_dtype == O.BF16:
        got = got.view(np.uint16)
    assert np.array_equal(got, want)


def test_paged_decode_rejects_bad_descriptors(kvc, cuda):
    layers, batch, heads, t, d, pt = 1, 2, 2, 45, 128, 8
    g_n = layers * 2 * batch * heads
    kv, mu, sig, samples = W.tiny_case(19, g_n, t, d, O.BF16)
    kv_d, mu_d, sig_d = kv.to(cuda), mu.to(cuda), sig.to(cuda)
    pref = kvc.kvc_build_marginal(samples.to(cuda))
    st = kvc.kvc_encode(kv_d, mu_d, sig_d, pref, (9500, 300), 16)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    max_pages, num_pages = 6, 12
    table = torch.arange(batch * max_pages, dtype=torch.int32, device=cuda).reshape(batch, max_pages)
    pools = make_pools(kvc, 2, num_pages, pt, heads, d, torch.int16, cuda, 0)
    ok = kvc.PagedKV(pools, table, pt)
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, ok, ws) == kvc.KVC_OK
    back = torch.stack(pools)                                      # [2, pages, pt, heads, d]
    for g in range(g_n):
        lk, b, h = g // (batch * heads), (g // heads) % batch, g % heads
        rows = back[lk, table[b].long()].reshape(-1, heads, d)[:t, h]
        assert torch.equal(rows, kv_d[g].view(torch.int16))
    # an entry outside the pool: reported, nothing written outside
    bad_table = table.clone()
    bad_table[1, 3] = num_pages
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, kvc.PagedKV(pools, bad_table, pt), ws) == kvc.KVC_ERR_INVALID
    bad_table[1, 3] = -1
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, kvc.PagedKV(pools, bad_table, pt), ws) == kvc.KVC_ERR_INVALID
    # a table narrower than the tokens need
    narrow = kvc.PagedKV(pools, table[:, :5].contiguous(), pt)
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, narrow, ws) == kvc.KVC_ERR_INVALID
    # planes that are not layers x 2 x batch x heads
    odd = kvc.PagedKV(pools, table, pt)
    odd.desc.heads = 3
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, odd, ws) == kvc.KVC_ERR_INVALID
    odd.desc.heads = heads
    odd.desc.reserved = 1
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, odd, ws) == kvc.KVC_ERR_INVALID
    odd.desc.reserved = 0
    # fewer pools than the planes need, pools shorter than num_pages pages
    odd.desc.n_pools = 1
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, odd, ws) == kvc.KVC_ERR_INVALID
    odd.desc.n_pools = 2
    odd.desc.pool_bytes -= 2
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, odd, ws) == kvc.KVC_ERR_INVALID
    # pools whose rows are not the stream's channels or element type
    wide = make_pools(kvc, 2, num_pages, pt, heads, 2 * d, torch.int16, cuda, 0)
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, kvc.PagedKV(wide, table, pt), ws) == kvc.KVC_ERR_INVALID
    bytes8 = make_pools(kvc, 2, num_pages, pt, heads, d, torch.uint8, cuda, 0)
    assert kvc.kvc_decode_paged(st, mu_d, sig_d, pref, kvc.PagedKV(bytes8, table, pt), ws) == kvc.KVC_ERR_INVALID


def test_paged_decode_full_size(kvc, cuda):
    """The Qwen3-8B-shaped cache (one call, the benchmark's chunk length)
    decoded into 16-token pages in shuffled order and read back through the
    table."""
    w = W.WORKLOADS[2]
    ppl = w.planes_per_layer
    G, T, D = w.planes, w.tokens, w.channels
    kv = torch.empty((G, T, D), dtype=torch.bfloat16, device=cuda)
    mu = torch.empty_like(kv)
    sig = torch.empty((G, D), dtype=torch.float32, device=cuda)
    for l in range(w.layers):
        k, m = W.layer_data(w, l, device=cuda)
        kv[l * ppl:(l + 1) * ppl] = k
        mu[l * ppl:(l + 1) * ppl] = m
        sig[l * ppl:(l + 1) * ppl] = W.layer_sigma_true(w, l, device=cuda)
    prefix = kvc.kvc_build_marginal(W.marginal_samples(w, device=cuda))
    st = kvc.kvc_encode(kv, mu, sig, prefix, (w.w_narrow_bp, w.w_wide_bp), w.chunk_tokens)
    pt = 16
    max_pages = T // pt
    num_pages = w.batch * max_pages
    g = torch.Generator(device="cpu").manual_seed(5)
    table = torch.randperm(num_pages, generator=g).to(torch.int32).reshape(w.batch, max_pages).to(cuda)
    pools = make_pools(kvc, w.layers * 2, num_pages, pt, w.heads, D, torch.int16, cuda, 0)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    say(f"decoding {kv.numel()} scalars into {len(pools)} pools of {num_pages} x {pt}-token pages")
    assert kvc.kvc_decode_paged(st, mu, sig, prefix, kvc.PagedKV(pools, table, pt), ws) == kvc.KVC_OK
    tl = table.long()
    for lk, pool in enumerate(pools):
        # [pages, pt, heads, D] -> per sequence [batch, T, heads, D] -> planes [batch * heads, T, D]
        seq = pool[tl].reshape(w.batch, T, w.heads, D).permute(0, 2, 1, 3).reshape(w.batch * w.heads, T, D)
        want = kv[lk * w.batch * w.heads:(lk + 1) * w.batch * w.heads].view(torch.int16)
        assert torch.equal(seq, want), f"pool {lk}"
