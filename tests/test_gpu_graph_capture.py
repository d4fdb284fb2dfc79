"""The asynchronous calls inside a captured HIP graph: once the per-device
tables exist (an eager call builds them), kvc_encode without a size pointer
and kvc_decode_async launch kernels only (the control block is cleared by a
kernel, never a memset), so a caller may capture them.  The graph is
replayed several times with eager work and synchronisations between the
replays, and every replay's stream, status and decoded KV must equal the
eager result."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("kv_dtype", [O.BF16, O.E4M3])
def test_encode_and_decode_replay_from_a_graph(kvc, cuda, kv_dtype):
    say(f"graph capture, kv dtype {kv_dtype}")
    planes, tokens, channels, tc = 4, 64, 128, 16
    kv, mu, sig, samples = W.tiny_case(5, planes, tokens, channels, kv_dtype)
    kv_d, mu_d, sig_d = kv.to(cuda), mu.to(cuda), sig.to(cuda)
    pref_d = kvc.kvc_build_marginal(samples.to(cuda), (9500, 300))
    p = kvc.make_params(kvc._kv_dtype(kv_d), kvc._mu_dtype(mu_d), planes, tokens, channels, (9500, 300), tc)
    enc = kvc.Encoder(p, cuda)
    # eager: the reference stream, and the per-device tables built
    ref = enc(kv_d, mu_d, sig_d, pref_d).clone()
    header = enc.header.copy()
    mun, sgn = W.to_numpy_bits(mu), sig.numpy()
    pref = pref_d.cpu().numpy().astype(np.int64)
    mu_code = O.BF16 if kv_dtype == O.BF16 else O.F32
    assert ref.cpu().numpy().tobytes() == O.encode(W.to_numpy_bits(kv), mun, sgn, pref, kv_dtype, mu_code,
                                                   9500, 300, tc)
    out_dt = torch.int16 if kv_dtype == O.BF16 else torch.uint8
    out = torch.zeros(kv_d.shape, dtype=out_dt, device=cuda)
    ws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=cuda)
    assert kvc.kvc_decode_into(ref, mu_d, sig_d, pref_d, out, ws) == kvc.KVC_OK
    n = ref.numel()
    stream_view = enc.out[:n]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enc.enqueue(kv_d, mu_d, sig_d, pref_d)
        rc = kvc.kvc_decode_async(stream_view, mu_d, sig_d, pref_d, out, ws, header)
    assert rc == kvc.KVC_OK
    for i in range(3):
        # eager work between the replays: the outputs cleared, a synchronisation
        out.zero_()
        enc.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(enc.result(), ref), f"replay {i}: stream"
        assert kvc.kvc_decode_result(ws) == kvc.KVC_OK, f"replay {i}: status"
        assert torch.equal(out, kv_d.view(out_dt)), f"replay {i}: decoded KV"
    del g
