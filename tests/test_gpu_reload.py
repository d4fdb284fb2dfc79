"""The host-offload reload through the library (kvc_reload): per-layer
streams in pinned host memory copied to the device on their own stream while
the layer before decodes; the decoded cache must equal the input on every
scalar, and a damaged layer, a wrong side input or a short staging buffer
must be reported with the layer it concerns."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from entropy_coding_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def cache(kvc, cuda):
    """Six layers of the Qwen3-0.6B-shaped workload (16 planes x 1024 tokens
    x 128 channels each), sigma calibrated per layer, each layer coded by its
    own call and moved to pinned host memory."""
    w = W.WORKLOADS[1]
    layers = 6
    kvs, mus, sigs, host = [], [], [], []
    prefix = kvc.kvc_build_marginal(W.marginal_samples(w, device=cuda), (w.w_narrow_bp, w.w_wide_bp))
    for l in range(layers):
        kv, mu = W.layer_data(w, l, device=cuda)
        ck, cm = W.layer_calibration(w, l, reps=w.calib_reps, device=cuda)
        sig = W.expand_sigma(w, kvc.kvc_calibrate_sigma(ck, cm))
        st = kvc.kvc_encode(kv, mu, sig, prefix, (w.w_narrow_bp, w.w_wide_bp), w.chunk_tokens)
        h = torch.empty(st.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(st)
        kvs.append(kv)
        mus.append(mu)
        sigs.append(sig)
        host.append(h)
    say(f"{layers} layer streams in pinned host memory: {sum(h.numel() for h in host)} bytes")
    return w, torch.stack(kvs), torch.stack(mus), torch.stack(sigs), prefix, host


def test_reload_decodes_every_layer(kvc, cuda, cache):
    w, kv, mu, sig, prefix, host = cache
    out = torch.zeros(kv.shape, dtype=torch.int16, device=cuda)
    st, failed = kvc.kvc_reload(host, mu, sig, prefix, out)
    assert st == kvc.KVC_OK and failed == -1
    assert torch.equal(out, kv.view(torch.int16))
    # layer 0's stream is the oracle's
    kvn, mun, sgn = W.to_numpy_bits(kv[0]), W.to_numpy_bits(mu[0]), sig[0].cpu().numpy()
    pref = prefix.cpu().numpy().astype(np.int64)
    want = O.encode(kvn, mun, sgn, pref, O.BF16, O.BF16, w.w_narrow_bp, w.w_wide_bp, w.chunk_tokens)
    assert host[0].numpy().tobytes() == want


def test_reload_reports_the_failing_layer(kvc, cuda, cache):
    w, kv, mu, sig, prefix, host = cache
    out = torch.zeros(kv.shape, dtype=torch.int16, device=cuda)
    # a damaged payload in layer 3
    bad = [h.clone().pin_memory() for h in host]
    bad[3][-9] ^= 4
    st, failed = kvc.kvc_reload(bad, mu, sig, prefix, out)
    assert st == kvc.KVC_ERR_CORRUPT and failed == 3
    assert torch.equal(out[:3], kv[:3].view(torch.int16))
    # another layer's sigma for layer 2
    sig2 = sig.clone()
    sig2[2] = sig[1]
    st, failed = kvc.kvc_reload(host, mu, sig2, prefix, out)
    assert st == kvc.KVC_ERR_MISMATCH and failed == 2
    # a damaged header in layer 4 is refused before anything of it runs
    bad = [h.clone().pin_memory() for h in host]
    bad[4][50] ^= 1
    st, failed = kvc.kvc_reload(bad, mu, sig, prefix, out)
    assert st == kvc.KVC_ERR_CORRUPT and failed == 4
    # staging halves smaller than the largest stream
    small = torch.empty(2 * 256 * ((max(h.numel() for h in host) - 1) // 256), dtype=torch.uint8, device=cuda)
    st, failed = kvc.kvc_reload(host, mu, sig, prefix, out, staging=small)
    assert st == kvc.KVC_ERR_CAPACITY
    # an output too small for what the headers describe
    st, failed = kvc.kvc_reload(host, mu, sig, prefix, out[:, :, :-1].contiguous())
    assert st == kvc.KVC_ERR_INVALID and failed == 0
