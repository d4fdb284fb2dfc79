"""Seeded synthetic KV workloads (input generators only: no coder arithmetic).

The pages measure on Qwen3 KV caches of C4 prompts and calibrate sigma on
128 C4 sequences of 1024 tokens; neither weights nor data are available, so
these generators stand in for them with the Qwen3 shapes (8 KV heads, head
dim 128) and residual statistics of the kind the pages describe: an FP8-like
predictor mean plus a long-tailed residual ([wiki] 'Speculative KV Coding',
§ mixture distribution; [blog] § engineering choice of predictor).

Layout: KV and mu are [G, T, D] with G = layers * 2 (K, V) * batch * heads
planes in that order, channel fastest.  sigma is [G, D] (or [G, blocks, D]
with one sigma per block of tokens).  Everything is drawn
with torch generators on the requested device, one seed per (purpose, layer),
so a long configuration can be produced one layer at a time.
"""

from __future__ import annotations

import dataclasses
import math

import torch

BF16, E4M3, F32 = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    layers: int
    batch: int
    heads: int
    tokens: int
    channels: int
    kv_dtype: int
    mu_dtype: int
    w_narrow_bp: int
    w_wide_bp: int
    rope_k_scale: bool        # upper 64 K channels get an 8x larger scale
    outliers: bool            # residual = 85% t3 / 14.5% normal / 0.5% 20x normal
    calib_reps: int           # 0: use the generating sigma directly
    calib_tokens: int
    chunk_tokens: int         # the library's default for the call shape (one layer per call for id 4)
    position_scale: bool = False   # residual scale varies with token position (see position_factor)

    @property
    def planes_per_layer(self) -> int:
        return 2 * self.batch * self.heads

    @property
    def planes(self) -> int:
        return self.layers * self.planes_per_layer

    @property
    def n_scalars(self) -> int:
        return self.planes * self.tokens * self.channels

    @property
    def kv_bytes(self) -> int:
        return self.n_scalars * (2 if self.kv_dtype == BF16 else 1)


WORKLOADS = {
    0: Workload(0, "tiny bf16 KV (1 layer, 8 KV heads, 512 tokens)", 1, 1, 8, 512, 128,
                BF16, BF16, 9500, 300, False, False, 0, 0, 512),
    1: Workload(1, "Qwen3-0.6B-shaped bf16 KV (28 layers, 1024 tokens)", 28, 1, 8, 1024, 128,
                BF16, BF16, 9500, 300, True, False, 8, 1024, 256),
    2: Workload(2, "Qwen3-8B-shaped bf16 KV (36 layers, batch 4, 4096 tokens)", 36, 4, 8, 4096, 128,
                BF16, BF16, 9500, 300, True, True, 128, 1024, 586),
    3: Workload(3, "FP8 e4m3 KV (36 layers, 8192 tokens, fp32 predictor)", 36, 1, 8, 8192, 128,
                E4M3, F32, 9500, 300, False, False, 128, 1024, 586),
    4: Workload(4, "Qwen3-32B-shaped long-context bf16 KV (64 layers, 32768 tokens)", 64, 1, 8, 32768, 128,
                BF16, BF16, 9500, 300, True, True, 128, 1024, 256),
    5: Workload(5, "Qwen3-8B-shaped bf16 KV with position-varying residual scale (36 layers, batch 4, 4096 tokens)",
                36, 4, 8, 4096, 128, BF16, BF16, 9500, 300, True, True, 32, 4096, 586, True),
}

PURPOSE = {"params": 0, "data": 1, "calib": 2, "marginal": 3, "noise": 4, "position": 5}


def seed_for(cid: int, purpose: str, layer: int = 0) -> int:
    return (1000 * (cid + 1) + PURPOSE[purpose]) * 1000 + layer


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def layer_params(w: Workload, layer: int, device="cpu"):
    """Per-(kv, head, channel) scale s and true residual sigma of one layer:
    s ~ LogNormal(0, 0.5) (x8 on the upper 64 K channels where requested, a
    stand-in for slowly rotating RoPE pairs), sigma = 2^U(-7, -3)."""
    g = _gen(device, seed_for(w.cid, "params", layer))
    shape = (2, w.heads, w.channels)
    s = torch.exp(0.5 * torch.randn(shape, generator=g, device=device))
    if w.rope_k_scale:
        s[0, :, w.channels // 2:] *= 8.0
    sig = torch.exp2(torch.empty(shape, device=device).uniform_(-7.0, -3.0, generator=g))
    return s, sig


def _student_t3(shape, g, device):
    z = torch.randn((4,) + tuple(shape), generator=g, device=device)
    chi2 = (z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0
    return z[0] / torch.sqrt(chi2)


def _residual(w: Workload, shape, g, device):
    t3 = _student_t3(shape, g, device) / math.sqrt(3.0)
    if not w.outliers:
        return t3
    u = torch.rand(shape, generator=g, device=device)
    n = torch.randn(shape, generator=g, device=device)
    return torch.where(u < 0.85, t3, torch.where(u < 0.995, n, 20.0 * n))


def _e4m3_ulp(x: torch.Tensor) -> torch.Tensor:
    a = x.abs()
    e = torch.floor(torch.log2(torch.where(a > 0, a, torch.ones_like(a))))
    e = torch.clamp(e, min=-6.0)                # subnormals and zero: 2^-9
    return torch.exp2(e - 3.0)


def position_factor(w: Workload, layer: int, tokens: int, device="cpu"):
    """Residual scale by position, [2, heads, tokens, D] (ones unless the
    workload has position_scale).  A stand-in for position structure the
    pages point at ([blog] § limitations and future directions): on the upper
    64 K channels (the slowly rotating RoPE pairs) the scale follows
    1 + 0.75 sin(2 pi t / P + phi) with a period P = 2^U(10, 13) tokens and a
    phase phi ~ U(0, 2 pi) per (head, channel); the first 4 tokens of every
    channel (attention sinks) have 4x the residual scale."""
    f = torch.ones((2, w.heads, tokens, w.channels), device=device)
    if not w.position_scale:
        return f
    g = _gen(device, seed_for(w.cid, "position", layer))
    half = w.channels // 2
    period = torch.exp2(torch.empty((w.heads, half), device=device).uniform_(10.0, 13.0, generator=g))
    phase = torch.empty((w.heads, half), device=device).uniform_(0.0, 2.0 * math.pi, generator=g)
    t = torch.arange(tokens, device=device, dtype=torch.float32)[None, :, None]
    f[0, :, :, half:] = 1.0 + 0.75 * torch.sin(2.0 * math.pi * t / period[:, None, :] + phase[:, None, :])
    f[:, :, :4, :] *= 4.0
    return f


def _draw(w: Workload, s, sig, reps: int, tokens: int, g, device, pos=None):
    """KV and mu draws shaped [reps, 2, heads, tokens, D]; pos: the residual
    scale by position [2, heads, tokens, D] (None: 1)."""
    shape = (reps, 2, w.heads, tokens, w.channels)
    s_b = s[None, :, :, None, :]
    if w.kv_dtype == E4M3:
        kv = (torch.randn(shape, generator=g, device=device) * s_b).to(torch.float8_e4m3fn)
        kvf = kv.float()
        mu = kvf + 0.5 * _e4m3_ulp(kvf) * torch.randn(shape, generator=g, device=device)
        return kv.view(torch.uint8), mu.float()
    mu = (torch.randn(shape, generator=g, device=device) * s_b).to(torch.bfloat16)
    eps = _residual(w, shape, g, device)
    if pos is not None:
        eps = eps * pos[None]
    kv = (mu.float() + sig[None, :, :, None, :] * eps).to(torch.bfloat16)
    return kv, mu


def layer_data(w: Workload, layer: int, device="cpu", tokens: int | None = None):
    """KV and mu of one layer as [2 * batch * heads, T, D] (planes ordered
    kv, batch, head).  bf16 workloads return bfloat16 tensors; the e4m3 one
    returns KV bit patterns as uint8 and mu as float32."""
    t = w.tokens if tokens is None else tokens
    s, sig = layer_params(w, layer, device)
    g = _gen(device, seed_for(w.cid, "data", layer))
    pos = position_factor(w, layer, t, device) if w.position_scale else None
    kv, mu = _draw(w, s, sig, w.batch, t, g, device, pos)
    # [B, 2, H, T, D] -> [2, B, H, T, D]
    kv = kv.transpose(0, 1).reshape(w.planes_per_layer, t, w.channels).contiguous()
    mu = mu.transpose(0, 1).reshape(w.planes_per_layer, t, w.channels).contiguous()
    return kv, mu


def layer_sigma_true(w: Workload, layer: int, device="cpu"):
    """The generating sigma broadcast to the layer's planes: [2*B*H, D] fp32."""
    _, sig = layer_params(w, layer, device)
    return sig[:, None].expand(2, w.batch, w.heads, w.channels).reshape(-1, w.channels).contiguous().float()


def layer_calibration(w: Workload, layer: int, reps: int, device="cpu", tokens: int | None = None):
    """Held-out draws for sigma calibration: [reps, 2 * heads, tokens, D]."""
    t = w.calib_tokens if tokens is None else tokens
    s, sig = layer_params(w, layer, device)
    g = _gen(device, seed_for(w.cid, "calib", layer))
    pos = position_factor(w, layer, t, device) if w.position_scale else None
    kv, mu = _draw(w, s, sig, reps, t, g, device, pos)
    return kv.reshape(reps, 2 * w.heads, t, w.channels), mu.reshape(reps, 2 * w.heads, t, w.channels)


def expand_sigma(w: Workload, sigma_kvh: torch.Tensor) -> torch.Tensor:
    """sigma [2*H, ..., D] per (kv, head) -> [2*B*H, ..., D] per plane of one
    layer (the middle dimension, if any, is the sigma block)."""
    rest = tuple(sigma_kvh.shape[1:])
    return sigma_kvh.reshape((2, 1, w.heads) + rest).expand((2, w.batch, w.heads) + rest) \
        .reshape((-1,) + rest).contiguous()


def marginal_samples(w: Workload, n: int = 1 << 20, device="cpu"):
    """Samples of the KV marginal for p_hat, from a separate seed: 2^20
    scalars drawn from layer-0 parameters (raw bit patterns)."""
    s, sig = layer_params(w, 0, device)
    g = _gen(device, seed_for(w.cid, "marginal"))
    tokens = max(1, n // (2 * w.heads * w.channels))
    kv, _ = _draw(w, s, sig, 1, tokens, g, device)
    kv = kv.reshape(-1)[:n]
    return kv


def noise_predictor(w: Workload, shape, device="cpu"):
    """An uninformative predictor mean (independent draw of the same law)."""
    g = _gen(device, seed_for(w.cid, "noise"))
    s, _ = layer_params(w, 0, device)
    x = torch.randn(shape, generator=g, device=device) * s.reshape(-1)[: shape[-1]]
    return x.to(torch.bfloat16)


def bits_u16(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensor -> its 16-bit patterns (int16 view)."""
    return t.view(torch.int16)


def to_numpy_bits(t: torch.Tensor):
    """Host copy of raw patterns: bf16 -> uint16, uint8 stays, float32 stays."""
    import numpy as np
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def tiny_case(seed: int = 7, planes: int = 3, tokens: int = 45, channels: int = 128, kv_dtype: int = BF16):
    """A small irregular case (ragged token chunks, special values planted)
    on the CPU: returns (kv, mu, sigma, marginal samples) as torch tensors."""
    g = _gen("cpu", seed)
    shape = (planes, tokens, channels)
    s = torch.exp(0.5 * torch.randn(channels, generator=g))
    sig = torch.exp2(torch.empty(planes, channels).uniform_(-7.0, -3.0, generator=g))
    if kv_dtype == E4M3:
        kv = (torch.randn(shape, generator=g) * s).to(torch.float8_e4m3fn).view(torch.uint8)
        kvf = kv.view(torch.float8_e4m3fn).float()
        mu = kvf + 0.5 * _e4m3_ulp(kvf) * torch.randn(shape, generator=g)
        kv[0, 0, :8] = torch.tensor([0x7F, 0xFF, 0x00, 0x80, 0x7E, 0xFE, 0x01, 0x81], dtype=torch.uint8)
        samples = (torch.randn(40000, generator=g)).to(torch.float8_e4m3fn).view(torch.uint8)
        return kv, mu.float(), sig, samples
    mu = (torch.randn(shape, generator=g) * s).to(torch.bfloat16)
    eps = _student_t3(shape, g, "cpu") / math.sqrt(3.0)
    kv = (mu.float() + sig[:, None, :] * eps).to(torch.bfloat16)
    special = torch.tensor([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x8001,
                            0x7F7F, 0xFF7F, 0x7FFF, 0xFFFF], dtype=torch.int32).to(torch.int16)
    kvb = kv.view(torch.int16)
    kvb[0, 0, : special.numel()] = special
    mub = mu.view(torch.int16)
    mub[min(1, planes - 1), min(2, tokens - 1), :4] = torch.tensor([0x7FC0, 0x7F80, 0xFF80, 0x0001], dtype=torch.int32).to(torch.int16)
    samples = (torch.randn(40000, generator=g) * 1.3).to(torch.bfloat16)
    return kv, mu, sig, samples
