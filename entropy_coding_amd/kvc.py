"""ctypes binding over libkvc.so (C ABI in include/kvc.h).

Argument marshalling only: every step of the coder runs in the library's
HIP kernels.  torch supplies device memory and the current HIP stream.
Importing this module loads the library and raises ImportError if it has not
been built (``python -m entropy_coding_amd.build``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVC_LIBRARY names another build of the same library (the CPU tests load
# the sanitizer build this way); by default the in-tree libkvc.so.
LIB_PATH = os.environ.get("KVC_LIBRARY") or os.path.join(_HERE, "libkvc.so")

KVC_OK, KVC_ERR_INVALID, KVC_ERR_CAPACITY, KVC_ERR_CORRUPT, KVC_ERR_MISMATCH, KVC_ERR_DEVICE = 0, -1, -2, -3, -4, -5
KVC_BF16, KVC_E4M3, KVC_F32 = 0, 1, 2
HEADER_BYTES = 128
DECODE_WORKSPACE_BYTES = 917504
NOALLOC_SCRATCH_BYTES = 917504
ESTIMATE_WORKSPACE_BYTES = 256
ENCODE_STAGES = 2     # side-information checksum + per-call tables, coding kernel (with the stream's layout)
DECODE_STAGES = 2     # side-information checksum + escape bucket table, decoding kernel

EXPORTS = [
    "kvc_version", "kvc_status_string", "kvc_phi_tables", "kvc_narrow_table", "kvc_encode_sizes", "kvc_encode", "kvc_encode_result",
    "kvc_stream_info", "kvc_decode", "kvc_decode_async", "kvc_decode_result", "kvc_decode_noalloc",
    "kvc_decode_paged", "kvc_reload",
    "kvc_calibrate_sigma", "kvc_calibrate_sigma_blocks", "kvc_calibrate_sigma_rate", "kvc_calibrate_split",
    "kvc_build_marginal", "kvc_estimate_bits", "kvc_cdf_table",
]

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m entropy_coding_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)


class kvc_params(ctypes.Structure):
    _fields_ = [
        ("kv_dtype", ctypes.c_int32), ("mu_dtype", ctypes.c_int32),
        ("w_narrow_bp", ctypes.c_uint32), ("w_wide_bp", ctypes.c_uint32),
        ("chunk_tokens", ctypes.c_uint32), ("sigma_block_tokens", ctypes.c_uint32),
        ("narrow_dof", ctypes.c_uint32), ("channel_split", ctypes.c_uint32),
        ("planes", ctypes.c_int64), ("tokens", ctypes.c_int64), ("channels", ctypes.c_int64),
    ]


class kvc_paged_kv(ctypes.Structure):
    _fields_ = [
        ("d_pools", ctypes.c_void_p), ("d_block_table", ctypes.c_void_p),
        ("n_pools", ctypes.c_int64), ("pool_bytes", ctypes.c_uint64),
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("max_pages", ctypes.c_int64),
        ("num_pages", ctypes.c_int64), ("page_tokens", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
    ]


class kvc_encode_info(ctypes.Structure):
    _fields_ = [("stage_ms", ctypes.c_float * ENCODE_STAGES)]


class kvc_decode_info(ctypes.Structure):
    _fields_ = [("stage_ms", ctypes.c_float * 2), ("reserved", ctypes.c_uint32),
                ("fallback_symbols", ctypes.c_uint64)]


_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_version = _sig("kvc_version", ctypes.c_int, [])
_lib_status_string = _sig("kvc_status_string", ctypes.c_char_p, [ctypes.c_int])
_lib_phi_tables = _sig("kvc_phi_tables", ctypes.c_int, [_P, _P])
_lib_narrow_table = _sig("kvc_narrow_table", ctypes.c_int, [_U32, _P])
_lib_encode_sizes = _sig("kvc_encode_sizes", ctypes.c_int, [ctypes.POINTER(kvc_params), ctypes.POINTER(_U64), ctypes.POINTER(_U64)])
_lib_encode = _sig("kvc_encode", ctypes.c_int,
                   [ctypes.POINTER(kvc_params), _P, _P, _P, _P, _P, _U64, ctypes.POINTER(_U64), _P, _P, _U64, _P, _P])
_lib_encode_result = _sig("kvc_encode_result", ctypes.c_int, [_P, _P, ctypes.POINTER(_U64), _P])
_lib_stream_info = _sig("kvc_stream_info", ctypes.c_int, [_P, _U64, ctypes.POINTER(kvc_params), ctypes.POINTER(_U64)])
_DECODE_ARGS = [_P, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P]
_lib_decode = _sig("kvc_decode", ctypes.c_int, _DECODE_ARGS + [_P])
_lib_decode_async = _sig("kvc_decode_async", ctypes.c_int, _DECODE_ARGS)
_lib_decode_result = _sig("kvc_decode_result", ctypes.c_int, [_P, _P, _P])
_lib_reload = _sig("kvc_reload", ctypes.c_int,
                   [_I64, _P, _P, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P, _P,
                    ctypes.POINTER(_I64)])
_lib_decode_noalloc = _sig("kvc_decode_noalloc", ctypes.c_int, [_P, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P, _U64, _P])
_lib_decode_paged = _sig("kvc_decode_paged", ctypes.c_int,
                         [_P, _P, _U64, _P, _U64, _P, _U64, _P, _U64, ctypes.POINTER(kvc_paged_kv), _P, _U64, _P, _P])
_lib_calibrate = _sig("kvc_calibrate_sigma", ctypes.c_int,
                      [_P, _P, _I32, _I32, _I64, _I64, _I64, _I64, ctypes.c_float, _P, _P, _U64, _P])
_lib_calibrate_blocks = _sig("kvc_calibrate_sigma_blocks", ctypes.c_int,
                             [_P, _P, _I32, _I32, _I64, _I64, _I64, _I64, _I64, ctypes.c_float, _P, _P, _U64, _P])
_lib_calibrate_rate = _sig("kvc_calibrate_sigma_rate", ctypes.c_int,
                           [_P, _P, _I32, _I32, _I64, _I64, _I64, _I64, _I64, ctypes.c_float, _U32, _U32, _U32, _P,
                            _P, _P, _U64, _P])
_lib_calibrate_split = _sig("kvc_calibrate_split", ctypes.c_int,
                            [_P, _P, _I32, _I32, _I64, _I64, _I64, _I64, _I64, _P, _U32, _U32, _U32, _P, _P, _P, _U64,
                             _P])
_lib_marginal = _sig("kvc_build_marginal", ctypes.c_int, [_P, _I32, _U64, _U32, _U32, _P, _P])
_lib_estimate = _sig("kvc_estimate_bits", ctypes.c_int, [ctypes.POINTER(kvc_params), _P, _P, _P, _P, _P, _P, _U64, _P])
_lib_cdf_table = _sig("kvc_cdf_table", ctypes.c_int, [_I32, _I32, _U32, _U32, _U32, _P, _P, _I64, _P, _P, _P])


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvc_status_string(status)} ({status})")


def _check(st: int, where: str):
    if st != KVC_OK:
        raise KvcError(st, where)


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _host_header(header) -> np.ndarray:
    """A host copy of a stream header (bytes, numpy or a device tensor holding
    at least the header) as a contiguous 128-byte array."""
    if isinstance(header, torch.Tensor):
        header = header[:HEADER_BYTES].cpu().numpy()
    h = np.frombuffer(bytes(header[:HEADER_BYTES]), dtype=np.uint8).copy()
    if h.size != HEADER_BYTES:
        raise KvcError(KVC_ERR_CORRUPT, "stream header")
    return h


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16 or t.dtype == torch.int16:
        return KVC_BF16
    if t.dtype == torch.float8_e4m3fn or t.dtype == torch.uint8:
        return KVC_E4M3
    raise TypeError(f"KV must be bf16 (or int16 patterns) or e4m3 (or uint8 patterns), got {t.dtype}")


def _mu_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16 or t.dtype == torch.int16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError(f"mu must be bf16 or float32, got {t.dtype}")


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def kvc_version() -> int:
    return _lib_version()


def kvc_status_string(status: int) -> str:
    return _lib_status_string(status).decode()


def kvc_phi_tables():
    """(narrow, wide) base tables of the library, computed on the host."""
    a = np.zeros(12289, dtype=np.uint32)
    b = np.zeros(12289, dtype=np.uint32)
    _check(_lib_phi_tables(a.ctypes.data, b.ctypes.data), "kvc_phi_tables")
    return a, b


def kvc_narrow_table(narrow_dof: int = 0):
    """The narrow part's base table (Phi, or Student's t with narrow_dof
    degrees of freedom), computed on the host."""
    a = np.zeros(12289, dtype=np.uint32)
    _check(_lib_narrow_table(narrow_dof, a.ctypes.data), "kvc_narrow_table")
    return a


def make_params(kv_dtype, mu_dtype, planes, tokens, channels, weights=(9500, 300), chunk_tokens=0,
                sigma_block_tokens=0, narrow_dof=0, channel_split=0) -> kvc_params:
    return kvc_params(kv_dtype, mu_dtype, weights[0], weights[1], chunk_tokens, sigma_block_tokens,
                      narrow_dof, channel_split, planes, tokens, channels)


def side_info(sigma: torch.Tensor, channel_split: torch.Tensor) -> torch.Tensor:
    """The side buffer of a stream with per-channel weights: sigma's words,
    then the narrow weights [G, D] (basis points) as uint32 words, in one
    float32 device tensor (pass it wherever sigma goes)."""
    w = channel_split.to(torch.int32).contiguous()
    return torch.cat([sigma.reshape(-1).to(torch.float32), w.view(torch.float32).reshape(-1)])


def sigma_shape(planes: int, tokens: int, channels: int, sigma_block_tokens: int = 0):
    """Shape of sigma: [G, D], or [G, ceil(T / B), D] with sigma blocks."""
    if sigma_block_tokens == 0:
        return (planes, channels)
    return (planes, -(-tokens // sigma_block_tokens), channels)


def kvc_encode_sizes(p: kvc_params):
    a, b = _U64(), _U64()
    _check(_lib_encode_sizes(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b)), "kvc_encode_sizes")
    return a.value, b.value


class Encoder:
    """Holds the output and workspace buffers of one shape so that repeated
    calls allocate nothing."""

    def __init__(self, p: kvc_params, device="cuda", out_capacity: int | None = None):
        self.p = p
        max_stream, ws = kvc_encode_sizes(p)
        self.capacity = max_stream if out_capacity is None else out_capacity
        self.out = torch.empty(self.capacity, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.header = np.zeros(HEADER_BYTES, dtype=np.uint8)     # host copy of the last stream's header

    def _check_inputs(self, kv, mu, sigma):
        p = self.p
        n = p.planes * p.tokens * p.channels
        if kv.numel() != n or mu.numel() != n or _kv_dtype(kv) != p.kv_dtype or _mu_dtype(mu) != p.mu_dtype:
            raise ValueError("kv / mu do not match the encoder's parameters")
        words = math.prod(sigma_shape(p.planes, p.tokens, p.channels, p.sigma_block_tokens))
        if p.channel_split:
            words += p.planes * p.channels                  # the narrow weights follow sigma
        if sigma.numel() != words:
            raise ValueError("sigma does not match the encoder's parameters")

    def __call__(self, kv, mu, sigma, prefix=None, stream=None, info: dict | None = None) -> torch.Tensor:
        self._check_inputs(kv, mu, sigma)
        n = _U64(0)
        inf = kvc_encode_info() if info is not None else None
        st = _lib_encode(ctypes.byref(self.p), _ptr(kv), _ptr(mu), _ptr(sigma), _ptr(prefix),
                         _ptr(self.out), self.capacity, ctypes.byref(n), self.header.ctypes.data,
                         _ptr(self.workspace), self.workspace.numel(), _stream(stream),
                         ctypes.byref(inf) if inf is not None else None)
        _check(st, "kvc_encode")
        if inf is not None:
            info["stage_ms"] = list(inf.stage_ms)
        return self.out[: n.value]

    def enqueue(self, kv, mu, sigma, prefix=None, stream=None):
        """Queue an encode without waiting for it; result() gives the stream."""
        self._check_inputs(kv, mu, sigma)
        st = _lib_encode(ctypes.byref(self.p), _ptr(kv), _ptr(mu), _ptr(sigma), _ptr(prefix),
                         _ptr(self.out), self.capacity, None, None, _ptr(self.workspace), self.workspace.numel(),
                         _stream(stream), None)
        _check(st, "kvc_encode")

    def result(self, stream=None) -> torch.Tensor:
        n = _U64(0)
        _check(_lib_encode_result(_ptr(self.workspace), _stream(stream), ctypes.byref(n), self.header.ctypes.data),
               "kvc_encode_result")
        return self.out[: n.value]


def kvc_encode(kv: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor, prefix: torch.Tensor | None = None,
               weights=(9500, 300), chunk_tokens: int = 0, stream=None,
               sigma_block_tokens: int = 0, narrow_dof: int = 0,
               channel_split: torch.Tensor | None = None) -> torch.Tensor:
    """Encode KV [G, T, D] under the mixture around mu with sigma [G, D] (or
    [G, ceil(T / B), D] with sigma_block_tokens = B) and, when channel_split
    [G, D] is given, each channel's own narrow weight (decode then takes
    side_info(sigma, channel_split) as its sigma); returns the stream as a
    uint8 device tensor."""
    for t, nm in ((kv, "kv"), (mu, "mu"), (sigma, "sigma")):
        _need(t, nm)
    if prefix is not None:
        _need(prefix, "prefix")
    g, t, d = kv.shape
    if tuple(mu.shape) != (g, t, d) or tuple(sigma.shape) != sigma_shape(g, t, d, sigma_block_tokens) \
            or sigma.dtype != torch.float32:
        raise ValueError("shapes: kv and mu [G, T, D], sigma [G, D] (or [G, ceil(T / B), D]) float32")
    split = 0
    if channel_split is not None:
        if tuple(channel_split.shape) != (g, d):
            raise ValueError("channel_split is [G, D]")
        sigma = side_info(sigma, channel_split)
        split = 1
    p = make_params(_kv_dtype(kv), _mu_dtype(mu), g, t, d, weights, chunk_tokens, sigma_block_tokens, narrow_dof,
                    split)
    return Encoder(p, kv.device)(kv, mu, sigma, prefix, stream).clone()


def kvc_stream_info(header: bytes | np.ndarray):
    h = np.frombuffer(bytes(header[:HEADER_BYTES]), dtype=np.uint8).copy()
    p = kvc_params()
    total = _U64()
    _check(_lib_stream_info(h.ctypes.data, h.size, ctypes.byref(p), ctypes.byref(total)), "kvc_stream_info")
    return p, total.value


def _decode_args(header, stream_bytes, mu, sigma, prefix, kv_out, workspace, stream):
    h = _host_header(stream_bytes if header is None else header)
    args = [h.ctypes.data, _ptr(stream_bytes), stream_bytes.numel(), _ptr(mu), _nbytes(mu), _ptr(sigma),
            _nbytes(sigma), _ptr(prefix), _nbytes(prefix), _ptr(kv_out), _nbytes(kv_out), _ptr(workspace),
            _nbytes(workspace), _stream(stream)]
    return h, args


def kvc_decode(stream_bytes: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor,
               prefix: torch.Tensor | None = None, kv_out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None, header=None) -> torch.Tensor:
    """Decode a KVC-1 stream (uint8 device tensor) back to KV bit patterns
    (int16 for bf16, uint8 for e4m3), shape [G, T, D].  header: a host copy
    of the stream's first 128 bytes; read from the device stream if None."""
    _need(stream_bytes, "stream")
    for t, nm in ((mu, "mu"), (sigma, "sigma")):
        _need(t, nm)
    if stream_bytes.numel() < HEADER_BYTES:
        raise KvcError(KVC_ERR_CORRUPT, "kvc_decode")
    h = _host_header(stream_bytes if header is None else header)
    p, _ = kvc_stream_info(h)
    shape = (p.planes, p.tokens, p.channels)
    if kv_out is None:
        kv_out = torch.empty(shape, dtype=torch.int16 if p.kv_dtype == KVC_BF16 else torch.uint8,
                             device=stream_bytes.device)
    if workspace is None:
        workspace = torch.empty(DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=stream_bytes.device)
    _, args = _decode_args(h, stream_bytes, mu, sigma, prefix, kv_out, workspace, stream)
    _check(_lib_decode(*args, None), "kvc_decode")
    return kv_out


def kvc_decode_into(stream_bytes, mu, sigma, prefix, kv_out, workspace, stream=None,
                    info: dict | None = None, header=None) -> int:
    """Decode into kv_out and return the status instead of raising (for
    timing loops and error-path tests).  header: a host copy of the stream's
    header (bytes or numpy); read from the device stream if None."""
    inf = kvc_decode_info() if info is not None else None
    try:
        _, args = _decode_args(header, stream_bytes, mu, sigma, prefix, kv_out, workspace, stream)
    except KvcError as e:                 # fewer bytes than a header
        return e.status
    st = _lib_decode(*args, ctypes.byref(inf) if inf is not None else None)
    if inf is not None:
        info["stage_ms"] = list(inf.stage_ms)
        info["fallback_symbols"] = inf.fallback_symbols
    return st


def kvc_decode_async(stream_bytes, mu, sigma, prefix, kv_out, workspace, header, stream=None) -> int:
    """Queue a decode (host checks only); kvc_decode_result gives its status."""
    _, args = _decode_args(header, stream_bytes, mu, sigma, prefix, kv_out, workspace, stream)
    return _lib_decode_async(*args)


def kvc_decode_result(workspace, stream=None, info: dict | None = None) -> int:
    inf = kvc_decode_info()
    st = _lib_decode_result(_ptr(workspace), _stream(stream), ctypes.byref(inf))
    if info is not None:
        info["fallback_symbols"] = inf.fallback_symbols
    return st


def kvc_decode_noalloc(stream_bytes, mu, sigma, prefix, kv_out, stream=None, header=None) -> int:
    """Decode into kv_out with the library's fixed device scratch (no
    workspace, nothing allocated); returns the status.  Calls on one device
    share the scratch and must not overlap."""
    try:
        h = _host_header(stream_bytes if header is None else header)
    except KvcError as e:
        return e.status
    return _lib_decode_noalloc(h.ctypes.data, _ptr(stream_bytes), stream_bytes.numel(), _ptr(mu), _nbytes(mu),
                               _ptr(sigma), _nbytes(sigma), _ptr(prefix), _nbytes(prefix), _ptr(kv_out),
                               _nbytes(kv_out), _stream(stream))


def kvc_reload(host_streams, mu: torch.Tensor, sigma: torch.Tensor, prefix, kv_out: torch.Tensor,
               staging: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
               copy_stream=None):
    """Decode the per-layer streams in `host_streams` (uint8 CPU tensors,
    pinned for asynchronous copies) into kv_out[l], with mu[l], sigma[l] and
    the shared prefix; copies overlap the decodes (the library's pipeline).
    Returns (status, index of the first failing layer or -1)."""
    n = len(host_streams)
    for t in host_streams:
        if t.is_cuda or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("host streams must be contiguous uint8 CPU tensors")
    for t, nm in ((mu, "mu"), (sigma, "sigma"), (kv_out, "kv_out")):
        _need(t, nm)
        if t.shape[0] != n:
            raise ValueError(f"{nm} must have one entry per stream")
    dev = kv_out.device
    if staging is None:
        half = max(t.numel() for t in host_streams) + 255
        staging = torch.empty(2 * (half // 256 * 256 + 256), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(n * DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=dev)
    ptrs = (ctypes.c_void_p * n)(*[t.data_ptr() for t in host_streams])
    sizes = (ctypes.c_uint64 * n)(*[t.numel() for t in host_streams])
    failed = _I64(-1)
    st = _lib_reload(n, ptrs, sizes, _ptr(mu), _nbytes(mu) // n, _ptr(sigma), _nbytes(sigma) // n, _ptr(prefix),
                     _nbytes(prefix), _ptr(kv_out), _nbytes(kv_out) // n, _ptr(staging), _nbytes(staging),
                     _ptr(workspace), _nbytes(workspace), _stream(stream), copy_stream.cuda_stream,
                     ctypes.byref(failed))
    return st, failed.value


class PagedKV:
    """A paged KV cache as the library sees it: one pool per (layer, kv),
    each [num_pages, page_tokens, heads, channels], and a block table
    [batch, max_pages] of int32 page numbers shared by every pool.  Holds
    the device array of pool pointers that the call reads."""

    def __init__(self, pools, block_table: torch.Tensor, page_tokens: int):
        pools = list(pools)
        if not pools:
            raise ValueError("no pools")
        for t in pools:
            _need(t, "pool")
        _need(block_table, "block_table")
        if block_table.dtype != torch.int32 or block_table.dim() != 2:
            raise ValueError("block_table must be int32 [batch, max_pages]")
        if pools[0].dim() != 4:
            raise ValueError("pools must be [num_pages, page_tokens, heads, channels]")
        n_pages, pt, heads, _ = pools[0].shape
        if pt != page_tokens or any(tuple(t.shape) != tuple(pools[0].shape) or t.dtype != pools[0].dtype
                                    for t in pools):
            raise ValueError("pools must all be [num_pages, page_tokens, heads, channels] of one dtype")
        self.pools = pools
        self.block_table = block_table
        self.ptrs = torch.tensor([t.data_ptr() for t in pools], dtype=torch.int64, device=block_table.device)
        self.channels = pools[0].shape[3]
        self.dtype = pools[0].dtype
        self.desc = kvc_paged_kv(self.ptrs.data_ptr(), block_table.data_ptr(), len(pools), _nbytes(pools[0]),
                                 block_table.shape[0], heads, block_table.shape[1], n_pages, page_tokens, 0)


def kvc_decode_paged(stream_bytes, mu, sigma, prefix, paged: PagedKV, workspace, stream=None,
                     info: dict | None = None, header=None) -> int:
    """Decode straight into a paged KV cache; returns the status.  The pools'
    channels and element type must be the stream's (checked here against
    the header; the library checks the pool count and sizes)."""
    h = _host_header(stream_bytes if header is None else header)
    p, _ = kvc_stream_info(h)
    esize = 2 if p.kv_dtype == KVC_BF16 else 1
    if paged.channels != p.channels or torch.empty(0, dtype=paged.dtype).element_size() != esize:
        return KVC_ERR_INVALID
    inf = kvc_decode_info() if info is not None else None
    st = _lib_decode_paged(h.ctypes.data, _ptr(stream_bytes), stream_bytes.numel(), _ptr(mu), _nbytes(mu),
                           _ptr(sigma), _nbytes(sigma), _ptr(prefix), _nbytes(prefix), ctypes.byref(paged.desc),
                           _ptr(workspace), _nbytes(workspace), _stream(stream),
                           ctypes.byref(inf) if inf is not None else None)
    if inf is not None:
        info["stage_ms"] = list(inf.stage_ms)
        info["fallback_symbols"] = inf.fallback_symbols
    return st


def calibrate_workspace_bytes(planes: int, channels: int) -> int:
    return planes * channels * 1024


def kvc_calibrate_sigma(kv: torch.Tensor, mu: torch.Tensor, sigma_floor: float = 2.0 ** -30,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None, block_tokens: int = 0) -> torch.Tensor:
    """kv, mu: [reps, planes, tokens, channels] -> sigma [planes, channels],
    or with block_tokens = B > 0 sigma [planes, ceil(tokens / B), channels]
    (one sigma per block of B tokens)."""
    _need(kv, "kv")
    _need(mu, "mu")
    r, g, t, d = kv.shape
    shape = sigma_shape(g, t, d, block_tokens)
    n_rows = g if block_tokens == 0 else g * shape[1]
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=kv.device)
    if workspace is None:
        workspace = torch.empty(calibrate_workspace_bytes(n_rows, d), dtype=torch.uint8, device=kv.device)
    if block_tokens == 0:
        st = _lib_calibrate(_ptr(kv), _ptr(mu), _kv_dtype(kv), _mu_dtype(mu), r, g, t, d, sigma_floor,
                            _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    else:
        st = _lib_calibrate_blocks(_ptr(kv), _ptr(mu), _kv_dtype(kv), _mu_dtype(mu), r, g, t, d, block_tokens,
                                   sigma_floor, _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "kvc_calibrate_sigma")
    return out


def kvc_calibrate_sigma_rate(kv: torch.Tensor, mu: torch.Tensor, prefix: torch.Tensor | None = None,
                             weights=(9500, 300), sigma_floor: float = 2.0 ** -30, block_tokens: int = 0,
                             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             stream=None, narrow_dof: int = 0) -> torch.Tensor:
    """Rate-fitted sigma: of the candidates max(floor, rms * (1 - j/32)),
    j = 0..24, the one with the least integer code length of the held-out
    kv [reps, planes, tokens, channels] under the mixture the data will be
    coded with.  Shapes as kvc_calibrate_sigma."""
    _need(kv, "kv")
    _need(mu, "mu")
    r, g, t, d = kv.shape
    shape = sigma_shape(g, t, d, block_tokens)
    n_rows = g if block_tokens == 0 else g * shape[1]
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=kv.device)
    if workspace is None:
        workspace = torch.empty(n_rows * d * (1024 + 12800) + 65536, dtype=torch.uint8, device=kv.device)
    st = _lib_calibrate_rate(_ptr(kv), _ptr(mu), _kv_dtype(kv), _mu_dtype(mu), r, g, t, d, block_tokens,
                             sigma_floor, weights[0], weights[1], narrow_dof, _ptr(prefix), _ptr(out), _ptr(workspace),
                             workspace.numel(), _stream(stream))
    _check(st, "kvc_calibrate_sigma_rate")
    return out


def kvc_calibrate_split(kv: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor, prefix: torch.Tensor | None = None,
                        weights=(9500, 300), block_tokens: int = 0, narrow_dof: int = 0,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Per-channel narrow weights: of w_j = max(w_n + w_w - 200 j, 0),
    j = 0..15, the one with the least integer code length of the held-out
    kv [reps, planes, tokens, channels] under sigma (the one the stream will
    use: [G, D], or [G, ceil(T / B), D] with block_tokens = B).  Returns
    int32 [G, D]."""
    _need(kv, "kv")
    _need(mu, "mu")
    _need(sigma, "sigma")
    r, g, t, d = kv.shape
    if out is None:
        out = torch.empty((g, d), dtype=torch.int32, device=kv.device)
    if workspace is None:
        workspace = torch.empty(g * d * 8192, dtype=torch.uint8, device=kv.device)
    st = _lib_calibrate_split(_ptr(kv), _ptr(mu), _kv_dtype(kv), _mu_dtype(mu), r, g, t, d, block_tokens, _ptr(sigma),
                              weights[0], weights[1], narrow_dof, _ptr(prefix), _ptr(out), _ptr(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, "kvc_calibrate_split")
    return out


def kvc_build_marginal(samples: torch.Tensor, weights=(9500, 300), stream=None) -> torch.Tensor:
    """Prefix table of the +1-smoothed marginal; returned as int32 (all
    values are below 2^31) with N + 1 entries."""
    _need(samples, "samples")
    dt = _kv_dtype(samples)
    n_sym = 65536 if dt == KVC_BF16 else 256
    out = torch.empty(n_sym + 1, dtype=torch.int32, device=samples.device)
    st = _lib_marginal(_ptr(samples), dt, samples.numel(), weights[0], weights[1], _ptr(out), _stream(stream))
    _check(st, "kvc_build_marginal")
    return out


def kvc_estimate_bits(kv, mu, sigma, prefix=None, weights=(9500, 300), stream=None, sigma_block_tokens: int = 0,
                      chunk_tokens: int = 0, narrow_dof: int = 0, channel_split: torch.Tensor | None = None):
    """(integer-model bits/scalar, float-model bits/scalar)."""
    g, t, d = kv.shape
    if channel_split is not None:
        sigma = side_info(sigma, channel_split)
    p = make_params(_kv_dtype(kv), _mu_dtype(mu), g, t, d, weights, chunk_tokens, sigma_block_tokens, narrow_dof,
                    0 if channel_split is None else 1)
    ws = torch.empty(ESTIMATE_WORKSPACE_BYTES, dtype=torch.uint8, device=kv.device)
    out = (ctypes.c_double * 2)()
    st = _lib_estimate(ctypes.byref(p), _ptr(kv), _ptr(mu), _ptr(sigma), _ptr(prefix), ctypes.addressof(out),
                       _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kvc_estimate_bits")
    return out[0], out[1]


def kvc_cdf_table(kv_dtype: int, mu: torch.Tensor, sigma: torch.Tensor, prefix=None, weights=(9500, 300),
                  stream=None, narrow_dof: int = 0) -> torch.Tensor:
    """C(b) for b = 0..N for each (mu, sigma) pair; int32 storage of uint32
    values (reinterpret as uint32 on the host)."""
    _need(mu, "mu")
    _need(sigma, "sigma")
    n_sym = 65536 if kv_dtype == KVC_BF16 else 256
    pairs = mu.numel()
    out = torch.empty((pairs, n_sym + 1), dtype=torch.int32, device=mu.device)
    st = _lib_cdf_table(kv_dtype, _mu_dtype(mu), weights[0], weights[1], narrow_dof, _ptr(mu), _ptr(sigma), pairs,
                        _ptr(prefix), _ptr(out), _stream(stream))
    _check(st, "kvc_cdf_table")
    return out
