"""The oracle's encoder over many planes at once, in worker processes (test
infrastructure, like the rest of this package).

Chunks depend only on their own rows of KV and mu, their 64 sigmas and the
marginal prefix, so a range of planes coded on its own yields exactly the
payloads that the same planes take in a stream of the whole cache.  Workers
are started from a fresh interpreter (the forkserver method), never forked
from a process that holds a GPU; they import only numpy and the oracle.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from . import kvc_oracle as K


def _encode_planes(args):
    """Code a range of planes with the oracle and compare its payload bytes
    with the expected ones; returns (equal, the range's own directory,
    index of the first differing chunk or -1)."""
    (kv, mu, sig, pref, kv_dtype, mu_dtype, w_n, w_w, tc, sigma_block_tokens, expect, batch, narrow_dof) = args
    st = K.encode(kv, mu, sig, pref, kv_dtype, mu_dtype, w_n, w_w, tc, batch_chunks=batch,
                  sigma_block_tokens=sigma_block_tokens, narrow_dof=narrow_dof)
    h = K.parse_header(st)
    n = h["n_chunks"]
    pay = K.HEADER_BYTES + 8 * (n + 1)
    directory = np.frombuffer(st, dtype="<u8", count=n + 1, offset=K.HEADER_BYTES).astype(np.int64)
    payload = st[pay:]
    if payload == expect:
        return True, directory, -1
    bad = -1
    for c in range(n):
        if payload[directory[c]:directory[c + 1]] != expect[directory[c]:directory[c + 1]]:
            bad = c
            break
    return False, directory, bad


def workers() -> int:
    """Worker count: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class Pool:
    """A process pool for :func:`_encode_planes` jobs."""

    def __init__(self, n: int | None = None):
        self.n = n or workers()
        self._pool = mp.get_context("forkserver").Pool(self.n)

    def submit(self, kv, mu, sig, pref, kv_dtype, mu_dtype, w_n, w_w, tc, expect: bytes,
               sigma_block_tokens: int = 0, batch: int = 64, narrow_dof: int = 0):
        return self._pool.apply_async(_encode_planes, ((kv, mu, sig, pref, kv_dtype, mu_dtype, w_n, w_w, tc,
                                                        sigma_block_tokens, expect, batch, narrow_dof),))

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self._pool.terminate()
        self._pool.join()
