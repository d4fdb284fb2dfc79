"""Plain CPU oracle of the KVC-1 lossless KV-cache coder (test infrastructure).

Pages cited:
  [wiki]  "Speculative KV Coding", aisparkup.com wiki
  [blog]  "推测性KV编码：用预测模型实现缓存无损压缩4倍", blog.hotdry.top

What the pages fix: each KV scalar is coded under a model q built from a
predictor mean mu and a calibrated per-(kv, head, channel) sigma; q is the
mixture 0.95 N(mu, sigma^2) + 0.03 N(mu, (3 sigma)^2) + 0.02 p_hat, where p_hat
is the empirical marginal over the BF16 alphabet ([wiki] § mixture
distribution; [blog] § engineering choice of predictor).  An arithmetic coder
emits about -log2 q(KV) bits per scalar and the decoder, holding the same
(mu, sigma), rebuilds KV exactly ([wiki] § pipeline; [blog] § information
theory view).  The two sides must agree on the CDF bit for bit ([blog] §
application scenarios and deployment parameters).

What the pages leave open (coder type, precision, discretisation, stream
layout) is fixed by the format KVC-1; the numbered steps S-0 .. S-10 below
follow it in order.  Everything is written for clarity, not speed: NumPy
vectorises over coder lanes, Python loops over token steps.  Floating point is
used only where KVC-1 prescribes IEEE float32 steps (S-3); everything after is
exact integer arithmetic.

Position-aware sigma ([blog] § limitations and future directions: a static
per-channel sigma ignores how the residual varies with position; [wiki] §
future directions: better residual models) is the optional S-11: sigma per
(plane, block of B tokens, channel) instead of per (plane, channel).
"""

from __future__ import annotations

import functools
import struct

import numpy as np

__all__ = [
    "BF16", "E4M3", "F32", "M", "L", "LANES", "HEADER_BYTES", "STATE_BYTES", "VERSION", "StreamError",
    "alphabet_size", "budgets", "order_index", "bits_of_order", "symbol_value",
    "boundary_positions", "phi_tables", "mixture_table", "h_fx", "mu_to_f32", "cdf",
    "gauss_cum", "escape_cum",
    "cdf_table", "build_marginal", "calibrate_sigma", "side_hash", "encode",
    "decode", "parse_header", "model_bits_int", "model_bits_float",
    "chunk_layout", "sigma_blocks", "crc32", "HEADER_CRC_OFFSET", "stream_header",
    "NARROW_DOF_MAX", "student_t_cdf_mp", "narrow_table",
]

# ---------------------------------------------------------------------------
# S-0  constants
# ---------------------------------------------------------------------------
BF16, E4M3, F32 = 0, 1, 2          # dtype codes shared by the stream header
LOG2_M = 31
M = 1 << LOG2_M                    # total of every integer CDF
LOG2_L = 47
L = 1 << LOG2_L                    # lower end of the rANS state interval
WORD_BITS = 16                     # rANS emits / reads 16-bit words
LANES = 64                         # interleaved rANS lanes per chunk
HEADER_BYTES = 128
STATE_BYTES = 8 * LANES            # 64 final states, u64 each
MAGIC = b"KVC1"
VERSION = 4


class StreamError(ValueError):
    """Raised by the oracle decoder on a malformed or corrupt stream."""


def alphabet_size(dtype: int) -> int:
    """Number of symbols: every 16-bit BF16 pattern or every 8-bit e4m3fn
    pattern ([wiki] § core idea: 16 bits per BF16 scalar; [blog] §
    measured compression: FP8 e4m3 targets)."""
    if dtype == BF16:
        return 1 << 16
    if dtype == E4M3:
        return 1 << 8
    raise ValueError(f"bad kv dtype {dtype}")


def budgets(dtype: int, w_narrow_bp: int, w_wide_bp: int):
    """Integer budgets of the three mixture parts.

    The mixture weights are 0.95 / 0.03 / 0.02 ([wiki] § mixture
    distribution); in basis points (9500, 300).  N units of the total M go to
    the +1 floor that every symbol gets, the remaining T = M - N are split by
    the weights with floors, and the escape part gets what is left.
    """
    if not (0 <= w_narrow_bp and 0 <= w_wide_bp and w_narrow_bp + w_wide_bp <= 10000):
        raise ValueError("weights out of range")
    n = alphabet_size(dtype)
    t = M - n
    t_n = t * w_narrow_bp // 10000
    t_w = t * w_wide_bp // 10000
    t_e = t - t_n - t_w
    return t_n, t_w, t_e


# ---------------------------------------------------------------------------
# S-1  ordered alphabet
# ---------------------------------------------------------------------------
def order_index(bits, dtype: int) -> np.ndarray:
    """Map raw bit patterns to the value-ordered symbol index.

    Positive patterns (sign 0) keep their order above the midpoint; negative
    patterns are reversed below it.  So -NaN < -Inf < ... < -0 < +0 < ... <
    +Inf < +NaN in index order.
    """
    k = 16 if dtype == BF16 else 8
    u = np.asarray(bits).astype(np.int64) & ((1 << k) - 1)
    sign = (u >> (k - 1)) & 1
    return np.where(sign == 0, u ^ (1 << (k - 1)), (~u) & ((1 << k) - 1))


def bits_of_order(b, dtype: int) -> np.ndarray:
    """Inverse of :func:`order_index`."""
    k = 16 if dtype == BF16 else 8
    b = np.asarray(b).astype(np.int64)
    half = 1 << (k - 1)
    return np.where(b >= half, b ^ half, (~b) & ((1 << k) - 1))


def _bf16_bits_to_f64(bits) -> np.ndarray:
    u = (np.asarray(bits).astype(np.uint32) & 0xFFFF) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _e4m3_bits_to_f64(bits) -> np.ndarray:
    """OCP float8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    S.1111.111 is NaN and there is no infinity; the largest value is 448."""
    u = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where(u & 0x80, -1.0, 1.0)
    e = (u >> 3) & 0xF
    man = (u & 7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    sub = man / 8.0 * 2.0 ** -6
    mag = np.where(e == 0, sub, normal)
    mag = np.where((u & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def symbol_value(b, dtype: int) -> np.ndarray:
    """Real value (float64) of ordered symbol b."""
    bits = bits_of_order(b, dtype)
    if dtype == BF16:
        return _bf16_bits_to_f64(bits)
    return _e4m3_bits_to_f64(bits)


# ---------------------------------------------------------------------------
# S-2  boundary positions
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=None)
def boundary_positions(dtype: int) -> np.ndarray:
    """pos[b] for b = 0..N: the edge between symbols b-1 and b (float32).

    Reading (the pages write densities, not a discretisation): each finite
    value owns the round-to-nearest cell around it; the cells of -max and +max
    extend to -inf / +inf; the edge between -0 and +0 is 0; non-finite symbols
    get no Gaussian mass, so every edge at or below the lower edge of -max is
    -inf and every edge at or above the upper edge of +max is +inf.
    """
    n = alphabet_size(dtype)
    b = np.arange(n + 1, dtype=np.int64)
    vals = symbol_value(np.arange(n), dtype)
    finite = np.isfinite(vals)
    lo_sym = int(np.argmax(finite))                 # index of -max
    hi_sym = int(n - 1 - np.argmax(finite[::-1]))   # index of +max
    zero_split = int(order_index(0, dtype))         # index of +0
    pos = np.empty(n + 1, dtype=np.float64)
    inner = (b > lo_sym) & (b <= hi_sym)
    bi = b[inner]
    pos[inner] = (vals[bi - 1] + vals[bi]) / 2.0
    pos[b <= lo_sym] = -np.inf
    pos[b > hi_sym] = np.inf
    pos[zero_split] = 0.0
    out = pos.astype(np.float32)
    assert np.array_equal(out.astype(np.float64), pos), "edge not exact in float32"
    return out


# ---------------------------------------------------------------------------
# S-4  integer mixture table
# ---------------------------------------------------------------------------
TABLE_STEPS_PER_UNIT = 256          # z grid step 1/256
TABLE_Z_MAX = 24                    # z grid covers [-24, 24]
TABLE_POINTS = 2 * TABLE_Z_MAX * TABLE_STEPS_PER_UNIT + 1    # 12289


@functools.lru_cache(maxsize=None)
def phi_tables():
    """Base tables of the standard normal CDF Phi on the z grid
    z_k = -24 + k/256, k = 0..12288:
      A[k] = round(2^31 Phi(z_k))      (the N(mu, sigma^2) part),
      B[k] = round(2^31 Phi(z_k / 3))  (the N(mu, (3 sigma)^2) part).
    Phi(x) = erfc(-x / sqrt 2) / 2, evaluated with mpmath at 50 digits; no
    entry lies near a rounding tie (a test checks the margin)."""
    import mpmath

    a, b = [], []
    with mpmath.workdps(50):
        two31 = mpmath.mpf(2) ** 31
        half = mpmath.mpf(1) / 2
        r2 = mpmath.sqrt(2)
        for k in range(TABLE_POINTS):
            z = mpmath.mpf(-TABLE_Z_MAX) + mpmath.mpf(k) / TABLE_STEPS_PER_UNIT
            a.append(int(mpmath.floor(two31 * mpmath.erfc(-z / r2) / 2 + half)))
            b.append(int(mpmath.floor(two31 * mpmath.erfc(-(z / 3) / r2) / 2 + half)))
    return np.array(a, dtype=np.int64), np.array(b, dtype=np.int64)


# ---------------------------------------------------------------------------
# S-13  Student-t narrow part (optional)
# ---------------------------------------------------------------------------
NARROW_DOF_MAX = 16


def student_t_cdf_mp(z, nu: int):
    """CDF of Student's t with nu degrees of freedom (integer nu >= 1) at z,
    in mpmath at the working precision, from the finite series for integer
    degrees of freedom: with theta = atan(|z| / sqrt(nu)) and c = cos^2 theta,
    odd nu: 1/2 + (theta + sin theta cos theta (1 + 2/3 c + (2 4)/(3 5) c^2
    + ... , (nu - 1)/2 terms)) / pi; even nu: 1/2 + sin theta / 2 (1 + 1/2 c +
    (1 3)/(2 4) c^2 + ... , nu/2 terms); F(-z) = 1 - F(z)."""
    import mpmath
    z = mpmath.mpf(z)
    th = mpmath.atan(abs(z) / mpmath.sqrt(nu))
    c = mpmath.cos(th) ** 2
    term, acc = mpmath.mpf(1), mpmath.mpf(0)
    if nu % 2:
        for k in range((nu - 1) // 2):
            if k:
                term *= mpmath.mpf(2 * k) / (2 * k + 1) * c
            acc += term
        f = mpmath.mpf(1) / 2 + (th + mpmath.sin(th) * mpmath.cos(th) * acc) / mpmath.pi
    else:
        for k in range(nu // 2):
            if k:
                term *= mpmath.mpf(2 * k - 1) / (2 * k) * c
            acc += term
        f = mpmath.mpf(1) / 2 + mpmath.sin(th) / 2 * acc
    return f if z >= 0 else 1 - f


@functools.lru_cache(maxsize=None)
def narrow_table(narrow_dof: int = 0) -> np.ndarray:
    """Base table of the narrow part on the z grid.  narrow_dof = 0: the
    pages' Gaussian, A of :func:`phi_tables`.  narrow_dof = nu in
    1..NARROW_DOF_MAX: Student's t with nu degrees of freedom, location mu
    and scale sigma, truncated to [-24, 24] scale units and renormalised
    there, A[k] = floor(2^31 (F(z_k) - F(-24)) / (F(24) - F(-24)) + 1/2), so
    that A[0] = 0 and A[12288] = 2^31 as for the Gaussian.

    Reading ([wiki] § future directions and [blog] § limitations and future
    directions name a better residual model without a form; the residual of
    an FP8 predictor is long-tailed, [wiki] § mixture distribution): the
    heavy-tailed narrow part replaces the Gaussian one inside the pages'
    mixture; the wide Gaussian and the escape part stay.  nu -> infinity
    gives back the Gaussian."""
    if narrow_dof == 0:
        return phi_tables()[0]
    if not 1 <= narrow_dof <= NARROW_DOF_MAX:
        raise ValueError("narrow_dof must be 0 or 1..16")
    import mpmath
    out = []
    with mpmath.workdps(50):
        lo = student_t_cdf_mp(-TABLE_Z_MAX, narrow_dof)
        span = 1 - 2 * lo
        two31 = mpmath.mpf(2) ** 31
        half = mpmath.mpf(1) / 2
        for k in range(TABLE_POINTS):
            z = mpmath.mpf(-TABLE_Z_MAX) + mpmath.mpf(k) / TABLE_STEPS_PER_UNIT
            out.append(int(mpmath.floor(two31 * (student_t_cdf_mp(z, narrow_dof) - lo) / span + half)))
    return np.array(out, dtype=np.int64)


@functools.lru_cache(maxsize=None)
def mixture_table(t_n: int, t_w: int, narrow_dof: int = 0) -> np.ndarray:
    """H[k] = floor(T_n A[k] / 2^31) + floor(T_w B[k] / 2^31): the narrow
    and the wide part of the mixture, in integer budget units, on the z grid
    (A the narrow part's table, S-13); H[12289] repeats H[12288] so that
    interpolation may read one past the end."""
    a = narrow_table(narrow_dof)
    b = phi_tables()[1]
    h = ((t_n * a) >> 31) + ((t_w * b) >> 31)
    return np.concatenate([h, h[-1:]])


def h_fx(q, table) -> np.ndarray:
    """Integer mixture CDF of z = q / 2^24, q in [-24 2^24, 24 2^24]: table
    lookup at step 1/256 with integer linear interpolation over the 16 low
    bits."""
    q = np.asarray(q).astype(np.int64)
    if np.any(np.abs(q) > TABLE_Z_MAX << 24):
        raise ValueError("h_fx argument out of range")
    u = q + (TABLE_Z_MAX << 24)
    i = u >> 16
    r = u & 0xFFFF
    lo = table[i]
    hi = table[i + 1]
    return lo + (((hi - lo) * r) >> 16)


def split_budgets(kv_dtype: int, w_narrow_bp: int, w_wide_bp: int, split):
    """S-14: per-channel split of the Gaussian budget.  ``split`` holds, per
    (plane, channel), the narrow part's weight w_c in basis points (0 ..
    w_n + w_w); the escape weight stays the call's, so T_e, the prefix and the
    floor-and-escape slots are shared by every lane.  T_n(c) = min(floor(T
    w_c / 10^4), T_n + T_w) and T_w(c) = T_n + T_w - T_n(c): w_c = w_n gives
    back the call's (T_n, T_w).  Returns the two int64 arrays."""
    t_n, t_w, _ = budgets(kv_dtype, w_narrow_bp, w_wide_bp)
    w = np.asarray(split, dtype=np.int64)
    if np.any(w < 0) or np.any(w > w_narrow_bp + w_wide_bp):
        raise ValueError("a channel's narrow weight must lie in [0, w_n + w_w]")
    big_t = M - alphabet_size(kv_dtype)
    tn = np.minimum((big_t * w) // 10000, t_n + t_w)
    return tn, (t_n + t_w) - tn


def h_fx_lanes(q, t_n, t_w, narrow_dof: int = 0) -> np.ndarray:
    """h_fx with each element's own mixture table (S-14): the same S-4 table,
    H[k] = floor(T_n A[k] / 2^31) + floor(T_w B[k] / 2^31) with
    H[12289] = H[12288], for that element's budgets, and the same integer
    interpolation."""
    q = np.asarray(q).astype(np.int64)
    if np.any(np.abs(q) > TABLE_Z_MAX << 24):
        raise ValueError("h_fx argument out of range")
    u = q + (TABLE_Z_MAX << 24)
    i = u >> 16
    r = u & 0xFFFF
    a = narrow_table(narrow_dof)
    b = phi_tables()[1]
    a = np.concatenate([a, a[-1:]])
    b = np.concatenate([b, b[-1:]])
    tn = np.asarray(t_n, dtype=np.int64)
    tw = np.asarray(t_w, dtype=np.int64)
    lo = ((tn * a[i]) >> 31) + ((tw * b[i]) >> 31)
    hi = ((tn * a[i + 1]) >> 31) + ((tw * b[i + 1]) >> 31)
    return lo + (((hi - lo) * r) >> 16)


# ---------------------------------------------------------------------------
# S-3 / S-5  the mixture CDF
# ---------------------------------------------------------------------------
def mu_to_f32(mu, mu_dtype: int) -> np.ndarray:
    """Predictor mean as float32.  BF16 mu arrives as 16-bit patterns; F32 as
    float32.  Reading: a non-finite mu carries no location information and is
    replaced by 0 (both sides do the same, so the code stays lossless)."""
    if mu_dtype == BF16:
        m = ((np.asarray(mu).astype(np.uint32) & 0xFFFF) << 16).view(np.float32)
    elif mu_dtype == F32:
        m = np.asarray(mu, dtype=np.float32)
    else:
        raise ValueError(f"bad mu dtype {mu_dtype}")
    return np.where(np.isfinite(m), m, np.float32(0.0)).astype(np.float32)


def cdf(b, mu32, inv32, dtype: int, t_n, t_w, prefix=None, narrow_dof: int = 0) -> np.ndarray:
    """C(b): cumulative frequency below symbol b under the mixture (t_n, t_w
    the budgets, or arrays of per-element budgets broadcast with b: S-14).

    S-3  d = pos(b) - mu and z' = d * (2^24/sigma), each one IEEE float32
         operation, where 2^24/sigma is the float32 1/sigma times 2^24 (exact
         for sigma in [2^-96, 2^96]); z' clamped to [-24 * 2^24, 24 * 2^24];
         q = floor(z').  (q / 2^24 is z; the fixed-point scale is applied
         before the product so that a tiny z keeps its sign through floor.)
    S-5  C(b) = b + h_fx(q) + prefix[b]: the +1 floor of every symbol below b,
         both Gaussian parts through the mixture table, and the escape part
         as the integer prefix of the marginal.
    """
    b = np.asarray(b).astype(np.int64)
    pos = boundary_positions(dtype)[b]
    mu32 = np.asarray(mu32, dtype=np.float32)
    inv32 = np.asarray(inv32, dtype=np.float32)
    inv24 = (inv32 * np.float32(1 << 24)).astype(np.float32)
    qmax = np.float32(TABLE_Z_MAX << 24)
    with np.errstate(over="ignore", under="ignore", invalid="raise"):
        d = (pos - mu32).astype(np.float32)
        z24 = (d * inv24).astype(np.float32)
    q = np.floor(np.clip(z24, -qmax, qmax)).astype(np.int64)
    if np.ndim(t_n) == 0 and np.ndim(t_w) == 0:
        g = h_fx(q, mixture_table(t_n, t_w, narrow_dof))
    else:                                              # per-element budgets (S-14)
        g = h_fx_lanes(q, t_n, t_w, narrow_dof)
    if prefix is not None:
        g = g + np.asarray(prefix, dtype=np.int64)[b]
    return b + g


def gauss_cum(b, mu32, inv32, dtype: int, t_n, t_w, narrow_dof: int = 0) -> np.ndarray:
    """G(b) = h(q_b): the narrow and wide parts of C below symbol b, 0 .. T_n + T_w."""
    return cdf(b, mu32, inv32, dtype, t_n, t_w, None, narrow_dof) - np.asarray(b).astype(np.int64)


def escape_cum(b, prefix=None) -> np.ndarray:
    """Q(b) = b + prefix[b]: the +1 floor and the escape part of C below
    symbol b, 0 .. N + T_e.  C(b) = G(b) + Q(b)."""
    b = np.asarray(b).astype(np.int64)
    return b if prefix is None else b + np.asarray(prefix, dtype=np.int64)[b]


SIGMA_MIN = np.float32(2.0 ** -96)
SIGMA_MAX = np.float32(2.0 ** 96)


def _inv_sigma(sigma) -> np.ndarray:
    """float32 1/sigma.  Reading: sigma must lie in [2^-96, 2^96] (a KV
    residual scale far outside that range is not a calibration result)."""
    s = np.asarray(sigma, dtype=np.float32)
    ok = (s >= SIGMA_MIN) & (s <= SIGMA_MAX)
    if not np.all(ok):
        raise ValueError("sigma must lie in [2^-96, 2^96]")
    return (np.float32(1.0) / s).astype(np.float32)


def sigma_blocks(sigma, tokens: int, sigma_block_tokens: int = 0):
    """S-11  sigma as [G, n_blocks, D] and the block length in tokens.

    sigma_block_tokens = 0: one sigma per (plane, channel), sigma [G, D], one
    block covering every token.  B > 0: sigma [G, ceil(T / B), D]; token t
    of plane g, channel d uses sigma[g, t // B, d].  Reading ([blog] §
    limitations and future directions name position-aware sigma without a
    form): blocks of B consecutive tokens, the plainest position dependence
    that stays per (kv, head, channel)."""
    sg = np.asarray(sigma, dtype=np.float32)
    if sigma_block_tokens == 0:
        if sg.ndim != 2:
            raise ValueError("sigma must be [planes, channels] without sigma blocks")
        return sg[:, None, :], max(int(tokens), 1)
    nb = -(-int(tokens) // int(sigma_block_tokens))
    if sg.ndim != 3 or sg.shape[1] != nb:
        raise ValueError("sigma must be [planes, ceil(tokens / B), channels]")
    return sg, int(sigma_block_tokens)


def _check_sigma_blocks(tokens: int, chunk_tokens: int, sigma_block_tokens: int) -> None:
    """A chunk must see one sigma: B is a multiple of the chunk length, or a
    single block covers every token."""
    if sigma_block_tokens < 0:
        raise ValueError("sigma_block_tokens must be >= 0")
    if sigma_block_tokens and sigma_block_tokens < tokens and sigma_block_tokens % chunk_tokens:
        raise ValueError("sigma_block_tokens must be a multiple of chunk_tokens")


def cdf_table(mu, sigma, dtype: int, mu_dtype: int, w_narrow_bp: int,
              w_wide_bp: int, prefix=None, narrow_dof: int = 0) -> np.ndarray:
    """C(b) for every b = 0..N, for each (mu, sigma) pair: shape [P, N+1]."""
    t_n, t_w, t_e = budgets(dtype, w_narrow_bp, w_wide_bp)
    if t_e and prefix is None:
        raise ValueError("mixture with an escape part needs the marginal prefix")
    mu32 = mu_to_f32(np.atleast_1d(mu), mu_dtype)
    inv = _inv_sigma(np.atleast_1d(sigma))
    n = alphabet_size(dtype)
    b = np.arange(n + 1, dtype=np.int64)
    out = np.empty((mu32.size, n + 1), dtype=np.int64)
    for i in range(mu32.size):
        out[i] = cdf(b, mu32[i], inv[i], dtype, t_n, t_w, prefix if t_e else None, narrow_dof)
    return out


# ---------------------------------------------------------------------------
# S-6  empirical marginal (the p_hat part)
# ---------------------------------------------------------------------------
def build_marginal(samples, dtype: int, w_narrow_bp: int, w_wide_bp: int) -> np.ndarray:
    """Integer prefix table of the +1-smoothed empirical marginal.

    c[j] = 1 + number of samples whose ordered index is j; cum is its
    exclusive prefix in index order; prefix[b] = floor(T_e cum[b] / cum[N]).
    p_hat is the empirical BF16 distribution that catches extreme outliers
    ([wiki] § mixture distribution; [blog] § engineering choice of predictor).
    """
    n = alphabet_size(dtype)
    _, _, t_e = budgets(dtype, w_narrow_bp, w_wide_bp)
    idx = order_index(np.asarray(samples).ravel(), dtype)
    counts = np.bincount(idx, minlength=n).astype(object) + 1
    cum = [0]
    for c in counts:
        cum.append(cum[-1] + int(c))
    total = cum[-1]
    return np.array([t_e * c // total for c in cum], dtype=np.int64)


# ---------------------------------------------------------------------------
# S-7  sigma calibration
# ---------------------------------------------------------------------------
def _values_f64(x, dtype: int) -> np.ndarray:
    if dtype == BF16:
        return _bf16_bits_to_f64(x)
    if dtype == E4M3:
        return _e4m3_bits_to_f64(x)
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def calibrate_sigma(kv, mu, kv_dtype: int, mu_dtype: int, sigma_floor: float,
                    block_tokens: int = 0) -> np.ndarray:
    """sigma[p, d] = max(floor, sqrt(mean over reps and tokens of (kv - mu)^2)).

    With block_tokens = B > 0 (S-11), sigma[p, j, d] takes the mean over reps
    and the tokens [jB, min((j+1)B, T)) only.

    Inputs are [reps, planes, tokens, channels].  sigma^2 is the mean squared
    residual about mu: it minimises the expected Gaussian cost, spread plus
    miss, of [blog] § information theory view, and the pages calibrate it per
    (kv, head, channel) on held-out data, then freeze it ([wiki] § predictor
    choice; [blog] § engineering choice of predictor).  Accumulated in float64,
    rounded once to float32.  Residuals that are not finite (a NaN or Inf in
    the calibration data) are left out of the mean; a channel with none left
    gets the floor.
    """
    k = _values_f64(kv, kv_dtype)
    m = _values_f64(mu, mu_dtype)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        r2 = (k - m) ** 2
    ok = np.isfinite(r2)                  # non-finite residuals are skipped
    r2 = np.where(ok, r2, 0.0)
    t_len = r2.shape[2]
    bounds = [(0, t_len)] if block_tokens == 0 else \
        [(j, min(j + block_tokens, t_len)) for j in range(0, t_len, block_tokens)]
    used = np.stack([ok[:, :, a:b].sum(axis=(0, 2)) for a, b in bounds], axis=1)
    total = np.stack([r2[:, :, a:b].sum(axis=(0, 2)) for a, b in bounds], axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        s = np.sqrt(total / used).astype(np.float32)
    fl = np.float32(sigma_floor)
    out = np.where((used > 0) & np.isfinite(s) & (s > fl), s, fl).astype(np.float32)
    return out[:, 0, :] if block_tokens == 0 else out


# ---------------------------------------------------------------------------
# S-12  rate-fitted sigma (an optional calibration)
# ---------------------------------------------------------------------------
RATE_STEPS = 25                    # candidate multipliers k_j = 1 - j/32, j = 0..24
LOG2_TABLE_BITS = 8


@functools.lru_cache(maxsize=None)
def log2_table_q16() -> np.ndarray:
    """round(2^16 log2(1 + m/256)) for m = 0..255."""
    m = np.arange(1 << LOG2_TABLE_BITS, dtype=np.float64)
    return np.floor(65536.0 * np.log2(1.0 + m / 256.0) + 0.5).astype(np.int64)


def code_len_q16(f) -> np.ndarray:
    """An integer stand-in for 2^16 (31 - log2 f), the code length of a
    symbol of frequency f in 2^-16 bits: with e the position of f's top bit
    and m the 8 bits below it, 2^16 (31 - e) - LOG2[m].  Exact at powers of
    two; high by less than 2^16 log2(1 + 1/256) (0.0056 bits) elsewhere
    (the bits of f below those 8 are dropped)."""
    f = np.asarray(f, dtype=np.int64)
    if np.any(f < 1) or np.any(f > M):
        raise ValueError("frequency outside [1, M]")
    e = np.floor(np.log2(f.astype(np.float64))).astype(np.int64)
    e = np.where((np.int64(1) << (e + 1)) <= f, e + 1, e)      # exact bit length - 1
    e = np.where((np.int64(1) << e) > f, e - 1, e)
    norm = (f << (31 - e)) & 0x7FFFFFFF                       # the bits below the top one, at 30..0
    m = norm >> 23
    return (31 - e) * 65536 - log2_table_q16()[m]


def calibrate_sigma_rate(kv, mu, kv_dtype: int, mu_dtype: int, sigma_floor: float, prefix,
                         w_narrow_bp: int, w_wide_bp: int, block_tokens: int = 0, base=None,
                         return_costs: bool = False, narrow_dof: int = 0):
    """S-12: the sigma among sigma_j = max(floor, fp32(base * k_j)), k_j =
    1 - j/32, j = 0..24, that gives the held-out data the least integer code
    length sum(code_len_q16(f)) under the format's CDF, f = C(s+1) - C(s);
    the first j on a tie.  base defaults to the RMS calibration (S-7).

    Reading ([blog] § limitations and future directions: better residual
    models; § engineering choice of predictor: sigma calibrated once on
    held-out data): the RMS is the variance estimate the pages name, but one
    outlier in a few hundred inflates it; fitting the scale to the code
    length the coder will actually spend is the plainest better estimate
    that keeps the pages' mixture.  The cost is an integer sum, so the
    choice does not depend on the order of summation."""
    if base is None:
        base = calibrate_sigma(kv, mu, kv_dtype, mu_dtype, sigma_floor, block_tokens)
    base = np.asarray(base, dtype=np.float32)
    kv = np.asarray(kv)
    reps, planes, t_len, ch = kv.shape
    base3 = base[:, None, :] if block_tokens == 0 else base
    blk = t_len if block_tokens == 0 else block_tokens
    t_n, t_w, t_e = budgets(kv_dtype, w_narrow_bp, w_wide_bp)
    pref = prefix if t_e else None
    s = order_index(kv, kv_dtype).astype(np.int64)
    m32 = mu_to_f32(mu, mu_dtype)
    fl = np.float32(sigma_floor)
    tok_block = np.arange(t_len) // blk
    costs = np.zeros((RATE_STEPS,) + base3.shape, dtype=np.int64)
    cands = []
    for j in range(RATE_STEPS):
        k = np.float32(1.0 - j / 32.0)
        sj = np.maximum((base3 * k).astype(np.float32), fl).astype(np.float32)
        cands.append(sj)
        inv = _inv_sigma(sj)[:, tok_block, :]                 # [planes, T, D]
        for r in range(reps):
            c0 = cdf(s[r], m32[r], inv, kv_dtype, t_n, t_w, pref, narrow_dof)
            c1 = cdf(s[r] + 1, m32[r], inv, kv_dtype, t_n, t_w, pref, narrow_dof)
            cl = code_len_q16(c1 - c0)                        # [planes, T, D]
            for b in range(base3.shape[1]):
                costs[j, :, b, :] += cl[:, b * blk:(b + 1) * blk, :].sum(axis=1)
    pick = np.argmin(costs, axis=0)                           # the first minimum
    out = np.take_along_axis(np.stack(cands), pick[None], axis=0)[0]
    out = out[:, 0, :] if block_tokens == 0 else out
    return (out, costs) if return_costs else out


__all__ += ["RATE_STEPS", "log2_table_q16", "code_len_q16", "calibrate_sigma_rate"]


# ---------------------------------------------------------------------------
# S-14  per-channel split of the Gaussian budget (an optional calibration)
# ---------------------------------------------------------------------------
SPLIT_STEPS = 16                   # candidate narrow weights w_n + w_w - SPLIT_STEP_BP * j
SPLIT_STEP_BP = 200


def split_candidates(w_narrow_bp: int, w_wide_bp: int) -> np.ndarray:
    """The narrow weights S-14 chooses from: W - 200 j for j = 0..15, W = w_n +
    w_w, those below 0 raised to 0."""
    w = w_narrow_bp + w_wide_bp
    return np.maximum(w - SPLIT_STEP_BP * np.arange(SPLIT_STEPS, dtype=np.int64), 0)


def calibrate_split(kv, mu, sigma, prefix, kv_dtype: int, mu_dtype: int, w_narrow_bp: int,
                    w_wide_bp: int, sigma_block_tokens: int = 0, narrow_dof: int = 0,
                    return_costs: bool = False):
    """S-14: per (plane, channel), the narrow weight among split_candidates
    that gives the held-out data [reps, planes, tokens, channels] the least
    integer code length sum(code_len_q16(f)) under the format's CDF with that
    channel's budgets (split_budgets); the first candidate on a tie.  sigma is
    the one the stream will use (per channel, or per block with
    sigma_block_tokens).

    Reading ([wiki] § future directions and [blog] § limitations and future
    directions ask for a better residual model; the pages' weights 0.95 /
    0.03 are one choice for every channel, [wiki] § mixture distribution):
    the escape weight stays the call's, so the marginal and its slots are
    shared, and each channel moves weight between its narrow and its wide
    Gaussian, fitted to the code length as S-12 fits sigma."""
    kv = np.asarray(kv)
    reps, planes, t_len, ch = kv.shape
    t_n, t_w, t_e = budgets(kv_dtype, w_narrow_bp, w_wide_bp)
    pref = prefix if t_e else None
    inv = _inv_sigma(sigma_per_token(sigma, t_len, sigma_block_tokens))   # [planes, T, D]
    s = order_index(kv, kv_dtype).astype(np.int64)
    m32 = mu_to_f32(mu, mu_dtype)
    cands = split_candidates(w_narrow_bp, w_wide_bp)
    costs = np.zeros((SPLIT_STEPS, planes, ch), dtype=np.int64)
    for j, wc in enumerate(cands):
        tn, tw = split_budgets(kv_dtype, w_narrow_bp, w_wide_bp, np.full((planes, ch), wc))
        for r in range(reps):
            c0 = cdf(s[r], m32[r], inv, kv_dtype, tn[:, None, :], tw[:, None, :], pref, narrow_dof)
            c1 = cdf(s[r] + 1, m32[r], inv, kv_dtype, tn[:, None, :], tw[:, None, :], pref, narrow_dof)
            costs[j] += code_len_q16(c1 - c0).sum(axis=1)
    out = cands[np.argmin(costs, axis=0)].astype(np.int64)     # the first minimum
    return (out, costs) if return_costs else out


__all__ += ["SPLIT_STEPS", "SPLIT_STEP_BP", "split_budgets", "h_fx_lanes", "split_candidates",
            "calibrate_split"]


# ---------------------------------------------------------------------------
# S-10  side-information checksum
# ---------------------------------------------------------------------------
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)


def _mix64(z: np.ndarray) -> np.ndarray:
    """splitmix64 output function (Vigna's published constants)."""
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _words_hash(words: np.ndarray, tag: int) -> int:
    w = np.ascontiguousarray(words).view(np.uint32).astype(np.uint64).ravel()
    i = np.arange(w.size, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = ((i << np.uint64(32)) | w) + np.uint64(tag) * _GOLDEN
        return int(np.sum(_mix64(z), dtype=np.uint64))


def side_hash(sigma, prefix=None, split=None) -> int:
    """64-bit checksum of the side information both ends must share
    (sum mod 2^64 of mixed (index, word) pairs; sigma words tag 1, followed
    in the same sequence by the per-channel split's words when there is one
    (S-14), prefix words tag 2).  Detects a decoder fed different sigma,
    split or p_hat."""
    words = np.ascontiguousarray(np.asarray(sigma, dtype=np.float32)).view(np.uint32).ravel()
    if split is not None:
        words = np.concatenate([words, np.asarray(split, dtype=np.int64).astype(np.uint32).ravel()])
    h = _words_hash(words, 1)
    if prefix is not None:
        h += _words_hash(np.asarray(prefix, dtype=np.int64).astype(np.uint32), 2)
    return h & ((1 << 64) - 1)


# ---------------------------------------------------------------------------
# S-8 .. S-10  rANS coder, interleaving and stream
# ---------------------------------------------------------------------------
def chunk_layout(planes: int, tokens: int, channels: int, chunk_tokens: int):
    """Chunk c = ((g * n_tok_chunks + tc) * (channels / 64) + k) codes tokens
    [tc*Tc, min((tc+1)*Tc, T)) of channels [64k, 64k+64) of plane g; lane l
    of the chunk is channel 64k + l."""
    n_tc = -(-tokens // chunk_tokens)
    n_k = channels // LANES
    cid = np.arange(planes * n_tc * n_k, dtype=np.int64)
    k = cid % n_k
    tc = (cid // n_k) % n_tc
    g = cid // (n_k * n_tc)
    length = np.minimum(chunk_tokens, tokens - tc * chunk_tokens)
    return g, tc, k, length


_HEADER_FMT = "<4sHHBBBBBBBBIIIIIIQQQQQQI"


HEADER_CRC_OFFSET = 92             # CRC-32 of header bytes [0, 92) at [92, 96)


def crc32(data: bytes) -> int:
    """CRC-32 as used by zlib, gzip and PNG (reflected polynomial
    0xEDB88320, initial value and final xor 0xFFFFFFFF), bit by bit from its
    definition."""
    c = 0xFFFFFFFF
    for byte in data:
        c ^= byte
        for _ in range(8):
            c = (c >> 1) ^ (0xEDB88320 if c & 1 else 0)
    return c ^ 0xFFFFFFFF


def stream_header(kv_dtype, mu_dtype, w_n, w_w, chunk_tokens, planes, tokens, channels,
            n_chunks, payload_bytes, shash, sigma_block_tokens=0, narrow_dof=0, channel_split=0) -> bytes:
    """S-10: the 128-byte header.  Bytes [0, 92) hold the fields, [92, 96)
    the CRC-32 of those 92 bytes (a damaged header is reported as such
    instead of steering the decoder with a wrong shape), the rest zero."""
    t_n, t_w, t_e = budgets(kv_dtype, w_n, w_w)
    h = struct.pack(
        _HEADER_FMT,
        MAGIC, VERSION, HEADER_BYTES, kv_dtype, mu_dtype, LOG2_M, LOG2_L,
        WORD_BITS, LANES, narrow_dof, channel_split, w_n, w_w, t_n, t_w, t_e, chunk_tokens,
        planes, tokens, channels, n_chunks, payload_bytes, shash, sigma_block_tokens)
    assert len(h) == HEADER_CRC_OFFSET
    h += struct.pack("<I", crc32(h))
    return h + bytes(HEADER_BYTES - len(h))


def parse_header(stream: bytes) -> dict:
    if len(stream) < HEADER_BYTES:
        raise StreamError("stream shorter than its header")
    f = struct.unpack_from(_HEADER_FMT, stream, 0)
    keys = ["magic", "version", "header_bytes", "kv_dtype", "mu_dtype", "log2_m",
            "log2_l", "word_bits", "lanes", "narrow_dof", "channel_split", "w_narrow_bp", "w_wide_bp",
            "t_n", "t_w", "t_e", "chunk_tokens", "planes", "tokens", "channels",
            "n_chunks", "payload_bytes", "side_hash", "sigma_block_tokens"]
    h = dict(zip(keys, f))
    if h["magic"] != MAGIC or h["version"] != VERSION or h["header_bytes"] != HEADER_BYTES:
        raise StreamError("bad magic/version")
    if struct.unpack_from("<I", stream, HEADER_CRC_OFFSET)[0] != crc32(stream[:HEADER_CRC_OFFSET]):
        raise StreamError("header checksum")
    if (h["log2_m"], h["log2_l"], h["word_bits"], h["lanes"]) != (LOG2_M, LOG2_L, WORD_BITS, LANES) \
            or h["channel_split"] > 1 or any(stream[HEADER_CRC_OFFSET + 4:HEADER_BYTES]):
        raise StreamError("unsupported coder parameters")
    if h["kv_dtype"] not in (BF16, E4M3) or h["mu_dtype"] not in (BF16, F32):
        raise StreamError("bad dtype")
    if h["narrow_dof"] > NARROW_DOF_MAX:
        raise StreamError("bad narrow part")
    try:
        bud = budgets(h["kv_dtype"], h["w_narrow_bp"], h["w_wide_bp"])
    except ValueError as e:
        raise StreamError(str(e)) from None
    if bud != (h["t_n"], h["t_w"], h["t_e"]):
        raise StreamError("budgets do not match weights")
    if h["chunk_tokens"] < 1 or h["channels"] % LANES or h["channels"] == 0 \
            or h["planes"] == 0 or h["tokens"] == 0:
        raise StreamError("bad shape")
    n_tc = -(-h["tokens"] // h["chunk_tokens"])
    if h["n_chunks"] != h["planes"] * n_tc * (h["channels"] // LANES):
        raise StreamError("chunk count does not match shape")
    try:
        _check_sigma_blocks(h["tokens"], h["chunk_tokens"], h["sigma_block_tokens"])
    except ValueError as e:
        raise StreamError(str(e)) from None
    return h


def _roundup8(x):
    return (x + 7) // 8 * 8


def encode(kv, mu, sigma, prefix, kv_dtype: int, mu_dtype: int, w_narrow_bp: int,
           w_wide_bp: int, chunk_tokens: int, batch_chunks: int = 2048,
           sigma_block_tokens: int = 0, narrow_dof: int = 0, channel_split=None) -> bytes:
    """Code kv [G, T, D] (raw bit patterns) under the mixture around mu [G, T, D]
    with sigma [G, D] (or, with sigma_block_tokens = B > 0, sigma
    [G, ceil(T / B), D]: S-11) and, when ``channel_split`` [G, D] is given,
    each channel's own split of the Gaussian budget (S-14); return the
    KVC-1 byte stream.

    Per chunk and lane, tokens are coded last to first so that the decoder
    runs first to last (rANS is last-in first-out).  Before a symbol with
    frequency f = C(s+1) - C(s) is pushed, the state x is renormalised down
    so that x < 2^32 f by emitting its low 16-bit word (count = [x/2^32 >= f]
    + [x/2^48 >= f] words); then x <- floor(x/f) * M + slot(s, x mod f).
    The symbol's f slots are its Gaussian slots [G(s), G(s+1)) in the range
    [0, T_n + T_w), then its floor-and-escape slots [Q(s), Q(s+1)) shifted
    by T_n + T_w: slot(s, r) = G(s) + r for r < f_G, else
    T_n + T_w + Q(s) + (r - f_G).
    The words of one token step are laid out in the order the decoder reads
    them: first, for every lane that emitted at least one word (ascending
    lane), its last-emitted word; then, for every lane that emitted two,
    its first-emitted word.
    """
    kv = np.asarray(kv)
    g_n, t_len, d_n = kv.shape
    if d_n % LANES or d_n == 0 or g_n == 0 or t_len == 0:
        raise ValueError("channels must be a positive multiple of 64")
    if chunk_tokens < 1:
        raise ValueError("chunk_tokens must be >= 1")
    _check_sigma_blocks(t_len, chunk_tokens, sigma_block_tokens)
    t_n, t_w, t_e = budgets(kv_dtype, w_narrow_bp, w_wide_bp)
    if t_e and prefix is None:
        raise ValueError("mixture with an escape part needs the marginal prefix")
    if not 0 <= narrow_dof <= NARROW_DOF_MAX:
        raise ValueError("narrow_dof must be 0 or 1..16")
    pref = prefix if t_e else None
    if channel_split is not None:
        channel_split = np.asarray(channel_split, dtype=np.int64)
        if channel_split.shape != (g_n, d_n):
            raise ValueError("the channel split is [planes, channels]")
        tn_all, tw_all = split_budgets(kv_dtype, w_narrow_bp, w_wide_bp, channel_split)
    else:
        tn_all = np.full((g_n, d_n), t_n, dtype=np.int64)
        tw_all = np.full((g_n, d_n), t_w, dtype=np.int64)
    mu32_all = mu_to_f32(mu, mu_dtype)
    sig3, blk = sigma_blocks(sigma, t_len, sigma_block_tokens)
    inv_all = _inv_sigma(sig3)
    sym_all = order_index(kv, kv_dtype)

    g_of, tc_of, k_of, len_of = chunk_layout(g_n, t_len, d_n, chunk_tokens)
    n_chunks = g_of.size
    lane = np.arange(LANES, dtype=np.int64)
    payloads = []
    for b0 in range(0, n_chunks, batch_chunks):
        sl = slice(b0, min(n_chunks, b0 + batch_chunks))
        g, tcid, k, ln = g_of[sl], tc_of[sl], k_of[sl], len_of[sl]
        nb = g.size
        d = 64 * k[:, None] + lane[None, :]
        inv = inv_all[g[:, None], (tcid * chunk_tokens // blk)[:, None], d]
        if channel_split is not None:
            ln_b, lw_b = tn_all[g[:, None], d], tw_all[g[:, None], d]
        else:
            ln_b, lw_b = t_n, t_w
        x = np.full((nb, LANES), L, dtype=np.uint64)
        words = np.zeros((nb, chunk_tokens, 2, LANES), dtype=np.uint16)
        emit = np.zeros((nb, chunk_tokens, 2, LANES), dtype=bool)
        for t in range(chunk_tokens - 1, -1, -1):
            active = (t < ln)[:, None]
            tok = np.minimum(tcid * chunk_tokens + t, t_len - 1)[:, None]
            s = sym_all[g[:, None], tok, d]
            mu32 = mu32_all[g[:, None], tok, d]
            g0 = gauss_cum(s, mu32, inv, kv_dtype, ln_b, lw_b, narrow_dof)
            fg = gauss_cum(s + 1, mu32, inv, kv_dtype, ln_b, lw_b, narrow_dof) - g0
            q0 = escape_cum(s, pref)
            f = fg + escape_cum(s + 1, pref) - q0
            fu = f.astype(np.uint64)
            count = ((x >> np.uint64(32)) >= fu).astype(np.int64) + \
                    ((x >> np.uint64(48)) >= fu).astype(np.int64)
            count = np.where(active, count, 0)
            first = (x & np.uint64(0xFFFF)).astype(np.uint16)
            second = ((x >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.uint16)
            words[:, t, 0, :] = np.where(count == 2, second, first)
            words[:, t, 1, :] = first
            emit[:, t, 0, :] = count >= 1
            emit[:, t, 1, :] = count == 2
            xs = x >> (np.uint64(16) * count.astype(np.uint64))
            r = (xs % fu).astype(np.int64)
            slot = np.where(r < fg, g0 + r, (t_n + t_w) + q0 + (r - fg))
            xn = ((xs // fu) << np.uint64(LOG2_M)) + slot.astype(np.uint64)
            x = np.where(active, xn, x)
        for i in range(nb):
            body = x[i].astype("<u8").tobytes() + words[i][emit[i]].astype("<u2").tobytes()
            payloads.append(body + bytes(_roundup8(len(body)) - len(body)))

    sizes = np.array([len(p) for p in payloads], dtype=np.int64)
    directory = np.concatenate([[0], np.cumsum(sizes)]).astype("<u8")
    shash = side_hash(sigma, prefix if t_e else None, channel_split)
    head = stream_header(kv_dtype, mu_dtype, w_narrow_bp, w_wide_bp, chunk_tokens,
                         g_n, t_len, d_n, n_chunks, int(directory[-1]), shash, sigma_block_tokens, narrow_dof,
                         0 if channel_split is None else 1)
    return head + directory.tobytes() + b"".join(payloads)


def decode(stream: bytes, mu, sigma, prefix, batch_chunks: int = 2048,
           chunk_ids=None, channel_split=None):
    """Rebuild the raw KV bit patterns [G, T, D] from a KVC-1 stream.

    Per token step and lane: target = x mod M.  A target below T_n + T_w is
    a Gaussian slot: the symbol is the unique s with G(s) <= target <
    G(s+1) and its rank r = target - G(s); otherwise y = target - T_n - T_w
    is a floor-and-escape slot: s is the unique symbol with Q(s) <= y <
    Q(s+1) and r = f_G(s) + y - Q(s) (both found here by plain bisection
    over the alphabet).  Then x <- f * floor(x / M) + r; then, while x < L, a
    16-bit word is shifted in (round 1 for every lane that needs one, in lane
    order, then round 2).  Every lane must end in state L and every chunk
    must consume exactly its payload, else the stream is corrupt.

    With ``chunk_ids`` only those chunks are decoded; the result is then a
    dict {chunk id: [length, 64] bit patterns}.  A stream coded with a
    per-channel split (S-14) needs the same split.
    """
    h = parse_header(stream)
    kv_dtype, mu_dtype = h["kv_dtype"], h["mu_dtype"]
    g_n, t_len, d_n, tcn = h["planes"], h["tokens"], h["channels"], h["chunk_tokens"]
    n_chunks = h["n_chunks"]
    t_n, t_w, t_e = h["t_n"], h["t_w"], h["t_e"]
    dof = h["narrow_dof"]
    pref = prefix if t_e else None
    if t_e and prefix is None:
        raise ValueError("stream uses an escape part; the marginal prefix is needed")
    split = None
    if h["channel_split"]:
        if channel_split is None:
            raise ValueError("stream uses a per-channel split; the split is needed")
        split = np.asarray(channel_split, dtype=np.int64)
        if split.shape != (g_n, d_n):
            raise ValueError("the channel split is [planes, channels]")
        tn_all, tw_all = split_budgets(kv_dtype, h["w_narrow_bp"], h["w_wide_bp"], split)
    if side_hash(sigma, pref, split) != h["side_hash"]:
        raise StreamError("side information does not match the stream")
    dir_off = HEADER_BYTES
    pay_off = dir_off + 8 * (n_chunks + 1)
    if len(stream) < pay_off:
        raise StreamError("stream shorter than its directory")
    directory = np.frombuffer(stream, dtype="<u8", count=n_chunks + 1, offset=dir_off).astype(np.int64)
    if directory[0] != 0 or np.any(np.diff(directory) < STATE_BYTES) \
            or directory[-1] != h["payload_bytes"] or pay_off + directory[-1] != len(stream):
        raise StreamError("bad chunk directory")
    if np.any(directory % 8):
        raise StreamError("misaligned chunk")

    mu32_all = mu_to_f32(mu, mu_dtype)
    try:
        sig3, blk = sigma_blocks(sigma, t_len, h["sigma_block_tokens"])
    except ValueError as e:
        raise StreamError(str(e)) from None
    inv_all = _inv_sigma(sig3)
    g_of, tc_of, k_of, len_of = chunk_layout(g_n, t_len, d_n, tcn)
    n_sym = alphabet_size(kv_dtype)
    steps = n_sym.bit_length() - 1
    lane = np.arange(LANES, dtype=np.int64)
    ids = np.arange(n_chunks) if chunk_ids is None else np.asarray(chunk_ids, dtype=np.int64)
    out_full = None
    out_dict = {}
    if chunk_ids is None:
        out_full = np.zeros((g_n, t_len, d_n), dtype=np.uint16 if kv_dtype == BF16 else np.uint8)

    for b0 in range(0, ids.size, batch_chunks):
        cid = ids[b0:b0 + batch_chunks]
        g, tcid, k, ln = g_of[cid], tc_of[cid], k_of[cid], len_of[cid]
        nb = cid.size
        d = 64 * k[:, None] + lane[None, :]
        inv = inv_all[g[:, None], (tcid * tcn // blk)[:, None], d]
        ln_b, lw_b = (tn_all[g[:, None], d], tw_all[g[:, None], d]) if split is not None else (t_n, t_w)
        start_b = pay_off + directory[cid]
        size_b = directory[cid + 1] - directory[cid]
        x = np.stack([np.frombuffer(stream, dtype="<u8", count=LANES, offset=int(o)) for o in start_b]).astype(np.uint64)
        # an encoder's final state lies in the state interval [L, 2^16 L)
        if np.any((x < np.uint64(L)) | (x >= np.uint64(L << 16))):
            raise StreamError("initial rANS state outside [L, 2^16 L)")
        nwords = (size_b - STATE_BYTES) // 2
        wmax = int(nwords.max()) if nb else 0
        words = np.zeros((nb, wmax + 1), dtype=np.uint64)
        for i in range(nb):
            w = np.frombuffer(stream, dtype="<u2", count=int(nwords[i]), offset=int(start_b[i] + STATE_BYTES))
            words[i, :w.size] = w
        ptr = np.zeros(nb, dtype=np.int64)
        sym = np.zeros((nb, tcn, LANES), dtype=np.int64)
        for t in range(tcn):
            active = (t < ln)[:, None]
            tok = np.minimum(tcid * tcn + t, t_len - 1)[:, None]
            mu32 = mu32_all[g[:, None], tok, d]
            target = (x & np.uint64(M - 1)).astype(np.int64)
            htot = t_n + t_w
            in_g = target < htot
            y = target - htot
            # bisection: largest b with G(b) <= target, and with Q(b) <= y
            lo_g = np.zeros((nb, LANES), dtype=np.int64)
            hi_g = np.full((nb, LANES), n_sym, dtype=np.int64)
            lo_q = np.zeros((nb, LANES), dtype=np.int64)
            hi_q = np.full((nb, LANES), n_sym, dtype=np.int64)
            for _ in range(steps):
                mid = (lo_g + hi_g) >> 1
                go = gauss_cum(mid, mu32, inv, kv_dtype, ln_b, lw_b, dof) <= target
                lo_g, hi_g = np.where(go, mid, lo_g), np.where(go, hi_g, mid)
                mid = (lo_q + hi_q) >> 1
                go = escape_cum(mid, pref) <= y
                lo_q, hi_q = np.where(go, mid, lo_q), np.where(go, hi_q, mid)
            lo = np.where(in_g, lo_g, lo_q)
            g0 = gauss_cum(lo, mu32, inv, kv_dtype, ln_b, lw_b, dof)
            fg = gauss_cum(lo + 1, mu32, inv, kv_dtype, ln_b, lw_b, dof) - g0
            q0 = escape_cum(lo, pref)
            f = (fg + escape_cum(lo + 1, pref) - q0).astype(np.uint64)
            r = np.where(in_g, target - g0, fg + (y - q0)).astype(np.uint64)
            xn = f * (x >> np.uint64(LOG2_M)) + r
            x = np.where(active, xn, x)
            for _round in range(2):
                need = active & (x < np.uint64(L))
                rank = np.cumsum(need, axis=1) - need
                idx = ptr[:, None] + rank
                if np.any(need & (idx >= nwords[:, None])):
                    raise StreamError("chunk payload exhausted")
                w = np.take_along_axis(words, np.minimum(idx, wmax), axis=1)
                x = np.where(need, (x << np.uint64(16)) | w, x)
                ptr = ptr + need.sum(axis=1)
            sym[:, t, :] = lo
        if np.any(x != np.uint64(L)):
            raise StreamError("final rANS state is not the initial state")
        if np.any(_roundup8(STATE_BYTES + 2 * ptr) != size_b):
            raise StreamError("chunk payload not consumed exactly")
        for i in range(nb):
            pad_lo = int(start_b[i] + STATE_BYTES + 2 * ptr[i])
            if any(stream[pad_lo:int(start_b[i] + size_b[i])]):
                raise StreamError("nonzero padding")
        bits = bits_of_order(sym, kv_dtype)
        for i in range(nb):
            n_t = int(ln[i])
            rows = bits[i, :n_t, :]
            if out_full is not None:
                t0 = int(tcid[i]) * tcn
                out_full[g[i], t0:t0 + n_t, 64 * k[i]:64 * k[i] + 64] = rows
            else:
                out_dict[int(cid[i])] = rows.astype(out_dict_dtype(kv_dtype))
    return out_full if out_full is not None else out_dict


def out_dict_dtype(kv_dtype):
    return np.uint16 if kv_dtype == BF16 else np.uint8


def chunk_payload(stream: bytes, chunk_id: int) -> bytes:
    """Bytes of one chunk's payload (states, words, padding)."""
    h = parse_header(stream)
    pay_off = HEADER_BYTES + 8 * (h["n_chunks"] + 1)
    a, b = np.frombuffer(stream, dtype="<u8", count=2, offset=HEADER_BYTES + 8 * chunk_id)
    return stream[pay_off + int(a):pay_off + int(b)]


def encode_chunks(kv, mu, sigma, prefix, kv_dtype, mu_dtype, w_narrow_bp, w_wide_bp,
                  chunk_tokens, chunk_ids, sigma_block_tokens=0, narrow_dof=0, channel_split=None):
    """Payloads of selected chunks only (for sampled parity at full size).

    Each chunk depends only on its own slice of kv and mu, on the sigma its
    tokens use and on its channels' split (S-14), so it is coded by running
    :func:`encode` on a one-plane view."""
    kv = np.asarray(kv)
    g_n, t_len, d_n = kv.shape
    sig3, blk = sigma_blocks(sigma, t_len, sigma_block_tokens)
    g_of, tc_of, k_of, len_of = chunk_layout(g_n, t_len, d_n, chunk_tokens)
    out = {}
    for cid in chunk_ids:
        g, tc, k, ln = int(g_of[cid]), int(tc_of[cid]), int(k_of[cid]), int(len_of[cid])
        t0 = tc * chunk_tokens
        sub_kv = kv[g:g + 1, t0:t0 + ln, 64 * k:64 * k + 64]
        sub_mu = np.asarray(mu)[g:g + 1, t0:t0 + ln, 64 * k:64 * k + 64]
        sub_sig = sig3[g:g + 1, t0 // blk, 64 * k:64 * k + 64]
        sub_split = None if channel_split is None else \
            np.asarray(channel_split)[g:g + 1, 64 * k:64 * k + 64]
        s = encode(sub_kv, sub_mu, sub_sig, prefix, kv_dtype, mu_dtype, w_narrow_bp,
                   w_wide_bp, chunk_tokens, narrow_dof=narrow_dof, channel_split=sub_split)
        out[int(cid)] = chunk_payload(s, 0)
    return out


def wrap_chunk(payload: bytes, sigma_sub, prefix, kv_dtype, mu_dtype, w_narrow_bp, w_wide_bp,
               chunk_tokens, tokens, narrow_dof=0) -> bytes:
    """A one-chunk stream around one chunk's payload (64 channels, `tokens`
    tokens of one plane, its 64 sigmas), so that :func:`decode` can check a
    chunk cut out of a large stream on its own."""
    t_e = budgets(kv_dtype, w_narrow_bp, w_wide_bp)[2]
    shash = side_hash(np.asarray(sigma_sub, dtype=np.float32).reshape(1, LANES), prefix if t_e else None)
    head = stream_header(kv_dtype, mu_dtype, w_narrow_bp, w_wide_bp, chunk_tokens, 1, tokens, LANES, 1,
                         len(payload), shash, 0, narrow_dof)
    directory = np.array([0, len(payload)], dtype="<u8")
    return head + directory.tobytes() + payload


__all__ += ["chunk_payload", "encode_chunks", "wrap_chunk"]


# ---------------------------------------------------------------------------
# Paged output: decoded rows placed in a paged KV cache
# ---------------------------------------------------------------------------
def scatter_to_pages(kv, batch: int, heads: int, block_table, page_tokens: int, num_pages: int,
                     fill: int = 0) -> np.ndarray:
    """The decoder's output placed in page pools, as a serving engine keeps
    its cache ([blog] § application scenarios and deployment parameters:
    a compressed cache entry is decompressed where it is consumed).

    kv is [G, T, D] with planes ordered (layer, kv, batch, head); the result
    is [layers * 2, num_pages, page_tokens, heads, D], pool 2 * layer + kv,
    with kv[g, t] at page block_table[b, t // page_tokens], row
    t % page_tokens, head h; entries no token maps to keep `fill`."""
    kv = np.asarray(kv)
    g_n, t_len, d_n = kv.shape
    per_layer = 2 * batch * heads
    if g_n % per_layer:
        raise ValueError("planes must be layers * 2 * batch * heads")
    table = np.asarray(block_table, dtype=np.int64)
    pools = np.full((g_n // per_layer * 2, num_pages, page_tokens, heads, d_n), fill, dtype=kv.dtype)
    g = np.arange(g_n)
    pool_of, b_of, h_of = g // (batch * heads), (g // heads) % batch, g % heads
    t = np.arange(t_len)
    page = table[b_of[:, None], t[None, :] // page_tokens]          # [G, T]
    if np.any((page < 0) | (page >= num_pages)):
        raise ValueError("block table entry outside the pool")
    pools[pool_of[:, None], page, (t % page_tokens)[None, :], h_of[:, None]] = kv
    return pools


__all__ += ["scatter_to_pages"]


# ---------------------------------------------------------------------------
# bits per scalar: the integer model and the continuous mixture
# ---------------------------------------------------------------------------
def sigma_per_token(sigma, tokens: int, sigma_block_tokens: int = 0) -> np.ndarray:
    """sigma of every (plane, token, channel): [G, T, D] (S-11)."""
    sig3, blk = sigma_blocks(sigma, tokens, sigma_block_tokens)
    return np.repeat(sig3, blk, axis=1)[:, :tokens, :]


def model_bits_int(kv, mu, sigma, prefix, kv_dtype, mu_dtype, w_narrow_bp, w_wide_bp,
                   sigma_block_tokens: int = 0, narrow_dof: int = 0, channel_split=None) -> float:
    """Mean of -log2(f(s) / M) over all scalars: the ideal code length of the
    integer model ([wiki] § core idea: bits = cross-entropy of q)."""
    kv = np.asarray(kv)
    g_n, t_len, d_n = kv.shape
    t_n, t_w, t_e = budgets(kv_dtype, w_narrow_bp, w_wide_bp)
    pref = prefix if t_e else None
    inv = _inv_sigma(sigma_per_token(sigma, t_len, sigma_block_tokens))
    mu32 = mu_to_f32(mu, mu_dtype)
    s = order_index(kv, kv_dtype)
    total = 0.0
    if channel_split is not None:
        tn_all, tw_all = split_budgets(kv_dtype, w_narrow_bp, w_wide_bp, channel_split)
    for g in range(g_n):
        ln_g, lw_g = (tn_all[g][None, :], tw_all[g][None, :]) if channel_split is not None else (t_n, t_w)
        c0 = cdf(s[g], mu32[g], inv[g], kv_dtype, ln_g, lw_g, pref, narrow_dof)
        c1 = cdf(s[g] + 1, mu32[g], inv[g], kv_dtype, ln_g, lw_g, pref, narrow_dof)
        total += float(np.sum(LOG2_M - np.log2((c1 - c0).astype(np.float64))))
    return total / kv.size


def _ndtr_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Phi(b) - Phi(a) for a <= b, using the upper-tail form when both are
    positive so that the difference does not cancel."""
    from scipy.special import ndtr
    upper = a > 0
    return np.where(upper, ndtr(-a) - ndtr(-b), ndtr(b) - ndtr(a))


def _stdtr_mass(a: np.ndarray, b: np.ndarray, nu: int) -> np.ndarray:
    """F(b) - F(a) for Student's t with nu degrees of freedom truncated to
    [-24, 24] and renormalised (S-13), a <= b; the upper-tail form when both
    are positive.  scipy's stdtr is the CDF."""
    from scipy.special import stdtr
    lim = float(TABLE_Z_MAX)
    a = np.clip(a, -lim, lim)
    b = np.clip(b, -lim, lim)
    span = 1.0 - 2.0 * stdtr(nu, -lim)
    upper = a > 0
    m = np.where(upper, stdtr(nu, -a) - stdtr(nu, -b), stdtr(nu, b) - stdtr(nu, a))
    return m / span


def model_bits_float(kv, mu, sigma, prefix, kv_dtype, mu_dtype, w_narrow_bp, w_wide_bp,
                     cap_bits: float = 64.0, sigma_block_tokens: int = 0, narrow_dof: int = 0,
                     channel_split=None) -> float:
    """Mean -log2 q(x) of the continuous mixture over the same cells, float64.

    q(x) = w_n [Phi((hi-mu)/sigma) - Phi((lo-mu)/sigma)]
         + w_w [same with 3 sigma] + w_e p_hat(x),
    (with narrow_dof = nu, the narrow part's Phi is the truncated Student-t
    of S-13; with a per-channel split, w_n and w_w are the channel's w_c and
    w_n + w_w - w_c, S-14),
    with p_hat(x) = (prefix[x+1] - prefix[x]) / T_e and the weights in basis
    points ([wiki] § mixture distribution).  A per-scalar cost is capped at
    ``cap_bits`` (only reachable without an escape part)."""
    kv = np.asarray(kv)
    t_n, t_w, t_e = budgets(kv_dtype, w_narrow_bp, w_wide_bp)
    wn, ww = w_narrow_bp / 1e4, w_wide_bp / 1e4
    we = 1.0 - wn - ww
    if channel_split is not None:
        wn = np.asarray(channel_split, dtype=np.float64)[:, None, :] / 1e4 * np.ones((1, kv.shape[1], 1))
        ww = (w_narrow_bp + w_wide_bp) / 1e4 - wn
    pos = boundary_positions(kv_dtype).astype(np.float64)
    sig = sigma_per_token(sigma, kv.shape[1], sigma_block_tokens).astype(np.float64)
    mu_all = mu_to_f32(mu, mu_dtype).astype(np.float64)
    s = order_index(kv, kv_dtype)
    total = 0.0
    for g in range(kv.shape[0]):
        lo = pos[s[g]]
        hi = pos[s[g] + 1]
        m = mu_all[g]
        sg = sig[g]
        with np.errstate(invalid="ignore"):
            a1, b1 = (lo - m) / sg, (hi - m) / sg
            a3, b3 = (lo - m) / (3 * sg), (hi - m) / (3 * sg)
        narrow = _ndtr_diff(a1, b1) if narrow_dof == 0 else _stdtr_mass(a1, b1, narrow_dof)
        wn_g = wn[g] if np.ndim(wn) else wn
        ww_g = ww[g] if np.ndim(ww) else ww
        q = wn_g * narrow + ww_g * _ndtr_diff(a3, b3)
        if t_e:
            p = np.asarray(prefix, dtype=np.float64)
            q = q + we * (p[s[g] + 1] - p[s[g]]) / t_e
        with np.errstate(divide="ignore"):
            bits = np.minimum(-np.log2(q), cap_bits)
        total += float(np.sum(bits))
    return total / kv.size
