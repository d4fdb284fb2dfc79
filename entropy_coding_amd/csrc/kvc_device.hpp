// Device-side building blocks of the KVC-1 coder for gfx950: the ordered
// alphabet, cell edges, the integer mixture CDF and the rANS arithmetic.
// Every floating-point step of the CDF is a single IEEE float32 operation
// with round to nearest (no contraction, denormals kept), so the CDF is
// bit-identical to the host-side specification; everything after the
// argument is integer.
//
// Model: q = 0.95 N(mu, sigma^2) + 0.03 N(mu, (3 sigma)^2) + 0.02 p_hat
// (wiki "Speculative KV Coding", section "mixture distribution"); encoder
// and decoder must evaluate its CDF identically (blog post on speculative
// KV coding, section "application scenarios and deployment parameters").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kBF16 = 0;
constexpr int kE4M3 = 1;
constexpr int kF32 = 2;

constexpr uint32_t kLog2M = 31;
constexpr uint32_t kM = 1u << kLog2M;         // total of every CDF
constexpr uint64_t kL = 1ull << 47;           // lower end of the rANS state interval
constexpr uint32_t kLHi = 1u << 15;           // kL >> 32
constexpr int kLanes = 64;                    // rANS lanes per chunk = one wavefront
constexpr int kStateBytes = 8 * kLanes;       // final states at the head of a chunk
constexpr int kHeaderBytes = 128;

// Mixture table: z grid -24 .. 24 at step 1/256, plus one repeated entry.
constexpr int kTableZMax = 24;
constexpr int kTablePoints = 2 * kTableZMax * 256 + 1;      // 12289
constexpr int kTableEntries = kTablePoints + 1;             // 12290
constexpr int32_t kQMax = kTableZMax << 24;                 // |q| <= 24 * 2^24
constexpr float kQMaxF = static_cast<float>(kQMax);

template <int KV> struct Alphabet;
template <> struct Alphabet<kBF16> {
    static constexpr uint32_t kSize = 65536;
    static constexpr int kLog2 = 16;
    static constexpr uint32_t kLoFinite = 128;      // index of -max
    static constexpr uint32_t kHiFinite = 65407;    // index of +max
    using Bits = uint16_t;
};
template <> struct Alphabet<kE4M3> {
    static constexpr uint32_t kSize = 256;
    static constexpr int kLog2 = 8;
    static constexpr uint32_t kLoFinite = 1;
    static constexpr uint32_t kHiFinite = 254;
    using Bits = uint8_t;
};

// Ordered symbol index of a bit pattern: positives keep their order above
// the midpoint, negatives are mirrored below it.
template <int KV>
__device__ __forceinline__ uint32_t order_of_bits(uint32_t u) {
    constexpr uint32_t half = Alphabet<KV>::kSize >> 1;
    constexpr uint32_t mask = Alphabet<KV>::kSize - 1;
    return (u & half) ? (~u & mask) : (u ^ half);
}

template <int KV>
__device__ __forceinline__ uint32_t bits_of_order(uint32_t b) {
    constexpr uint32_t half = Alphabet<KV>::kSize >> 1;
    constexpr uint32_t mask = Alphabet<KV>::kSize - 1;
    return (b & half) ? (b ^ half) : (~b & mask);
}

// Edge between ordered bf16 symbols b-1 and b.  For neighbours with
// magnitude patterns m and m+1 the midpoint is the fp32 whose pattern is
// m << 16 plus half a bf16 step (0x8000), also across a binade change.
__device__ __forceinline__ float edge_bf16(uint32_t b) {
    const uint32_t m = (b > 32768u) ? (b - 32769u) : (32767u - b);
    const float v = __uint_as_float((m << 16) | 0x8000u);
    float e = (b > 32768u) ? v : -v;
    e = (b == 32768u) ? 0.0f : e;
    e = (b <= 128u) ? -__builtin_huge_valf() : e;     // at or below -max's lower edge
    e = (b >= 65408u) ? __builtin_huge_valf() : e;    // at or above +max's upper edge
    return e;
}

// Magnitude of the e4m3fn pattern m (0..126): bias 7, 3 mantissa bits.
__device__ __forceinline__ float e4m3_magnitude(uint32_t m) {
    const uint32_t e = m >> 3, man = m & 7u;
    return e == 0 ? static_cast<float>(man) * 0x1p-9f
                  : __uint_as_float(((e + 120u) << 23) | (man << 20));
}

__device__ __forceinline__ float edge_e4m3(uint32_t b) {
    const uint32_t m = (b > 128u) ? (b - 128u) : (128u - b);
    const uint32_t mm = (m >= 1u && m <= 126u) ? m : 1u;   // keep the helper in range
    const float v = (e4m3_magnitude(mm - 1u) + e4m3_magnitude(mm)) * 0.5f;
    float e = (b > 128u) ? v : -v;
    e = (b == 128u) ? 0.0f : e;
    e = (b <= 1u) ? -__builtin_huge_valf() : e;
    e = (b >= 255u) ? __builtin_huge_valf() : e;
    return e;
}

template <int KV>
__device__ __forceinline__ float edge(uint32_t b) {
    if constexpr (KV == kBF16) return edge_bf16(b);
    else return edge_e4m3(b);
}

// Predictor mean as float32; a non-finite mean is replaced by 0.
template <int MU> struct MuT;
template <> struct MuT<kBF16> { using T = uint16_t; };
template <> struct MuT<kF32> { using T = float; };

template <int MU>
__device__ __forceinline__ float mu_value(typename MuT<MU>::T v) {
    float m;
    if constexpr (MU == kBF16) m = __uint_as_float(static_cast<uint32_t>(v) << 16);
    else m = v;
    return __builtin_isfinite(m) ? m : 0.0f;
}

// q = floor(clamp(d * inv, +-24) * 2^24) computed as floor(clamp(d * inv24,
// +-24 * 2^24)) with inv24 = inv * 2^24: identical for every sigma in the
// accepted range [2^-96, 2^96] (the power-of-two scaling is exact there and
// both forms saturate together).  Floor and conversion are one instruction
// (v_cvt_flr_i32_f32).
__device__ __forceinline__ int32_t z_fixed(float edge_pos, float mu, float inv24) {
    const float d = __fsub_rn(edge_pos, mu);
    float zq = __fmul_rn(d, inv24);
    zq = __builtin_amdgcn_fmed3f(zq, -kQMaxF, kQMaxF);
    int32_t q;
    __asm__("v_cvt_flr_i32_f32 %0, %1" : "=v"(q) : "v"(zq));
    return q;
}

// floor(dlt r / 2^16) for the 16 low bits r of u: the high word of
// dlt (r 2^16), and r 2^16 is u shifted left by 16 (one shift and one
// multiply, exact for any dlt < 2^32).
__device__ __forceinline__ uint32_t interp_step(uint32_t dlt, uint32_t u) {
    return __umulhi(dlt, u << 16);
}

// Integer mixture CDF of z = q / 2^24: table step 1/256 with integer linear
// interpolation over the 16 low bits of q.
__device__ __forceinline__ uint32_t h_fx(int32_t q, const uint32_t* __restrict__ tab) {
    const uint32_t u = static_cast<uint32_t>(q + kQMax);
    const uint32_t i = u >> 16;
    const uint32_t a = tab[i], c = tab[i + 1];
    return a + interp_step(c - a, u);
}

// Raw buffer resource over `bytes` bytes at p (gfx9 layout: no stride,
// dword 3 = 0x00020000).  An access through it takes a per-lane byte offset
// in a vector register and a wave-uniform one in a scalar register, so the
// address costs no vector arithmetic; reads beyond the range return 0 and
// writes beyond it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

struct Model {
    const uint32_t* __restrict__ tab;      // mixture table in LDS
    const uint32_t* __restrict__ prefix;   // escape prefix (N + 1 entries; zeros without an escape part)
    const uint32_t* small;                 // e4m3 only: prefix and edges in LDS
    const uint32_t* __restrict__ eslots;   // bf16 encoder only: the escape slot table (k_prologue)
    uint32_t htot;                         // T_n + T_w, where the floor-and-escape range starts
    const uint32_t* __restrict__ ecount;   // bf16 decoder only: the escape count table (k_prologue)

    // The narrow and wide parts of the CDF at q (both Gaussian parts, 0 .. htot).
    __device__ __forceinline__ uint32_t h(int32_t q) const { return h_fx(q, tab); }

    // The model of lane L, for a search the whole wave makes for one lane
    // (the same on every lane here).
    __device__ __forceinline__ Model of_lane(int) const { return *this; }
};

// (a b) >> 31 for a < 2^31 and b <= 2^31 (the product is below 2^62).
__device__ __forceinline__ uint32_t mul_shr31(uint32_t a, uint32_t b) {
    return static_cast<uint32_t>((static_cast<uint64_t>(a) * b) >> 31);
}

// A lane's own split of the Gaussian budget: T_n(c) = min(floor(T w_c /
// 10^4), T_n + T_w) for the narrow weight w_c in basis points (T = M - N);
// the wide part gets the rest of T_n + T_w.
__device__ __forceinline__ uint32_t split_narrow_budget(uint32_t w, uint32_t t_all, uint32_t htot) {
    const uint64_t v = static_cast<uint64_t>(t_all) * w / 10000u;
    return v < htot ? static_cast<uint32_t>(v) : htot;
}

// h_fx with the lane's own budgets: the pair table holds (A[k], B[k]), the
// narrow and wide base tables (the last entry repeated), and the lane's
// mixture table entry floor(tn A[k] / 2^31) + floor(tw B[k] / 2^31) is
// formed at the two entries the interpolation reads.
__device__ __forceinline__ uint32_t h_fx_split(int32_t q, const uint2* __restrict__ ab, uint32_t tn, uint32_t tw,
                                               uint32_t& step) {
    const uint32_t u = static_cast<uint32_t>(q + kQMax);
    const uint32_t i = u >> 16;
    const uint2 p0 = ab[i], p1 = ab[i + 1];
    const uint32_t a = mul_shr31(tn, p0.x) + mul_shr31(tw, p0.y);
    const uint32_t c = mul_shr31(tn, p1.x) + mul_shr31(tw, p1.y);
    step = c - a;
    return a + interp_step(c - a, u);
}

// The model of a chunk whose lanes each split the Gaussian budget their own
// way: tab points at the pair table in LDS, tn / tw are the lane's budgets
// (tn + tw = htot on every lane, so the floor-and-escape range and its
// tables are shared).
struct SplitModel : Model {
    uint32_t tn, tw;

    __device__ __forceinline__ uint32_t h(int32_t q) const {
        uint32_t step;
        return h_fx_split(q, reinterpret_cast<const uint2*>(tab), tn, tw, step);
    }

    // The model of lane L on every lane: its budgets.
    __device__ __forceinline__ SplitModel of_lane(int L) const {
        SplitModel r = *this;
        r.tn = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tn), L));
        r.tw = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tw), L));
        return r;
    }

    // The decoder's aim for target t from a z that inverts the call's own
    // mixture table: two Newton steps on the logarithm of this lane's
    // table, counted from the nearer end of the range (t, or T_n + T_w - t
    // in the upper half), whose slope over a grid step (1/256 in z) is the
    // interpolation step.  The tails, where the lane's wide weight decides
    // and the call's aim is furthest off, are close to exponential in z,
    // and the logarithm makes them close to linear.  Only the cost of the
    // search depends on it.
    __device__ __forceinline__ float aim(float z, uint32_t t) const {
        const uint32_t ht = tn + tw;
        const bool upper = ht - t < t;
        const float ldt = __builtin_amdgcn_logf(fmaxf(static_cast<float>(upper ? ht - t : t), 1.0f));
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            float zq = __fmul_rn(z, 16777216.0f);
            zq = __builtin_amdgcn_fmed3f(zq, -kQMaxF, kQMaxF);
            int32_t q;
            __asm__("v_cvt_flr_i32_f32 %0, %1" : "=v"(q) : "v"(zq));
            uint32_t step;
            const uint32_t hq = h_fx_split(q, reinterpret_cast<const uint2*>(tab), tn, tw, step);
            const float dh = fmaxf(static_cast<float>(upper ? ht - hq : hq), 1.0f);
            // d ln D / dz = +-256 step / D (ln 2 turns log2 into ln)
            float dz = (ldt - __builtin_amdgcn_logf(dh)) * 0.69314718f * dh *
                       __builtin_amdgcn_rcpf(static_cast<float>(step) * 256.0f);
            dz = upper ? -dz : dz;
            z = step ? z + dz : z;
            z = __builtin_amdgcn_fmed3f(z, -static_cast<float>(kTableZMax), static_cast<float>(kTableZMax));
        }
        return z;
    }
};

// Two consecutive u32 at byte offset `off` of `base` in one 8-byte read
// (4-byte aligned), addressed as a scalar base plus a 32-bit lane offset.
struct alignas(4) U32Pair {
    uint32_t a, b;
};
__device__ __forceinline__ U32Pair load_pair(const uint32_t* base, uint32_t off) {
    return *reinterpret_cast<const U32Pair*>(reinterpret_cast<const char*>(base) + off);
}

// C(b) = b + h(q(b)) + prefix[b].
template <int KV, class M>
__device__ __forceinline__ uint32_t cdf_at(uint32_t b, float mu, float inv24, const M& m) {
    uint32_t g = b + m.h(z_fixed(edge<KV>(b), mu, inv24));
    g += m.prefix[b];
    return g;
}

// Rank of this lane among the set bits of `mask` below it.
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Accepted sigma: finite, within [2^-96, 2^96].
__device__ __forceinline__ bool sigma_ok(float s) {
    return s >= 0x1p-96f && s <= 0x1p96f;
}

// floor(x / f) and x mod f for x = xh * 2^32 + xl < 2^32 f (the quotient
// fits 32 bits), without a hardware divider: a float64 quotient from the
// hardware reciprocal refined by one Newton step is within 2^-16 of x / f;
// truncating it plus one half gives the quotient or one above it, which one
// borrow test settles.  The conversions are written as the instructions
// (the compiler's own form of the first one adds a float64 zero, and the
// last one saturates at 2^32 - 1 by itself, which an estimate of 2^32 needs).
// x - q0 f then lies in [-f, f), so below 2^31 in magnitude: its low 32
// bits, read as signed, are its value.
__device__ __forceinline__ void divmod_q32(uint32_t xh, uint32_t xl, uint32_t f, uint32_t& q, uint32_t& r) {
    const double fd = static_cast<double>(f);
    double rc = __builtin_amdgcn_rcp(fd);
    rc = __fma_rn(rc, __fma_rn(-fd, rc, 1.0), rc);
    double dh, dl;
    __asm__("v_cvt_f64_u32 %0, %1" : "=v"(dh) : "v"(xh));
    __asm__("v_cvt_f64_u32 %0, %1" : "=v"(dl) : "v"(xl));
    const double est = __fma_rn(__fma_rn(dh, 4294967296.0, dl), rc, 0.5);
    uint32_t q0;
    __asm__("v_cvt_u32_f64 %0, %1" : "=v"(q0) : "v"(est));
    const int32_t rem = static_cast<int32_t>(xl - q0 * f);
    const uint32_t neg = static_cast<uint32_t>(rem >> 31);     // all ones when x - q0 f < 0
    q = q0 + neg;
    r = static_cast<uint32_t>(rem) + (neg & f);
}

// Both cell edges of the bf16 symbol with bit pattern u: the inner edge
// (towards zero) is the midpoint below the magnitude, the outer edge the
// midpoint above; the -max / +max cells open to -inf / +inf, Inf and NaN
// patterns get two infinite edges, and the edge between -0 and +0 is 0.
__device__ __forceinline__ void bf16_cell_edges(uint32_t u, float& lo, float& hi) {
    const uint32_t m = u & 0x7FFFu;
    uint32_t ob = (m << 16) | 0x8000u;
    uint32_t ib = ob - 0x10000u;
    ob = m >= 0x7F7Fu ? 0x7F800000u : ob;
    ib = m >= 0x7F80u ? 0x7F800000u : ib;
    ib = m == 0u ? 0u : ib;
    const uint32_t sb = (u & 0x8000u) << 16;
    const bool neg = sb != 0u;
    lo = __uint_as_float((neg ? ob : ib) | sb);
    hi = __uint_as_float((neg ? ib : ob) | sb);
}

}  // namespace kvc
