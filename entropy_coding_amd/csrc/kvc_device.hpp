// Device-side building blocks of the KVC-1 coder for gfx950: the ordered
// alphabet, cell edges, the integer Phi and the mixture CDF.  Every
// floating-point step is a single IEEE float32 operation with round to
// nearest (no contraction, denormals kept), so the CDF is bit-identical to
// the host-side specification; everything after the argument is integer.
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
constexpr int kLanes = 64;                    // rANS lanes per chunk = one wavefront
constexpr int kStateBytes = 8 * kLanes;       // final states at the head of a chunk
constexpr int kPhiEntries = 4098;             // Phi(-8 + k/256), k = 0..4096, plus a copy
constexpr int kHeaderBytes = 128;

template <int KV> struct Alphabet;
template <> struct Alphabet<kBF16> {
    static constexpr uint32_t kSize = 65536;
    static constexpr int kLog2 = 16;
    using Bits = uint16_t;
};
template <> struct Alphabet<kE4M3> {
    static constexpr uint32_t kSize = 256;
    static constexpr int kLog2 = 8;
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

// Integer Phi of z = q / 2^24, q in [-2^27, 2^27]: table step 1/256 with
// integer linear interpolation over the 16 low bits.
__device__ __forceinline__ uint32_t phi_fx(int32_t q, const uint32_t* __restrict__ phi) {
    const uint32_t u = static_cast<uint32_t>(q + (1 << 27));
    const uint32_t i = u >> 16, r = u & 0xFFFFu;
    const uint32_t a = phi[i], c = phi[i + 1];
    return a + static_cast<uint32_t>((static_cast<uint64_t>(c - a) * r) >> 16);
}

struct Budgets {
    uint32_t tn, tw;                  // narrow and wide Gaussian budgets
    const uint32_t* __restrict__ prefix;  // escape prefix (N + 1 entries) or null
};

// C(b) = b + floor(T_n Phi(q1) / 2^31) + floor(T_w Phi(floor(q/3)) / 2^31) + prefix[b]
// with q = rint(clamp((edge(b) - mu) * inv, +-24) * 2^24) and q1 = clamp(q, +-2^27).
template <int KV>
__device__ __forceinline__ uint32_t cdf_at(uint32_t b, float mu, float inv,
                                           const uint32_t* __restrict__ phi, const Budgets& m) {
    const float d = __fsub_rn(edge<KV>(b), mu);
    float z = __fmul_rn(d, inv);
    z = fminf(fmaxf(z, -24.0f), 24.0f);
    const int32_t q = __float2int_rn(z * 16777216.0f);
    const int32_t q1 = min(max(q, -(1 << 27)), 1 << 27);
    // floor(q / 3): shift q by 3 * 2^28 so the dividend is non-negative
    const int32_t q3 = static_cast<int32_t>(static_cast<uint32_t>(q + 3 * (1 << 28)) / 3u) - (1 << 28);
    const uint32_t g1 = static_cast<uint32_t>((static_cast<uint64_t>(m.tn) * phi_fx(q1, phi)) >> 31);
    const uint32_t g3 = static_cast<uint32_t>((static_cast<uint64_t>(m.tw) * phi_fx(q3, phi)) >> 31);
    uint32_t g = b + g1 + g3;
    if (m.prefix) g += m.prefix[b];
    return g;
}

// Rank of this lane among the set bits of `mask` below it.
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ bool sigma_ok(float s, float inv) {
    return __builtin_isfinite(s) && s > 0.0f && __builtin_isfinite(inv);
}

// Bits per element of a KV dtype.
__host__ __device__ constexpr int kv_bytes(int kv) { return kv == kBF16 ? 2 : 1; }

}  // namespace kvc
