// HIP kernels of the KVC-1 coder for gfx950 (MI355X).
//
// One 64-lane wavefront owns one chunk: lane l codes channel 64k + l of one
// plane over a run of tokens, so every token step reads one contiguous
// 64-element row of KV and mu per wave, and the 64 interleaved rANS states
// live in registers.  Renormalisation words are placed with two wave ballots
// and mbcnt ranks.  Each workgroup builds the mixture table (and, for the
// decoder, its inverse index and every 64th escape-prefix entry) in LDS
// from two per-device Phi tables; the escape prefix itself (256 KB for bf16)
// is read through L2 (e4m3's 1 KB prefix sits in LDS).  Sources for the
// model: wiki "Speculative KV Coding" (sections "pipeline", "mixture
// distribution"); blog post on speculative KV coding (sections "information
// theory view", "engineering choice of predictor", "deployment parameters").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {

// ---------------------------------------------------------------------------
// Phi base tables: A[k] = round(2^31 Phi(z_k)), B[k] = round(2^31 Phi(z_k/3))
// on z_k = -24 + k/256, computed on the host with the C library's erfc in
// double precision (no entry lies within 4e-6 of a rounding tie, far above
// double's error) and copied to each device once.
// ---------------------------------------------------------------------------
__device__ uint32_t g_phi_a[kTablePoints];
__device__ uint32_t g_phi_b[kTablePoints];
// Stands in for the escape prefix when the weights leave no escape part, so
// that the kernels read a prefix unconditionally (zero-initialised, never
// written).
__device__ uint32_t g_zero_prefix[65537];

void host_phi_tables(uint32_t* a, uint32_t* b) {
    for (int k = 0; k < kTablePoints; ++k) {
        const double z = -24.0 + k / 256.0;
        const double s = 0.70710678118654752440;
        a[k] = static_cast<uint32_t>(std::floor(std::ldexp(0.5 * std::erfc(-z * s), 31) + 0.5));
        b[k] = static_cast<uint32_t>(std::floor(std::ldexp(0.5 * std::erfc(-(z / 3.0) * s), 31) + 0.5));
    }
}

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_phi_once[kMaxDevices];
PhiTables g_phi_dev[kMaxDevices];
hipError_t g_phi_err[kMaxDevices];
}  // namespace

PhiTables device_phi_tables(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = (e != hipSuccess) ? e : hipErrorInvalidDevice;
        return PhiTables{nullptr, nullptr, nullptr};
    }
    std::call_once(g_phi_once[dev], [dev]() {
        static uint32_t ha[kTablePoints], hb[kTablePoints];
        host_phi_tables(ha, hb);
        hipError_t r = hipMemcpyToSymbol(HIP_SYMBOL(g_phi_a), ha, sizeof(ha), 0, hipMemcpyHostToDevice);
        if (r == hipSuccess) r = hipMemcpyToSymbol(HIP_SYMBOL(g_phi_b), hb, sizeof(hb), 0, hipMemcpyHostToDevice);
        void* pa = nullptr;
        void* pb = nullptr;
        void* pz = nullptr;
        if (r == hipSuccess) r = hipGetSymbolAddress(&pa, HIP_SYMBOL(g_phi_a));
        if (r == hipSuccess) r = hipGetSymbolAddress(&pb, HIP_SYMBOL(g_phi_b));
        if (r == hipSuccess) r = hipGetSymbolAddress(&pz, HIP_SYMBOL(g_zero_prefix));
        g_phi_err[dev] = r;
        g_phi_dev[dev] = PhiTables{static_cast<const uint32_t*>(pa), static_cast<const uint32_t*>(pb),
                                   static_cast<const uint32_t*>(pz)};
    });
    *err = g_phi_err[dev];
    return g_phi_dev[dev];
}

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
// H[k] = floor(T_n A[k] / 2^31) + floor(T_w B[k] / 2^31), H[12289] = H[12288].
__device__ __forceinline__ void build_table_lds(uint32_t* s_tab, const PhiTables& phi, uint32_t tn, uint32_t tw) {
    for (int k = threadIdx.x; k < kTableEntries; k += blockDim.x) {
        const int kk = k < kTablePoints ? k : kTablePoints - 1;
        const uint32_t h = static_cast<uint32_t>((static_cast<uint64_t>(tn) * phi.a[kk]) >> 31) +
                           static_cast<uint32_t>((static_cast<uint64_t>(tw) * phi.b[kk]) >> 31);
        s_tab[k] = h;
    }
    __syncthreads();
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

struct ChunkPos {
    int64_t g;
    uint32_t t0, len, k;
};

__device__ __forceinline__ ChunkPos chunk_pos(const ChunkGeom& geo, int64_t c) {
    ChunkPos p;
    p.k = static_cast<uint32_t>(c % geo.n_groups);
    const int64_t rest = c / geo.n_groups;
    const uint32_t tc = static_cast<uint32_t>(rest % geo.n_tok_chunks);
    p.g = rest / geo.n_tok_chunks;
    p.t0 = tc * geo.chunk_tokens;
    const int64_t left = geo.tokens - static_cast<int64_t>(p.t0);
    p.len = static_cast<uint32_t>(left < geo.chunk_tokens ? left : geo.chunk_tokens);
    return p;
}

// ---------------------------------------------------------------------------
// control block and side-information checksum
// ---------------------------------------------------------------------------
__global__ void k_clear_control(Control* ctl) {
    uint32_t* w = reinterpret_cast<uint32_t*>(ctl);
    if (threadIdx.x < sizeof(Control) / 4) w[threadIdx.x] = 0u;
}

hipError_t launch_clear_control(Control* ctl, hipStream_t s) {
    hipLaunchKernelGGL(k_clear_control, dim3(1), dim3(64), 0, s, ctl);
    return hipGetLastError();
}

// splitmix64 output function (Vigna's published constants).
__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) k_side_hash(const uint32_t* __restrict__ sigma_words, uint64_t n1,
                                                   const uint32_t* __restrict__ prefix, uint64_t n2,
                                                   Control* ctl) {
    const unsigned long long golden = 0x9E3779B97F4A7C15ull;
    unsigned long long acc = 0;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t j = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < n1 + n2; j += stride) {
        unsigned long long i, w, tag;
        if (j < n1) { i = j; w = sigma_words[j]; tag = 1; }
        else { i = j - n1; w = prefix[j - n1]; tag = 2; }
        acc += mix64(((i << 32) | w) + tag * golden);
    }
    acc = wave_sum_u64(acc);
    if ((threadIdx.x & 63) == 0 && acc) atomicAdd(&ctl->side_hash, acc);
}

hipError_t launch_side_hash(const float* sigma, uint64_t n_sigma, const uint32_t* prefix,
                            uint64_t n_prefix, Control* ctl, hipStream_t s) {
    const uint64_t n = n_sigma + n_prefix;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 512) blocks = 512;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_side_hash, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(sigma), n_sigma, prefix, n_prefix, ctl);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// e4m3: the 257 cell edges and the 257-entry escape prefix fit in LDS, so the
// small alphabet's CDF needs no global reads and no edge arithmetic.
// Layout of a block's table: prefix[0..256], then edges (fp32) at
// kE4EdgeOff .. kE4EdgeOff + 256.
// ---------------------------------------------------------------------------
constexpr int kE4EdgeOff = 260;
constexpr int kE4Words = kE4EdgeOff + 257;

__device__ __forceinline__ void build_e4_lds(uint32_t* t, const uint32_t* __restrict__ prefix) {
    for (int j = threadIdx.x; j <= 256; j += blockDim.x) {
        t[j] = prefix[j];
        t[kE4EdgeOff + j] = __float_as_uint(edge_e4m3(static_cast<uint32_t>(j)));
    }
}

__device__ __forceinline__ float e4_edge(const uint32_t* t, uint32_t b) {
    return __uint_as_float(t[kE4EdgeOff + b]);
}

// Nearest e4m3 cell edge to x, for aiming only: the magnitude pattern h of
// |x| truncated to the e4m3 grid (3 mantissa bits; steps of 2^-9 below 2^-6)
// puts |x| between symbols h and h + 1, whose midpoint is the nearest edge.
__device__ __forceinline__ uint32_t nearest_edge_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    const float ax = __builtin_fabsf(x);
    int32_t h = ax < 0x1p-6f ? static_cast<int32_t>(ax * 512.0f)
                             : static_cast<int32_t>((u & 0x7FFFFFFFu) >> 20) - (120 << 3);
    h = h < 126 ? h : 126;
    return (u >> 31) ? static_cast<uint32_t>(127 - h) : static_cast<uint32_t>(129 + h);
}

// ---------------------------------------------------------------------------
// encoder: one wave per chunk, tokens last to first.  The model side of a
// batch of tokens (loads, symbol, both CDF edges) does not depend on the
// coder state, so it runs ahead of the serial rANS pushes.
// ---------------------------------------------------------------------------
constexpr int kEncodeBlock = 1024;
constexpr int kEncodeBatch = 5;

struct PushState {
    uint32_t xl, xh;                 // 64-bit rANS state
    uint32_t wp;                     // words left free in the slot (wave-uniform)
};

// A symbol's f slots: its Gaussian slots G(s) .. G(s+1) - 1 in
// [0, T_n + T_w), then its floor-and-escape slots T_n + T_w + Q(s) ..
// (Q(s) = s + prefix[s]).  slot(r) = g0 + r for r < fg, else qb + r with
// qb = T_n + T_w + Q(s) - fg.
struct SymSlots {
    uint32_t g0, fg, qb, f;
};

// Push one symbol onto the 64 lane states; emitted words go to the slot
// block of this token step, in decoder read order.
__device__ __forceinline__ void rans_push(PushState& st, const SymSlots& y, uint16_t* __restrict__ slot) {
    const uint32_t f = y.f;
    const bool e1 = st.xh >= f;               // x / 2^32 >= f: one word out
    const bool e2 = (st.xh >> 16) >= f;       // x / 2^48 >= f: two words out
    const uint64_t m1 = __ballot(e1);
    const uint64_t m2 = __ballot(e2);
    const uint32_t n1 = __popcll(m1), n2 = __popcll(m2);
    st.wp -= n1 + n2;
    // wave-uniform bases in scalar registers, 32-bit lane offsets
    char* r1 = reinterpret_cast<char*>(slot + st.wp);
    char* r2 = reinterpret_cast<char*>(slot + st.wp + n1);
    if (e1) *reinterpret_cast<uint16_t*>(r1 + 2u * lane_rank(m1)) = static_cast<uint16_t>(e2 ? (st.xl >> 16) : st.xl);
    if (e2) *reinterpret_cast<uint16_t*>(r2 + 2u * lane_rank(m2)) = static_cast<uint16_t>(st.xl);
    // drop the emitted words: x >> 16 per word (e2 implies e1)
    const uint32_t sh = e2 ? 32u : (e1 ? 16u : 0u);
    const unsigned long long xs = ((static_cast<unsigned long long>(st.xh) << 32) | st.xl) >> sh;
    const uint32_t lo = static_cast<uint32_t>(xs), hi = static_cast<uint32_t>(xs >> 32);
    uint32_t q, r;
    divmod_q32(hi, lo, f, q, r);
    // x = q * 2^31 + slot(r), slot < 2^31: no carry into bit 31
    const uint32_t sl = r + (r < y.fg ? y.g0 : y.qb);
    st.xh = q >> 1;
    st.xl = (q << 31) | sl;
}

// Slots of the symbol with bit pattern kb under the mixture: ga, gb are the
// mixture-table values at its two cell edges (in either order), s its index.
__device__ __forceinline__ SymSlots make_slots(uint32_t s, uint32_t ga, uint32_t gb, const Model& m, uint32_t htot) {
    const uint32_t g0 = __builtin_elementwise_min(ga, gb);
    const uint32_t fg = __builtin_elementwise_max(ga, gb) - g0;
    const uint32_t p0 = m.prefix[s], p1 = m.prefix[s + 1];
    SymSlots y;
    y.g0 = g0;
    y.fg = fg;
    y.qb = htot + s + p0 - fg;
    y.f = fg + 1u + (p1 - p0);
    return y;
}

template <int KV, int MU>
__device__ __forceinline__ SymSlots symbol_slots(uint32_t kb, float mu, float inv24, const Model& m, uint32_t htot) {
    if constexpr (KV == kBF16 && MU == kBF16) {
        // ord(u): u ^ 0x8000 for a positive pattern, u ^ 0xFFFF for a negative one
        const uint32_t s = (kb ^ 0x8000u) ^ (static_cast<uint32_t>(static_cast<int32_t>(kb << 16) >> 31) & 0x7FFFu);
        // both cell edges carry the value's sign; h is monotone in the
        // position, so the lower edge's h is the smaller one on either side
        uint32_t mg = kb & 0x7FFFu;
        mg = __builtin_elementwise_min(mg, 0x7F80u);                  // Inf and NaN as Inf
        const uint32_t ob0 = (mg << 16) | 0x8000u;
        const uint32_t ib = __builtin_elementwise_sub_sat(ob0, 0x10000u);  // 0 for +-0
        const uint32_t ob = __builtin_elementwise_min(ob0, 0x7F800000u);
        const uint32_t sb = (kb & 0x8000u) << 16;
        const uint32_t ha = h_fx(z_fixed(__uint_as_float(ib | sb), mu, inv24), m.tab);
        const uint32_t hb = h_fx(z_fixed(__uint_as_float(ob | sb), mu, inv24), m.tab);
        return make_slots(s, ha, hb, m, htot);
    }
    const uint32_t s = order_of_bits<KV>(kb);
    if constexpr (KV == kE4M3) {
        const uint32_t ha = h_fx(z_fixed(e4_edge(m.small, s), mu, inv24), m.tab);
        const uint32_t hb = h_fx(z_fixed(e4_edge(m.small, s + 1u), mu, inv24), m.tab);
        const uint32_t p0 = m.small[s], p1 = m.small[s + 1u];
        SymSlots y;
        y.g0 = ha;
        y.fg = hb - ha;
        y.qb = htot + s + p0 - y.fg;
        y.f = y.fg + 1u + (p1 - p0);
        return y;
    }
    float lo, hi;
    bf16_cell_edges(kb, lo, hi);
    const uint32_t ha = h_fx(z_fixed(lo, mu, inv24), m.tab);
    const uint32_t hb = h_fx(z_fixed(hi, mu, inv24), m.tab);
    return make_slots(s, ha, hb, m, htot);
}

// Element `lane` of a row whose base is wave-uniform: the base stays in
// scalar registers and the lane adds a 32-bit byte offset.
template <typename T>
__device__ __forceinline__ const T& row_elem(const T* __restrict__ row, uint32_t lane) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(row) + lane * static_cast<uint32_t>(sizeof(T)));
}

template <int KV, int MU, int U>
__device__ __forceinline__ void encode_batch(int t, PushState& st, const typename Alphabet<KV>::Bits* __restrict__ kvb,
                                             const typename MuT<MU>::T* __restrict__ mub, uint32_t D, uint32_t lane,
                                             float inv24, const Model& m, uint32_t htot, uint16_t* __restrict__ slot) {
    uint32_t kb[U];
    typename MuT<MU>::T mb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t row = static_cast<uint64_t>(t - u) * D;
        kb[u] = row_elem(kvb + row, lane);
        mb[u] = row_elem(mub + row, lane);
    }
    SymSlots y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) y[u] = symbol_slots<KV, MU>(kb[u], mu_value<MU>(mb[u]), inv24, m, htot);
#pragma unroll
    for (int u = 0; u < U; ++u) rans_push(st, y[u], slot);
}

template <int KV, int MU>
__global__ void __launch_bounds__(kEncodeBlock) k_encode(EncodeArgs a) {
    __shared__ uint32_t s_tab[kTableEntries];
    __shared__ uint32_t s_small[KV == kE4M3 ? kE4Words : 1];
    if constexpr (KV == kE4M3) build_e4_lds(s_small, a.prefix);
    build_table_lds(s_tab, a.phi, a.tn, a.tw);

    const uint32_t lane = threadIdx.x & 63u;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * (kEncodeBlock / 64) + wave;
    if (chunk >= a.geom.n_chunks) return;
    const ChunkPos cp = chunk_pos(a.geom, chunk);
    const uint32_t D = static_cast<uint32_t>(a.geom.channels);

    const float sigma = a.sigma[cp.g * D + cp.k * 64 + lane];
    float inv24 = __frcp_rn(sigma) * 16777216.0f;
    if (__ballot(!sigma_ok(sigma))) {
        if (lane == 0) atomicOr(&a.ctl->flags, kFlagBadSigma);
        inv24 = 16777216.0f;
    }
    const Model m{s_tab, a.prefix, s_small};

    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    // wave-uniform bases; lanes index them with 32-bit offsets
    const int64_t row0 = (cp.g * a.geom.tokens + cp.t0) * static_cast<int64_t>(D) + cp.k * 64;
    const KB* __restrict__ kvb = static_cast<const KB*>(a.kv) + row0;
    const MT* __restrict__ mub = static_cast<const MT*>(a.mu) + row0;
    uint16_t* __restrict__ slot = a.slots + static_cast<uint64_t>(chunk) * a.slot_words;

    PushState st{static_cast<uint32_t>(kL), kLHi, static_cast<uint32_t>(a.slot_words)};
    int t = static_cast<int>(cp.len) - 1;
    const uint32_t htot = a.tn + a.tw;
    for (; t >= kEncodeBatch - 1; t -= kEncodeBatch)
        encode_batch<KV, MU, kEncodeBatch>(t, st, kvb, mub, D, lane, inv24, m, htot, slot);
    for (; t >= 0; --t) encode_batch<KV, MU, 1>(t, st, kvb, mub, D, lane, inv24, m, htot, slot);

    a.states[chunk * 64 + lane] = (static_cast<unsigned long long>(st.xh) << 32) | st.xl;
    if (lane == 0) a.chunk_words[chunk] = static_cast<uint32_t>(a.slot_words) - st.wp;
}

hipError_t launch_encode(const EncodeArgs& a, int kv_dtype, int mu_dtype, hipStream_t s) {
    constexpr int waves = kEncodeBlock / 64;
    const uint64_t blocks = (static_cast<uint64_t>(a.geom.n_chunks) + waves - 1) / waves;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(kEncodeBlock);
    if (kv_dtype == kBF16 && mu_dtype == kBF16) hipLaunchKernelGGL((k_encode<kBF16, kBF16>), grid, block, 0, s, a);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) hipLaunchKernelGGL((k_encode<kBF16, kF32>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) hipLaunchKernelGGL((k_encode<kE4M3, kBF16>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) hipLaunchKernelGGL((k_encode<kE4M3, kF32>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// stream compaction: exclusive scan of chunk sizes (one workgroup, wave
// scans), then one workgroup per chunk copies states and words to the
// chunk's final offset with 8-byte stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long chunk_bytes(uint32_t words) {
    return (static_cast<unsigned long long>(kStateBytes) + 2ull * words + 7ull) & ~7ull;
}

__device__ __forceinline__ unsigned long long wave_inclusive_scan(unsigned long long v) {
    const int lane = threadIdx.x & 63;
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

__global__ void __launch_bounds__(1024) k_scan(const uint32_t* __restrict__ words, int64_t n,
                                               unsigned long long* __restrict__ dir, Control* ctl) {
    __shared__ unsigned long long s_wave[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t per = (n + 1023) / 1024;
    const int64_t lo = tid * per;
    const int64_t hi = (lo + per < n) ? lo + per : n;
    unsigned long long local = 0;
    for (int64_t i = lo; i < hi; ++i) local += chunk_bytes(words[i]);
    const unsigned long long inc = wave_inclusive_scan(local);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        unsigned long long w = (lane < 16) ? s_wave[lane] : 0ull;
        const unsigned long long wi = wave_inclusive_scan(w);
        if (lane < 16) s_wave[lane] = wi - w;      // exclusive over waves
    }
    __syncthreads();
    unsigned long long run = s_wave[wave] + inc - local;
    for (int64_t i = lo; i < hi; ++i) {
        dir[i] = run;
        run += chunk_bytes(words[i]);
    }
    if (tid == 1023) {
        dir[n] = run;
        ctl->total_payload = run;
    }
}

hipError_t launch_scan(const uint32_t* chunk_words, int64_t n_chunks, unsigned long long* directory,
                       Control* ctl, hipStream_t s) {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, chunk_words, n_chunks, directory, ctl);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) k_compact(CompactArgs a, StreamHeader h) {
    const int64_t n = a.geom.n_chunks;
    const unsigned long long total = a.ctl->total_payload;
    const uint64_t dir_off = kHeaderBytes;
    const uint64_t pay_off = dir_off + 8ull * static_cast<uint64_t>(n + 1);
    if (pay_off + total > a.out_capacity) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&a.ctl->flags, kFlagCapacity);
        return;
    }
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid < kHeaderBytes / 8) {
        unsigned long long w;
        __builtin_memcpy(&w, h.bytes + 8 * tid, 8);
        if (tid == 72 / 8) w = total;
        if (tid == 80 / 8) w = a.ctl->side_hash;
        reinterpret_cast<unsigned long long*>(a.out)[tid] = w;
    }
    unsigned long long* odir = reinterpret_cast<unsigned long long*>(a.out + dir_off);
    for (int64_t c = blockIdx.x; c < n; c += gridDim.x) {
        const unsigned long long beg = a.directory[c];
        if (tid == 0) {
            odir[c] = beg;
            if (c == n - 1) odir[n] = total;
        }
        uint8_t* dst = a.out + pay_off + beg;
        if (tid < 64) reinterpret_cast<unsigned long long*>(dst)[tid] = a.states[c * 64 + tid];
        // words [w0, w0 + nw) of the slot -> dst + 512, zero padded to 8 bytes;
        // the slot is 8-byte aligned, so read aligned dwords and realign by
        // half a dword when w0 is odd
        const uint32_t nw = a.chunk_words[c];
        const uint64_t w0 = a.slot_words - nw;
        const uint32_t* src32 = reinterpret_cast<const uint32_t*>(a.slots + static_cast<uint64_t>(c) * a.slot_words);
        const uint32_t s_dw = static_cast<uint32_t>(w0 >> 1);                    // first source dword
        const bool odd = (w0 & 1) != 0;
        const uint32_t out_dw = static_cast<uint32_t>((chunk_bytes(nw) - kStateBytes) / 4);   // multiple of 2
        const uint32_t src_end_dw = static_cast<uint32_t>(a.slot_words >> 1);   // exclusive
        uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + kStateBytes);
        for (uint32_t i = 2 * tid; i < out_dw; i += 2 * blockDim.x) {
            uint32_t v[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const uint32_t sd = s_dw + i + j;
                v[j] = sd < src_end_dw ? src32[sd] : 0u;
            }
            uint32_t o0 = odd ? __builtin_amdgcn_alignbit(v[1], v[0], 16) : v[0];
            uint32_t o1 = odd ? __builtin_amdgcn_alignbit(v[2], v[1], 16) : v[1];
            // words past nw are padding
            const uint32_t wi = 2 * i;                     // first word of o0
            if (wi + 0 >= nw) o0 = 0u;
            else if (wi + 1 >= nw) o0 &= 0xFFFFu;
            if (wi + 2 >= nw) o1 = 0u;
            else if (wi + 3 >= nw) o1 &= 0xFFFFu;
            *reinterpret_cast<uint2*>(d32 + i) = make_uint2(o0, o1);
        }
    }
}

hipError_t launch_compact(const CompactArgs& a, const StreamHeader& h, hipStream_t s) {
    int64_t blocks = a.geom.n_chunks;
    if (blocks > 65535) blocks = 65535;
    hipLaunchKernelGGL(k_compact, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, a, h);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// decoder: one wave per chunk, tokens first to last.
//
// A target below T_n + T_w is a Gaussian slot: the symbol s has
// G(s) <= target < G(s+1) with G the mixture-table term alone.  The aim
// inverts G through a float table of z at evenly spaced values of it; the
// edge E nearest the aimed position and one neighbour are evaluated
// exactly.  Lanes the aim misses (0.07% of symbols on the 8B-shaped
// workload) are resolved one at a time by the whole wave: 63 lanes probe
// the missing lane's bracket at once (geometrically spaced from the known end
// first, then evenly).  A target above is a floor-and-escape slot, whose
// symbol depends only on the static prefix: the wave looks it up (three
// ballot rounds), then evaluates G at the symbol's two edges for its
// frequency.  The result is exact whatever the aim; the aim only sets the
// cost.
// ---------------------------------------------------------------------------
constexpr int kDecodeBlock = 1024;
constexpr int kDecodeBatch = 4;
constexpr int kZinvSteps = 4096;

// zinv[j] = z at which the (interpolated) mixture table reaches
// floor(j * htot / kZinvSteps); one repeated entry past the end lets the aim
// truncate without a bound check.
__device__ __forceinline__ void build_zinv_lds(float* s_zinv, const uint32_t* s_tab, uint32_t htot) {
    for (int j = threadIdx.x; j <= kZinvSteps + 1; j += blockDim.x) {
        const int jj = j > kZinvSteps ? kZinvSteps : j;
        const uint32_t e = static_cast<uint32_t>((static_cast<uint64_t>(htot) * jj) / kZinvSteps);
        uint32_t lo = 0, hi = kTablePoints;           // largest k with H[k] <= e
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (s_tab[mid] <= e) lo = mid;
            else hi = mid;
        }
        float z;
        if (lo >= static_cast<uint32_t>(kTablePoints - 1)) {
            z = static_cast<float>(kTableZMax);
        } else {
            const float fr = static_cast<float>(e - s_tab[lo]) / static_cast<float>(s_tab[lo + 1] - s_tab[lo]);
            z = (static_cast<float>(lo) + fr) * (1.0f / 256.0f) - static_cast<float>(kTableZMax);
        }
        s_zinv[j] = z;
    }
    __syncthreads();
}

struct Aim {
    const float* __restrict__ zinv;    // LDS
    float scale;                       // kZinvSteps / htot (0 when there is no Gaussian part)
};

// Position where H reaches `e` (clamped to [0, htot]).
__device__ __forceinline__ float aim_pos(int32_t e, float mu, float sg, const Aim& a) {
    const float ef = __builtin_amdgcn_fmed3f(static_cast<float>(e) * a.scale, 0.0f, static_cast<float>(kZinvSteps));
    const int j = static_cast<int>(ef);                // ef >= 0: truncation is floor
    const float fr = __builtin_amdgcn_fractf(ef);
    const float z0 = a.zinv[j], z1 = a.zinv[j + 1];
    const float z = __fmaf_rn(fr, z1 - z0, z0);
    return __fmaf_rn(z, sg, mu);
}

// bf16 edge nearest to x, as its index and the magnitude pattern of its
// position.  x is first clamped to the outer edges of -max / +max, so the
// edge is m * 2^16 + 2^15 with m the upper half of x's magnitude pattern.
// The outermost edges come out finite (the midpoints above +max and below
// -max); edge_pattern() turns them into the infinities of the format.
struct Bf16Edge {
    uint32_t e;      // edge index, kLoFinite .. kHiFinite + 1
    uint32_t mag;    // m * 2^16 + 2^15, at most 0x7F7F8000
    uint32_t sign;   // 0x80000000 when x < 0
};
constexpr uint32_t kBf16OuterMag = 0x7F7F8000u;    // midpoint above +max

__device__ __forceinline__ Bf16Edge nearest_edge_bf16(float x) {
    const float lim = __uint_as_float(kBf16OuterMag);
    const uint32_t u = __float_as_uint(__builtin_amdgcn_fmed3f(x, -lim, lim));
    const uint32_t h = u >> 16;                      // bf16 pattern below x's magnitude
    Bf16Edge r;
    r.sign = u & 0x80000000u;
    r.e = r.sign ? (h ^ 0xFFFFu) : h + 32769u;       // 32767 - m or 32769 + m
    r.mag = (u & 0x7FFF0000u) | 0x8000u;
    return r;
}

// Position of the edge with magnitude pattern `mag` (at most one step past
// kBf16OuterMag, or 0 for the edge between -0 and +0).  With a bf16 mean the
// outer edge itself may stay finite: the mean lies inside [-max, max], at
// least half a bf16 step from it, so z saturates at +-24 exactly as it does
// for an infinite edge (sigma <= 2^96).  An fp32 mean can sit beyond it, so
// there the edge becomes infinite as the format defines.
template <int MU>
__device__ __forceinline__ float edge_pattern(uint32_t mag, uint32_t sign) {
    if constexpr (MU == kBF16) mag = mag < 0x7F800000u ? mag : 0x7F800000u;
    else mag = mag < kBf16OuterMag ? mag : 0x7F800000u;
    return __uint_as_float(mag | sign);
}

// Position of bf16 edge b (any b in 0..N) through edge_pattern: magnitude
// |b - 32768| * 2^16 - 2^15 (0 for the edge between -0 and +0), negative
// below b = 32768; beyond the outer edges the pattern is pinned to Inf.
template <int MU>
__device__ __forceinline__ float edge_from_index_bf16(uint32_t b) {
    const uint32_t a = b >= 32768u ? b - 32768u : 32768u - b;
    const uint32_t mag = __builtin_elementwise_sub_sat(a << 16, 0x8000u);    // a <= 32768
    return edge_pattern<MU>(mag, b < 32768u ? 0x80000000u : 0u);
}

// G(b), the mixture-table term of the CDF at edge b, for the
// wave-cooperative search (bf16 edge from the index; e4m3 edge from LDS).
template <int KV, int MU>
__device__ __forceinline__ uint32_t gauss_probe(uint32_t b, float mu, float inv24, const Model& m) {
    if constexpr (KV == kBF16) return h_fx(z_fixed(edge_from_index_bf16<MU>(b), mu, inv24), m.tab);
    else return h_fx(z_fixed(e4_edge(m.small, b), mu, inv24), m.tab);
}

// Probe offsets for the first cooperative round: 1, 2, 3, ... then growing
// geometrically to 65535 over the 63 probing lanes.
__device__ __forceinline__ uint32_t geo_offset(int lane) {
    const float g = __builtin_amdgcn_exp2f(static_cast<float>(lane) * (16.0f / 62.0f));
    const uint32_t o = static_cast<uint32_t>(g);
    return o > static_cast<uint32_t>(lane + 1) ? o : static_cast<uint32_t>(lane + 1);
}

// Gaussian-range slot not bracketed by the aim: the whole wave resolves
// every lane with `need` set, one lane at a time.  [lo, hi) brackets the
// lane's symbol with G(lo) = glo <= target < G(hi) = ghi; `up` tells which
// end is the known near one (lo if up).  Returns s, G(s), G(s+1) - G(s).
template <int KV, int MU>
__device__ __forceinline__ void coop_gauss(bool need, uint32_t target, float mu, float inv24, bool up, uint32_t lo,
                                           uint32_t hi, uint32_t glo, uint32_t ghi, const Model& m, uint32_t geo,
                                           uint32_t& s_out, uint32_t& g0_out, uint32_t& fg_out) {
    const int lane = threadIdx.x & 63;
    uint64_t pend = __ballot(need);
    while (pend) {
        const int L = __builtin_ctzll(pend);
        pend &= pend - 1;
        const uint32_t t = __builtin_amdgcn_readlane(target, L);
        const float mL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu), L));
        const float iL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv24), L));
        const bool upL = __builtin_amdgcn_readlane(static_cast<int>(up), L) != 0;
        uint32_t a = __builtin_amdgcn_readlane(lo, L), b = __builtin_amdgcn_readlane(hi, L);
        uint32_t ga = __builtin_amdgcn_readlane(glo, L), gb = __builtin_amdgcn_readlane(ghi, L);
        bool first = true;
        for (int round = 0; round < 8 && b - a > 1; ++round) {
            const uint32_t span = b - a;
            const bool geometric = first && span > 64u;
            uint32_t p;
            if (geometric) {
                const uint32_t off = geo < span - 1u ? geo : span - 1u;
                p = upL ? a + off : b - off;
            } else {
                __builtin_assume(span <= Alphabet<KV>::kSize);      // (lane + 1) * span < 2^23
                p = a + ((static_cast<uint32_t>(lane + 1) * span) >> 6);
            }
            const bool valid = lane < 63 && p > a && p < b;
            const uint32_t c = gauss_probe<KV, MU>(valid ? p : a, mL, iL, m);
            const uint64_t mle = __ballot(valid && c <= t);
            const uint64_t mgt = __ballot(valid && c > t);
            // probe positions increase with the lane, except geometric probes
            // taken down from the upper end
            const bool rising = !(geometric && !upL);
            if (mle) {
                const int k = rising ? 63 - __builtin_clzll(mle) : __builtin_ctzll(mle);
                a = __builtin_amdgcn_readlane(p, k);
                ga = __builtin_amdgcn_readlane(c, k);
            }
            if (mgt) {
                const int k = rising ? __builtin_ctzll(mgt) : 63 - __builtin_clzll(mgt);
                b = __builtin_amdgcn_readlane(p, k);
                gb = __builtin_amdgcn_readlane(c, k);
            }
            first = false;
        }
        if (lane == L) {
            s_out = a;
            g0_out = ga;
            fg_out = gb - ga;
        }
    }
}

// Floor-and-escape slot y: the symbol s with Q(s) <= y < Q(s+1), Q(b) = b +
// prefix[b], which does not depend on the lane's model.  The whole wave
// looks each such lane up: bf16 in three ballot rounds (every 16th entry of
// the every-64th-entry LDS copy, then the 16 entries after the match, then
// the 64 exact entries of that segment, one contiguous read); e4m3 in two
// rounds over the exact LDS copy.  Returns s, Q(s), Q(s+1) - Q(s).  Lane 0
// always matches for a valid prefix (Q(0) = 0 <= y); it is counted as a
// match regardless, so a damaged prefix still keeps every index in range
// (the decode then fails its checks).
template <int KV>
__device__ __forceinline__ void escape_search(bool need, uint32_t y, const uint32_t* s_pc,
                                              const uint32_t* __restrict__ prefix, uint32_t& s_out,
                                              uint32_t& q_out, uint32_t& fq_out) {
    const uint32_t lane = threadIdx.x & 63u;
    uint64_t pend = __ballot(need);
    while (pend) {
        const int L = __builtin_ctzll(pend);
        pend &= pend - 1;
        const uint32_t yl = __builtin_amdgcn_readlane(y, L);
        uint32_t sv, q0, q1;
        if constexpr (KV == kBF16) {
            // Qc(j) = Q(64 j) = 64 j + s_pc[j], j = 0 .. 1024; Qc(0) = 0 <= y < Qc(1024)
            uint32_t j = 16u * lane;                                        // 0 .. 1008
            uint64_t le = __ballot(64u * j + s_pc[j] <= yl);
            const uint32_t k = 63u - __builtin_clzll(le | 1ull);
            j = 16u * k + (lane & 15u);                                     // <= 1023
            le = __ballot(lane < 16u && 64u * j + s_pc[j] <= yl);
            const uint32_t jj = 16u * k + (63u - __builtin_clzll(le | 1ull));
            const uint32_t b = 64u * jj + lane;                            // <= 65535
            const uint32_t qb = b + prefix[b];
            le = __ballot(qb <= yl);
            const uint32_t kk = 63u - __builtin_clzll(le | 1ull);
            sv = 64u * jj + kk;
            q0 = __builtin_amdgcn_readlane(qb, kk);
            q1 = kk < 63u ? __builtin_amdgcn_readlane(qb, kk + 1u) : 64u * (jj + 1u) + s_pc[jj + 1u];
        } else {
            // s_pc[b] = prefix[b], b = 0 .. 256
            uint32_t b = 4u * lane;                                         // 0 .. 252
            uint64_t le = __ballot(b + s_pc[b] <= yl);
            const uint32_t k = 63u - __builtin_clzll(le | 1ull);
            b = 4u * k + (lane & 3u);                                       // <= 255
            le = __ballot(lane < 4u && b + s_pc[b] <= yl);
            sv = 4u * k + (63u - __builtin_clzll(le | 1ull));
            q0 = sv + s_pc[sv];
            q1 = sv + 1u + s_pc[sv + 1u];
        }
        if (lane == static_cast<uint32_t>(L)) {
            s_out = sv;
            q_out = q0;
            fq_out = q1 - q0;
        }
    }
}

// Stream words of a chunk, staged through a per-wave LDS ring of two
// 128-word blocks.  The block after next is loaded into registers (one
// dword per lane) as soon as a block is entered and written to the ring
// when the one before it is left, so no global read sits on the serial
// decode chain; a refill read is one LDS access.
struct WordRing {
    const uint32_t* __restrict__ dw;   // chunk words as dwords (8-byte aligned)
    uint32_t n_dw;                     // dwords in the chunk's word area
    uint32_t* ring;                    // this wave's 128 dwords of LDS
    uint32_t base;                     // first word of the block being read
    uint32_t ahead;                    // this lane's dword of block base/128 + 2

    __device__ __forceinline__ uint32_t load(uint32_t block, uint32_t lane) const {
        const uint32_t d = block * 64u + lane;
        return d < n_dw ? dw[d] : 0u;
    }
    __device__ __forceinline__ void init(uint32_t lane) {
        base = 0;
        ring[lane] = load(0, lane);
        ring[64u + lane] = load(1, lane);
        ahead = load(2, lane);
    }
    // word p, base <= p < base + 256
    __device__ __forceinline__ uint32_t word(uint32_t p) const {
        return reinterpret_cast<const uint16_t*>(ring)[p & 255u];
    }
    __device__ __forceinline__ void advance(uint32_t rp, uint32_t lane) {
        if (rp >= base + 128u) {                       // wave-uniform
            // the block just left (slot of base) takes the block after next
            ring[((base >> 7) & 1u) * 64u + lane] = ahead;
            base += 128u;
            ahead = load((base >> 7) + 2u, lane);
        }
    }
};

// Every 64th escape-prefix entry in LDS, for the lookup of floor-and-escape
// slots (e4m3 keeps its whole prefix there instead).
constexpr int kCoarseEntries = 1026;             // 65536 / 64 + 1, plus one repeat

template <int KV>
struct Coarse {
    static constexpr int kShift = KV == kBF16 ? 6 : 0;
    static constexpr uint32_t kLast = Alphabet<KV>::kSize >> kShift;     // index of the entry for b = N
};

template <int KV>
__device__ __forceinline__ void build_coarse_lds(uint32_t* s_pc, const uint32_t* __restrict__ prefix) {
    constexpr uint32_t last = Coarse<KV>::kLast;
    for (uint32_t j = threadIdx.x; j <= last + 1u; j += blockDim.x) {
        const uint32_t jj = j > last ? last : j;
        s_pc[j] = prefix[jj << Coarse<KV>::kShift];
    }
}

template <int KV, int MU>
__global__ void __launch_bounds__(kDecodeBlock) k_decode(DecodeArgs a) {
    __shared__ uint32_t s_tab[kTableEntries];
    __shared__ float s_zinv[kZinvSteps + 2];
    __shared__ uint32_t s_ring[kDecodeBlock / 64][128];
    __shared__ uint32_t s_pc[kCoarseEntries];
    static_assert(kE4Words <= kCoarseEntries, "e4m3 tables share the coarse-prefix array");
    if constexpr (KV == kE4M3) build_e4_lds(s_pc, a.prefix);      // exact prefix + edges
    else build_coarse_lds<KV>(s_pc, a.prefix);
    build_table_lds(s_tab, a.phi, a.tn, a.tw);
    const uint32_t htot = a.tn + a.tw;
    build_zinv_lds(s_zinv, s_tab, htot);              // all z = 24 when htot = 0

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * (kDecodeBlock / 64) + wave;
    if (chunk >= a.geom.n_chunks) return;
    const ChunkPos cp = chunk_pos(a.geom, chunk);
    const uint32_t D = static_cast<uint32_t>(a.geom.channels);

    // the chunk's directory entry must describe an aligned, in-bounds payload
    const unsigned long long beg = a.directory[chunk], end = a.directory[chunk + 1];
    if (beg > end || end > a.payload_bytes || end - beg < kStateBytes || (beg & 7ull) || (end & 7ull)) {
        if (lane == 0) atomicOr(&a.ctl->flags, kFlagCorrupt);
        return;
    }
    const uint8_t* base = a.payload + beg;
    unsigned long long x = reinterpret_cast<const unsigned long long*>(base)[lane];
    // an encoder leaves every state in [L, 2^63); decoding keeps it there,
    // which the step below relies on (x >> 31 fits 32 bits)
    if (__ballot(x < kL || (x >> 63) != 0ull)) {
        if (lane == 0) atomicOr(&a.ctl->flags, kFlagCorrupt);
        return;
    }
    const uint32_t avail = static_cast<uint32_t>((end - beg - kStateBytes) / 2);     // a multiple of 4
    WordRing win{reinterpret_cast<const uint32_t*>(base + kStateBytes), avail / 2u, s_ring[wave], 0u, 0u};
    win.init(static_cast<uint32_t>(lane));

    const float sigma = a.sigma[cp.g * D + cp.k * 64 + lane];
    float inv24 = __frcp_rn(sigma) * 16777216.0f;
    float sg = sigma;
    if (__ballot(!sigma_ok(sigma))) {
        if (lane == 0) atomicOr(&a.ctl->flags, kFlagBadSigma);
        inv24 = 16777216.0f;
        sg = 1.0f;
    }
    const Model m{s_tab, a.prefix, s_pc};
    const Aim aim{s_zinv, htot ? static_cast<float>(kZinvSteps) / static_cast<float>(htot) : 0.0f};
    const uint32_t geo = geo_offset(lane);

    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    const int64_t row0 = (cp.g * a.geom.tokens + cp.t0) * static_cast<int64_t>(D) + cp.k * 64;
    KB* __restrict__ outp = static_cast<KB*>(a.kv_out) + row0;
    const MT* __restrict__ mup = static_cast<const MT*>(a.mu) + row0;

    uint32_t rp = 0, misses = 0;
    for (uint32_t t0 = 0; t0 < cp.len; t0 += kDecodeBatch) {
        // model side of the batch: predictor means
        float mus[kDecodeBatch];
        MT raw[kDecodeBatch];
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) {
            const uint32_t t = t0 + u < cp.len ? t0 + u : cp.len - 1;
            raw[u] = row_elem(mup + static_cast<uint64_t>(t) * D, static_cast<uint32_t>(lane));
        }
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) mus[u] = mu_value<MU>(raw[u]);
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) {
            if (t0 + u >= cp.len) break;                 // wave-uniform
            const float mu = mus[u];
            const uint32_t target = static_cast<uint32_t>(x) & (kM - 1u);
            const bool in_g = target < htot;             // a Gaussian slot
            // Gaussian slots: aim through the inverse table, check the nearest
            // edge and one neighbour.  Floor-and-escape slots: look the symbol
            // up (it does not depend on the model) and evaluate its two edges.
            uint32_t E, qe = 0, fqe = 0;
            uint32_t mag = 0, sgn = 0;                   // bf16: E's edge as magnitude pattern and sign
            if constexpr (KV == kBF16) {
                const Bf16Edge ed = nearest_edge_bf16(aim_pos(static_cast<int32_t>(target), mu, sg, aim));
                E = ed.e;
                mag = ed.mag;
                sgn = ed.sign;
            } else {
                E = nearest_edge_e4m3(aim_pos(static_cast<int32_t>(target), mu, sg, aim));
            }
            if (__ballot(!in_g)) {
                uint32_t se = 0;
                escape_search<KV>(!in_g, target - htot, s_pc, m.prefix, se, qe, fqe);
                if (!in_g) {
                    E = se;
                    if constexpr (KV == kBF16) {
                        const uint32_t ad = se >= 32768u ? se - 32768u : 32768u - se;
                        mag = __builtin_elementwise_sub_sat(ad << 16, 0x8000u);     // 0 for the edge 0
                        sgn = se < 32768u ? 0x80000000u : 0u;
                    }
                }
                misses += in_g ? 0u : 1u;
            }
            uint32_t gE, gE2, E2, p0, p1, p2;
            bool up;
            if constexpr (KV == kBF16) {
                // prefix at E-1, E, E+1 (one 12-byte read; escape lanes use
                // their lookup instead, so their base is only kept in range)
                const uint32_t pb = E - 1u < 65535u ? E - 1u : 0u;          // reads pb .. pb + 2 <= N
                const uint32_t* pp = m.prefix + pb;
                p0 = pp[0];
                p1 = pp[1];
                p2 = pp[2];
                gE = h_fx(z_fixed(edge_pattern<MU>(mag, sgn), mu, inv24), m.tab);
                up = !in_g || target >= gE;
                // the neighbour one step away from zero (up on the positive
                // side) or towards it; away from the edge 0 is 2^15
                const bool outward = up != (sgn != 0u);
                const uint32_t mag2 = outward ? ((mag + 0x8000u) | 0x8000u) : __builtin_elementwise_sub_sat(mag, 0x10000u);
                E2 = up ? E + 1u : E - 1u;
                gE2 = h_fx(z_fixed(edge_pattern<MU>(mag2, sgn), mu, inv24), m.tab);
            } else {
                const uint32_t pb = E - 1u < 255u ? E - 1u : 0u;            // reads pb .. pb + 2 <= N
                p0 = s_pc[pb];
                p1 = s_pc[pb + 1u];
                p2 = s_pc[pb + 2u];
                gE = h_fx(z_fixed(e4_edge(s_pc, E), mu, inv24), m.tab);
                up = !in_g || target >= gE;
                E2 = up ? E + 1u : E - 1u;
                gE2 = h_fx(z_fixed(e4_edge(s_pc, E2), mu, inv24), m.tab);
            }
            uint32_t sym = up ? E : E2;
            uint32_t g0 = up ? gE : gE2;
            uint32_t fg = up ? gE2 - gE : gE - gE2;
            uint32_t qs = in_g ? sym + (up ? p1 : p0) : qe;              // Q(s)
            uint32_t fq = in_g ? 1u + (up ? p2 - p1 : p1 - p0) : fqe;    // Q(s+1) - Q(s)
            // bracketed: target < G(E+1) going up, target >= G(E-1) going down
            const bool need = in_g && ((target < gE2) != up);
            if (__ballot(need)) {
                misses += need ? 1u : 0u;
                coop_gauss<KV, MU>(need, target, mu, inv24, up, up ? E2 : 0u, up ? Alphabet<KV>::kSize : E2,
                                   up ? gE2 : 0u, up ? htot : gE2, m, geo, sym, g0, fg);
                if (need) {
                    const uint32_t* pq = KV == kBF16 ? m.prefix : s_pc;
                    const uint32_t a0 = pq[sym], a1 = pq[sym + 1u];
                    qs = sym + a0;
                    fq = 1u + (a1 - a0);
                }
            }
            // rank within the symbol's f = fg + fq slots
            const uint32_t f = fg + fq;
            const uint32_t r = in_g ? target - g0 : fg + (target - htot - qs);
            // x < 2^63, so x >> 31 fits 32 bits: one 32 x 32 -> 64 multiply-add
            x = static_cast<unsigned long long>(f) * static_cast<uint32_t>(x >> kLog2M) + r;

            // refill: a lane takes one word when x < 2^47 and a second one
            // when x < 2^31 (then x << 16 is still below 2^47); round one
            // holds one word per taking lane in lane order, round two the
            // second words, so both reads are placed before either is used
            const uint32_t xh = static_cast<uint32_t>(x >> 32), xl = static_cast<uint32_t>(x);
            const bool take1 = xh < kLHi;
            const bool take2 = xh == 0u && xl < 0x80000000u;
            const uint64_t m1 = __ballot(take1), m2 = __ballot(take2);
            const uint32_t n1 = __popcll(m1);
            const uint32_t w1 = win.word(rp + lane_rank(m1));
            const uint32_t w2 = win.word(rp + n1 + lane_rank(m2));
            const uint32_t hi1 = __builtin_amdgcn_alignbit(xh, xl, 16);     // (x << 16) >> 32
            const uint32_t lo1 = (xl << 16) | w1;
            const uint32_t lo2 = (w1 << 16) | w2;
            const uint32_t nh = take2 ? xl : (take1 ? hi1 : xh);
            const uint32_t nl = take2 ? lo2 : (take1 ? lo1 : xl);
            x = (static_cast<unsigned long long>(nh) << 32) | nl;
            rp += n1 + __popcll(m2);
            win.advance(rp, static_cast<uint32_t>(lane));
            KB* orow = outp + static_cast<uint64_t>(t0 + u) * D;
            *reinterpret_cast<KB*>(reinterpret_cast<char*>(orow) + static_cast<uint32_t>(lane) * sizeof(KB)) =
                static_cast<KB>(bits_of_order<KV>(sym));
        }
    }
    // every lane back at the initial state, the payload consumed exactly,
    // the padding zero
    bool bad = (x != kL) || (chunk_bytes(rp) != end - beg);
    if (!bad) {
        const uint32_t pad_words = avail - rp;        // 0..3
        const uint16_t* words = reinterpret_cast<const uint16_t*>(base + kStateBytes);
        if (static_cast<uint32_t>(lane) < pad_words && words[rp + lane] != 0) bad = true;
    }
    if (__ballot(bad) && lane == 0) atomicOr(&a.ctl->flags, kFlagCorrupt);
    const unsigned long long mw = wave_sum_u64(misses);
    if (lane == 0 && mw) atomicAdd(&a.ctl->misses, mw);
}

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int mu_dtype, hipStream_t s) {
    constexpr int waves = kDecodeBlock / 64;
    const uint64_t blocks = (static_cast<uint64_t>(a.geom.n_chunks) + waves - 1) / waves;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(kDecodeBlock);
    if (kv_dtype == kBF16 && mu_dtype == kBF16) hipLaunchKernelGGL((k_decode<kBF16, kBF16>), grid, block, 0, s, a);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) hipLaunchKernelGGL((k_decode<kBF16, kF32>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) hipLaunchKernelGGL((k_decode<kE4M3, kBF16>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) hipLaunchKernelGGL((k_decode<kE4M3, kF32>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// sigma calibration: one workgroup of 16 waves per (plane, 64-channel
// group); wave w sums rows w, w+16, ... in float64; the 16 partial sums are
// added in wave order, so the result does not depend on scheduling.
// Non-finite residuals carry no scale information and are skipped.
// ---------------------------------------------------------------------------
template <int KV>
__device__ __forceinline__ double kv_value_f64(typename Alphabet<KV>::Bits b) {
    if constexpr (KV == kBF16) {
        return static_cast<double>(__uint_as_float(static_cast<uint32_t>(b) << 16));
    } else {
        const uint32_t u = b;
        const uint32_t m = u & 0x7Fu;
        if (m == 0x7Fu) return __builtin_nan("");
        const double v = static_cast<double>(e4m3_magnitude(m));
        return (u & 0x80u) ? -v : v;
    }
}

// Pass 1: block (plane and 64-channel group, split) sums the squared
// residuals of a contiguous range of the reps x tokens rows.  Its 4 waves
// take every 4th row; each lane keeps one channel's float64 sum in row order
// and the waves are added in wave order, so the partial does not depend on
// scheduling.  Rows are loaded 4 at a time to keep loads in flight.
constexpr int kCalibBlock = 256;
constexpr int kCalibWaves = kCalibBlock / 64;
constexpr int kCalibUnroll = 4;

template <int KV, int MU>
__global__ void __launch_bounds__(kCalibBlock) k_calibrate_part(const void* kv_, const void* mu_, int64_t reps,
                                                                int64_t planes, int64_t tokens, int64_t channels,
                                                                CalibPart* __restrict__ part) {
    __shared__ double s_sum[kCalibWaves][64];
    __shared__ unsigned long long s_used[kCalibWaves][64];
    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    const KB* __restrict__ kv = static_cast<const KB*>(kv_);
    const MT* __restrict__ mu = static_cast<const MT*>(mu_);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t groups = channels / 64;
    const int64_t p = blockIdx.x / groups;
    const int64_t d = (blockIdx.x % groups) * 64 + lane;
    const int64_t splits = gridDim.y, s = blockIdx.y;
    const int64_t rows = reps * tokens;
    const int64_t r1 = rows * (s + 1) / splits;
    int64_t r = rows * s / splits + wave;
    int64_t rep = r / tokens, t = r - rep * tokens;      // advanced by carries below
    double acc = 0.0;
    unsigned long long used = 0;
    while (r < r1) {                                     // wave-uniform
        KB kb[kCalibUnroll];
        MT mb[kCalibUnroll];
        bool live[kCalibUnroll];
#pragma unroll
        for (int u = 0; u < kCalibUnroll; ++u) {
            live[u] = r < r1;
            if (live[u]) {
                const int64_t off = ((rep * planes + p) * tokens + t) * channels + d;
                kb[u] = kv[off];
                mb[u] = mu[off];
            }
            r += kCalibWaves;
            t += kCalibWaves;
            while (t >= tokens) {
                t -= tokens;
                ++rep;
            }
        }
#pragma unroll
        for (int u = 0; u < kCalibUnroll; ++u) {
            if (!live[u]) continue;
            const double e = kv_value_f64<KV>(kb[u]) - static_cast<double>(mu_value<MU>(mb[u]));
            const double e2 = e * e;
            if (__builtin_isfinite(e2)) {
                acc += e2;
                ++used;
            }
        }
    }
    s_sum[wave][lane] = acc;
    s_used[wave][lane] = used;
    __syncthreads();
    if (wave == 0) {
        double sum = 0.0;
        unsigned long long u = 0;
        for (int w = 0; w < kCalibWaves; ++w) {
            sum += s_sum[w][lane];
            u += s_used[w][lane];
        }
        part[s * planes * channels + p * channels + d] = CalibPart{sum, u};
    }
}

// Pass 2: one thread per (plane, channel) adds the splits in order.
__global__ void k_calibrate_final(const CalibPart* __restrict__ part, int64_t splits, int64_t n, float floor_,
                                  float* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double sum = 0.0;
    unsigned long long u = 0;
    for (int64_t s = 0; s < splits; ++s) {
        sum += part[s * n + i].sum;
        u += part[s * n + i].used;
    }
    const float sg = u ? static_cast<float>(sqrt(sum / static_cast<double>(u))) : 0.0f;
    out[i] = (sg > floor_ && __builtin_isfinite(sg)) ? sg : floor_;
}

int64_t calibrate_splits(int64_t reps, int64_t planes, int64_t tokens, int64_t channels) {
    const int64_t pairs = planes * (channels / 64);
    int64_t sp = (4096 + pairs - 1) / pairs;             // about 4096 blocks in all
    sp = sp < 1 ? 1 : (sp > kCalibSplitsMax ? kCalibSplitsMax : sp);
    const int64_t rows = reps * tokens;
    return sp > rows ? rows : sp;
}

hipError_t launch_calibrate(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps,
                            int64_t planes, int64_t tokens, int64_t channels, float sigma_floor,
                            float* sigma_out, CalibPart* part, hipStream_t s) {
    const int64_t splits = calibrate_splits(reps, planes, tokens, channels);
    const dim3 grid(static_cast<uint32_t>(planes * (channels / 64)), static_cast<uint32_t>(splits)), block(kCalibBlock);
    if (kv_dtype == kBF16 && mu_dtype == kBF16)
        hipLaunchKernelGGL((k_calibrate_part<kBF16, kBF16>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels, part);
    else if (kv_dtype == kBF16 && mu_dtype == kF32)
        hipLaunchKernelGGL((k_calibrate_part<kBF16, kF32>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels, part);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16)
        hipLaunchKernelGGL((k_calibrate_part<kE4M3, kBF16>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels, part);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32)
        hipLaunchKernelGGL((k_calibrate_part<kE4M3, kF32>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels, part);
    else return hipErrorInvalidValue;
    const int64_t n = planes * channels;
    hipLaunchKernelGGL(k_calibrate_final, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s, part, splits,
                       n, sigma_floor, sigma_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// empirical marginal: histogram in value order (integer atomics, so the
// result does not depend on order), then one workgroup turns counts + 1
// into the scaled prefix in place.
// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* __restrict__ p, uint64_t n, uint32_t v) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

template <int KV>
__global__ void __launch_bounds__(256) k_histogram(const void* samples_, uint64_t n, uint32_t* __restrict__ hist) {
    using KB = typename Alphabet<KV>::Bits;
    const KB* __restrict__ s = static_cast<const KB*>(samples_);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        atomicAdd(&hist[order_of_bits<KV>(s[i])], 1u);
}

// THREADS * PER = N.  Reads every count into registers before writing.
template <int THREADS, int PER>
__global__ void __launch_bounds__(THREADS) k_marginal_prefix(uint32_t* __restrict__ hist, uint32_t te) {
    __shared__ unsigned long long s_wave[THREADS / 64];
    constexpr int N = THREADS * PER;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t c[PER];
    unsigned long long local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        c[j] = hist[tid * PER + j] + 1u;
        local += c[j];
    }
    const unsigned long long inc = wave_inclusive_scan(local);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const unsigned long long w = (lane < THREADS / 64) ? s_wave[lane] : 0ull;
        const unsigned long long wi = wave_inclusive_scan(w);
        if (lane < THREADS / 64) s_wave[lane] = wi;          // inclusive over waves
    }
    __syncthreads();
    const unsigned long long total = s_wave[THREADS / 64 - 1];
    unsigned long long run = (wave ? s_wave[wave - 1] : 0ull) + inc - local;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        hist[tid * PER + j] = static_cast<uint32_t>((static_cast<unsigned long long>(te) * run) / total);
        run += c[j];
    }
    if (tid == THREADS - 1) hist[N] = te;
}

hipError_t launch_marginal(const void* samples, int dtype, uint64_t n, uint32_t te, uint32_t* prefix_out,
                           hipStream_t s) {
    const uint64_t nsym = dtype == kBF16 ? 65536u : 256u;
    hipLaunchKernelGGL(k_fill_u32, dim3(64), dim3(256), 0, s, prefix_out, nsym + 1, 0u);
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks == 0) blocks = 1;
    if (dtype == kBF16) {
        hipLaunchKernelGGL(k_histogram<kBF16>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, samples, n, prefix_out);
        hipLaunchKernelGGL((k_marginal_prefix<1024, 64>), dim3(1), dim3(1024), 0, s, prefix_out, te);
    } else {
        hipLaunchKernelGGL(k_histogram<kE4M3>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, samples, n, prefix_out);
        hipLaunchKernelGGL((k_marginal_prefix<256, 1>), dim3(1), dim3(256), 0, s, prefix_out, te);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bits estimates: integer model (exact f of the coder) and the continuous
// mixture over the same cells in float64
// ---------------------------------------------------------------------------
__device__ __forceinline__ double gauss_mass(double a, double b) {
    // Phi(b) - Phi(a) for a <= b; the upper-tail form avoids cancellation
    const double k = 0.70710678118654752440;
    if (a > 0.0) return 0.5 * (erfc(a * k) - erfc(b * k));
    return 0.5 * (erfc(-b * k) - erfc(-a * k));
}

template <int KV, int MU>
__global__ void __launch_bounds__(256) k_estimate(EstimateArgs a) {
    __shared__ uint32_t s_tab[kTableEntries];
    __shared__ double s_red[2][4];
    build_table_lds(s_tab, a.phi, a.tn, a.tw);
    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    const KB* __restrict__ kv = static_cast<const KB*>(a.kv);
    const MT* __restrict__ mup = static_cast<const MT*>(a.mu);
    const Model model{s_tab, a.prefix};
    const int64_t D = a.geom.channels, T = a.geom.tokens;
    const int64_t n = a.geom.planes * T * D;
    const double wn = a.w_narrow_bp / 1e4, ww = a.w_wide_bp / 1e4, we = 1.0 - wn - ww;
    double acc_i = 0.0, acc_f = 0.0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t d = i % D;
        const int64_t g = i / (T * D);
        const float sg = a.sigma[g * D + d];
        const float inv24 = __frcp_rn(sg) * 16777216.0f;
        const float mu = mu_value<MU>(mup[i]);
        const uint32_t s = order_of_bits<KV>(kv[i]);
        const uint32_t c0 = cdf_at<KV>(s, mu, inv24, model);
        const uint32_t c1 = cdf_at<KV>(s + 1, mu, inv24, model);
        acc_i += 31.0 - log2(static_cast<double>(c1 - c0));
        const double lo = edge<KV>(s), hi = edge<KV>(s + 1);
        const double m = mu, sd = sg;
        double q = wn * gauss_mass((lo - m) / sd, (hi - m) / sd) +
                   ww * gauss_mass((lo - m) / (3.0 * sd), (hi - m) / (3.0 * sd));
        if (a.te) q += we * static_cast<double>(a.prefix[s + 1] - a.prefix[s]) / a.te;
        const double b = -log2(q);
        acc_f += (b < 64.0) ? b : 64.0;
    }
    acc_i = wave_sum_f64(acc_i);
    acc_f = wave_sum_f64(acc_f);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { s_red[0][wave] = acc_i; s_red[1][wave] = acc_f; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double si = 0.0, sf = 0.0;
        for (int w = 0; w < 4; ++w) { si += s_red[0][w]; sf += s_red[1][w]; }
        atomicAdd(&a.ctl->bits[0], si);
        atomicAdd(&a.ctl->bits[1], sf);
    }
}

hipError_t launch_estimate(const EstimateArgs& a, int kv_dtype, int mu_dtype, hipStream_t s) {
    const dim3 grid(1024), block(256);
    if (kv_dtype == kBF16 && mu_dtype == kBF16) hipLaunchKernelGGL((k_estimate<kBF16, kBF16>), grid, block, 0, s, a);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) hipLaunchKernelGGL((k_estimate<kBF16, kF32>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) hipLaunchKernelGGL((k_estimate<kE4M3, kBF16>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) hipLaunchKernelGGL((k_estimate<kE4M3, kF32>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// the CDF table for given (mu, sigma) pairs
// ---------------------------------------------------------------------------
template <int KV, int MU>
__global__ void __launch_bounds__(256) k_cdf_table(const void* mu_, const float* __restrict__ sigma, int64_t pairs,
                                                   uint32_t tn, uint32_t tw, const uint32_t* __restrict__ prefix,
                                                   uint32_t* __restrict__ out, PhiTables phi) {
    __shared__ uint32_t s_tab[kTableEntries];
    build_table_lds(s_tab, phi, tn, tw);
    using MT = typename MuT<MU>::T;
    constexpr uint32_t N1 = Alphabet<KV>::kSize + 1;
    const Model model{s_tab, prefix};
    const int64_t total = pairs * N1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t p = i / N1;
        const uint32_t b = static_cast<uint32_t>(i - p * N1);
        const float mu = mu_value<MU>(static_cast<const MT*>(mu_)[p]);
        const float inv24 = __frcp_rn(sigma[p]) * 16777216.0f;
        out[i] = cdf_at<KV>(b, mu, inv24, model);
    }
}

hipError_t launch_cdf_table(int kv_dtype, int mu_dtype, uint32_t tn, uint32_t tw, const void* mu,
                            const float* sigma, int64_t pairs, const uint32_t* prefix, uint32_t* out,
                            PhiTables phi, hipStream_t s) {
    const dim3 grid(512), block(256);
    if (kv_dtype == kBF16 && mu_dtype == kBF16) hipLaunchKernelGGL((k_cdf_table<kBF16, kBF16>), grid, block, 0, s, mu, sigma, pairs, tn, tw, prefix, out, phi);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) hipLaunchKernelGGL((k_cdf_table<kBF16, kF32>), grid, block, 0, s, mu, sigma, pairs, tn, tw, prefix, out, phi);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) hipLaunchKernelGGL((k_cdf_table<kE4M3, kBF16>), grid, block, 0, s, mu, sigma, pairs, tn, tw, prefix, out, phi);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) hipLaunchKernelGGL((k_cdf_table<kE4M3, kF32>), grid, block, 0, s, mu, sigma, pairs, tn, tw, prefix, out, phi);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kvc
