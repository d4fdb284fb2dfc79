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
#include <type_traits>

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

// ---------------------------------------------------------------------------
// Student-t narrow part (optional): A[k] = round(2^31 (F(z_k) - F(-24)) /
// (F(24) - F(-24))) for Student's t with nu = 1..16 degrees of freedom,
// truncated to [-24, 24] scale units and renormalised there.  F comes from
// the finite series for integer degrees of freedom (theta = atan(|z| /
// sqrt(nu)), c = cos^2 theta; odd nu: 1/2 + (theta + sin theta cos theta
// (1 + 2/3 c + (2 4)/(3 5) c^2 + ...)) / pi; even nu: 1/2 + sin theta / 2
// (1 + 1/2 c + (1 3)/(2 4) c^2 + ...)), in double precision: every entry
// lies more than 1e-5 from a rounding tie.  Built on the host and copied to
// a device on its first call that uses it.
// ---------------------------------------------------------------------------
__host__ __device__ inline double student_t_cdf(double z, int nu) {
    const double th = atan(fabs(z) / sqrt(static_cast<double>(nu)));
    const double c = cos(th) * cos(th);
    double term = 1.0, acc = 0.0, f;
    if (nu & 1) {
        for (int k = 0; k < (nu - 1) / 2; ++k) {
            if (k) term *= (2.0 * k) / (2.0 * k + 1.0) * c;
            acc += term;
        }
        f = 0.5 + (th + sin(th) * cos(th) * acc) * 0.31830988618379067154;
    } else {
        for (int k = 0; k < nu / 2; ++k) {
            if (k) term *= (2.0 * k - 1.0) / (2.0 * k) * c;
            acc += term;
        }
        f = 0.5 + 0.5 * sin(th) * acc;
    }
    return z >= 0.0 ? f : 1.0 - f;
}

void host_narrow_table(uint32_t narrow_dof, uint32_t* a) {
    if (narrow_dof == 0) {
        static uint32_t wide[kTablePoints];
        host_phi_tables(a, wide);
        return;
    }
    const int nu = static_cast<int>(narrow_dof);
    const double lo = student_t_cdf(-kTableZMax, nu);
    const double span = 1.0 - 2.0 * lo;
    for (int k = 0; k < kTablePoints; ++k) {
        const double z = -24.0 + k / 256.0;
        a[k] = static_cast<uint32_t>(std::floor(std::ldexp((student_t_cdf(z, nu) - lo) / span, 31) + 0.5));
    }
}

__device__ uint32_t g_t_tables[kNarrowDofMax][kTablePoints];

namespace {
std::once_flag g_t_once[kMaxDevices][kNarrowDofMax];
const uint32_t* g_t_dev[kMaxDevices][kNarrowDofMax];
hipError_t g_t_err[kMaxDevices][kNarrowDofMax];
}  // namespace

PhiTables device_phi_tables(hipError_t* err, uint32_t narrow_dof) {
    PhiTables t = device_phi_tables(err);
    if (*err != hipSuccess || narrow_dof == 0) return t;
    if (narrow_dof > static_cast<uint32_t>(kNarrowDofMax)) {
        *err = hipErrorInvalidValue;
        return PhiTables{nullptr, nullptr, nullptr};
    }
    int dev = 0;
    (void)hipGetDevice(&dev);                                 // checked by the call above
    const int j = static_cast<int>(narrow_dof) - 1;
    std::call_once(g_t_once[dev][j], [dev, j, narrow_dof]() {
        static uint32_t h[kTablePoints];                      // serialised by call_once per (device, nu)
        static std::mutex m;
        std::lock_guard<std::mutex> lock(m);
        host_narrow_table(narrow_dof, h);
        hipError_t r = hipMemcpyToSymbol(HIP_SYMBOL(g_t_tables), h, sizeof(h), sizeof(h) * j, hipMemcpyHostToDevice);
        void* p = nullptr;
        if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(g_t_tables));
        g_t_err[dev][j] = r;
        g_t_dev[dev][j] = r == hipSuccess ? static_cast<const uint32_t*>(p) + static_cast<size_t>(j) * kTablePoints
                                          : nullptr;
    });
    *err = g_t_err[dev][j];
    t.a = g_t_dev[dev][j];
    return t;
}

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
// Scratch of the allocation-free decode: a fixed array in device memory
// (each device holds its own copy while the process lives).  Host code
// takes its device address once per device with hipGetSymbolAddress; the
// array's name is not a device address on the host.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_dev[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

void* noalloc_scratch(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = (e != hipSuccess) ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = r;
        g_scratch_dev[dev] = (r == hipSuccess) ? p : nullptr;
    });
    *err = g_scratch_err[dev];
    return g_scratch_dev[dev];
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

// Copy of a per-call table from global memory into LDS, 16 bytes per
// thread and step (n16 = bytes / 16); ends with a barrier.
__device__ __forceinline__ void copy_to_lds(void* dst, const void* __restrict__ src, uint32_t n16) {
    uint4* d = static_cast<uint4*>(dst);
    const uint4* __restrict__ q = static_cast<const uint4*>(src);
    for (uint32_t k = threadIdx.x; k < n16; k += blockDim.x) d[k] = q[k];
    __syncthreads();
}

// The pair table of a per-lane split: (A[k], B[k]) for k = 0 .. 12291, the
// narrow and wide base tables with their last entry repeated; ends with a
// barrier.
__device__ __forceinline__ void fill_pairs_lds(uint2* s_ab, const uint32_t* __restrict__ a,
                                               const uint32_t* __restrict__ b) {
    for (int k = threadIdx.x; k < static_cast<int>(kTableWordsPadded); k += blockDim.x) {
        const int kk = k < kTablePoints ? k : kTablePoints - 1;
        s_ab[k] = make_uint2(a[kk], b[kk]);
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
    int64_t srow;                       // row of sigma: [planes][sigma_blocks] flattened
    uint32_t t0, len, k;
};

__device__ __forceinline__ ChunkPos chunk_pos(const ChunkGeom& geo, int64_t c) {
    ChunkPos p;
    p.k = static_cast<uint32_t>(c % geo.n_groups);
    const int64_t rest = c / geo.n_groups;
    const uint32_t tc = static_cast<uint32_t>(rest % geo.n_tok_chunks);
    p.g = rest / geo.n_tok_chunks;
    // a chunk lies within one sigma block (the block length is a multiple
    // of the chunk length)
    p.srow = p.g * geo.sigma_blocks + (geo.sigma_tc ? tc / geo.sigma_tc : 0u);
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

// Slots of a bf16 symbol under the mixture: ga, gb are the mixture-table
// values at its two cell edges (in either order), q its escape slot table
// entry (T_n + T_w + Q(s), Q(s + 1) - Q(s)).
__device__ __forceinline__ SymSlots make_slots(uint32_t ga, uint32_t gb, U32Pair q) {
    const uint32_t g0 = __builtin_elementwise_min(ga, gb);
    const uint32_t fg = __builtin_elementwise_max(ga, gb) - g0;
    SymSlots y;
    y.g0 = g0;
    y.fg = fg;
    y.qb = q.a - fg;
    y.f = fg + q.b;
    return y;
}

// bf16: the escape slot table's entry of pattern kb (a global read that
// does not depend on the model); e4m3 reads its prefix from LDS instead.
template <int KV>
__device__ __forceinline__ U32Pair escape_entry(uint32_t kb, const Model& m) {
    if constexpr (KV == kBF16) return load_pair(m.eslots, kb << 3);
    else return U32Pair{0u, 0u};
}

template <int KV, int MU, class M>
__device__ __forceinline__ SymSlots symbol_slots(uint32_t kb, float mu, float inv24, const M& m, U32Pair q) {
    if constexpr (KV == kBF16 && MU == kBF16) {
        // both cell edges carry the value's sign; h is monotone in the
        // position, so the lower edge's h is the smaller one on either side
        uint32_t mg = kb & 0x7FFFu;
        mg = __builtin_elementwise_min(mg, 0x7F80u);                  // Inf and NaN as Inf
        const uint32_t ob0 = (mg << 16) | 0x8000u;
        const uint32_t ib = __builtin_elementwise_sub_sat(ob0, 0x10000u);  // 0 for +-0
        const uint32_t ob = __builtin_elementwise_min(ob0, 0x7F800000u);
        const uint32_t sb = (kb & 0x8000u) << 16;
        const uint32_t ha = m.h(z_fixed(__uint_as_float(ib | sb), mu, inv24));
        const uint32_t hb = m.h(z_fixed(__uint_as_float(ob | sb), mu, inv24));
        return make_slots(ha, hb, q);
    }
    if constexpr (KV == kE4M3) {
        const uint32_t s = order_of_bits<KV>(kb);
        const uint32_t ha = m.h(z_fixed(e4_edge(m.small, s), mu, inv24));
        const uint32_t hb = m.h(z_fixed(e4_edge(m.small, s + 1u), mu, inv24));
        const uint32_t p0 = m.small[s], p1 = m.small[s + 1u];
        SymSlots y;
        y.g0 = ha;
        y.fg = hb - ha;
        y.qb = m.htot + s + p0 - y.fg;
        y.f = y.fg + 1u + (p1 - p0);
        return y;
    }
    float lo, hi;
    bf16_cell_edges(kb, lo, hi);
    const uint32_t ha = m.h(z_fixed(lo, mu, inv24));
    const uint32_t hb = m.h(z_fixed(hi, mu, inv24));
    return make_slots(ha, hb, q);
}

// Rows of the chunk through buffer resources: the lane's byte offset in a
// vector register, the row's in a scalar one.
template <typename T>
__device__ __forceinline__ uint32_t load_row_elem(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t row_off) {
    if constexpr (sizeof(T) == 1) return __builtin_amdgcn_raw_buffer_load_b8(r, lane_off, row_off, 0);
    else if constexpr (sizeof(T) == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, lane_off, row_off, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, lane_off, row_off, 0);
}

template <int KV, int MU, int U, class M>
__device__ __forceinline__ void encode_batch(int t, PushState& st, __amdgpu_buffer_rsrc_t kvr,
                                             __amdgpu_buffer_rsrc_t mur, uint32_t D, uint32_t lane,
                                             float inv24, const M& m, uint16_t* __restrict__ slot) {
    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    uint32_t kb[U];
    float mus[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t row = static_cast<uint32_t>(t - u) * D;
        kb[u] = load_row_elem<KB>(kvr, lane * static_cast<uint32_t>(sizeof(KB)), row * static_cast<uint32_t>(sizeof(KB)));
        const uint32_t mr = load_row_elem<MT>(mur, lane * static_cast<uint32_t>(sizeof(MT)), row * static_cast<uint32_t>(sizeof(MT)));
        mus[u] = MU == kBF16 ? __uint_as_float(mr << 16) : __uint_as_float(mr);
    }
    // a non-finite mean counts as 0 (rare: one test for the batch)
    uint64_t odd = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) odd |= __ballot(!__builtin_isfinite(mus[u]));
    if (odd) {
        __asm__ volatile("");                       // a branch, not selects on every step
#pragma unroll
        for (int u = 0; u < U; ++u) mus[u] = __builtin_isfinite(mus[u]) ? mus[u] : 0.0f;
    }
    SymSlots y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) y[u] = symbol_slots<KV, MU>(kb[u], mus[u], inv24, m, escape_entry<KV>(kb[u], m));
#pragma unroll
    for (int u = 0; u < U; ++u) rans_push(st, y[u], slot);
}

// The rows of tokens t, t - 1, ..., t - U + 1 (a row before the chunk's first
// stands in as row 0: its values are never used).
template <int KV, int MU, int U>
__device__ __forceinline__ void load_rows(int t, uint32_t (&kr)[U], uint32_t (&mr)[U], __amdgpu_buffer_rsrc_t kvr,
                                          __amdgpu_buffer_rsrc_t mur, uint32_t D, uint32_t lane) {
    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t row = static_cast<uint32_t>(t - u >= 0 ? t - u : 0) * D;
        kr[u] = load_row_elem<KB>(kvr, lane * static_cast<uint32_t>(sizeof(KB)), row * static_cast<uint32_t>(sizeof(KB)));
        mr[u] = load_row_elem<MT>(mur, lane * static_cast<uint32_t>(sizeof(MT)), row * static_cast<uint32_t>(sizeof(MT)));
    }
}

// A batch whose rows were read one batch ahead (kr, mr); it reads the rows
// of the batch after it (from t_next) into the same registers.  The order of
// the reads matters: the vector-memory counter completes in order, so this
// batch's escape-entry reads are issued before the next batch's rows and
// their wait does not include those HBM reads.
template <int KV, int MU, int U, class M>
__device__ __forceinline__ void encode_batch_ahead(uint32_t (&kr)[U], uint32_t (&mr)[U], int t_next, PushState& st,
                                                   __amdgpu_buffer_rsrc_t kvr, __amdgpu_buffer_rsrc_t mur,
                                                   uint32_t D, uint32_t lane, float inv24, const M& m,
                                                   uint16_t* __restrict__ slot) {
    uint32_t kb[U];
    float mus[U];
    U32Pair q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        kb[u] = kr[u];
        mus[u] = MU == kBF16 ? __uint_as_float(mr[u] << 16) : __uint_as_float(mr[u]);
        q[u] = escape_entry<KV>(kb[u], m);
    }
    __asm__ volatile("" : : : "memory");
    load_rows<KV, MU, U>(t_next, kr, mr, kvr, mur, D, lane);
    uint64_t odd = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) odd |= __ballot(!__builtin_isfinite(mus[u]));
    if (odd) {
        __asm__ volatile("");
#pragma unroll
        for (int u = 0; u < U; ++u) mus[u] = __builtin_isfinite(mus[u]) ? mus[u] : 0.0f;
    }
    SymSlots y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) y[u] = symbol_slots<KV, MU>(kb[u], mus[u], inv24, m, q[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) rans_push(st, y[u], slot);
}

// ---------------------------------------------------------------------------
// stream layout helpers
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

// Exclusive prefix of the chunk sizes in chunk order, by decoupled look-back:
// status[c] is 0 until chunk c publishes, then kAggregate | its own size,
// then kInclusive | the sum of the sizes of chunks 0..c.  A chunk publishes
// its size, then reads the 64 entries before it at a time (lane i the
// entry i + 1 back): the nearest inclusive entry and the sizes up to it give
// its prefix; an entry not yet published between them is waited for.
// Workgroups start in index order, so every chunk waited for is running or
// done, and each publishes before it waits: every wait ends.  A wait longer
// than kLookBackSpins polls (far beyond any launch) raises kFlagStall and
// counts the entry as 0, so the kernel ends whatever happens.  The entries
// are read and written with device-scope atomics: chunks on different XCDs
// see each other's entries through memory, not their L2s.
constexpr unsigned long long kAggregate = 1ull << 62, kInclusive = 2ull << 62, kStatusValue = kAggregate - 1;
constexpr uint32_t kLookBackSpins = 1u << 18;      // polls of up to 16 x 512 cycles (about 1 s): far beyond any launch

__device__ __forceinline__ unsigned long long look_back(unsigned long long* status, int64_t chunk,
                                                        unsigned long long size, Control* ctl) {
    const int lane = threadIdx.x & 63;
    if (chunk == 0) {
        if (lane == 0) __hip_atomic_store(&status[0], kInclusive | size, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    if (lane == 0) __hip_atomic_store(&status[chunk], kAggregate | size, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long acc = 0;
    int64_t base = chunk - 1;
    uint32_t spins = 0;                              // polls so far; at the cap, no more waiting
    for (;;) {
        const int64_t idx = base - lane;
        // before chunk 0: an inclusive prefix of 0
        unsigned long long v =
            idx >= 0 ? __hip_atomic_load(&status[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kInclusive;
        uint64_t waiting = __ballot((v >> 62) == 0ull);
        uint64_t inclusive = __ballot((v >> 62) == 2ull);
        // lanes up to and including the nearest inclusive entry
        uint64_t upto = inclusive ? (inclusive ^ (inclusive - 1ull)) : ~0ull;
        if ((waiting & upto) && spins < kLookBackSpins) {
            // one entry still being coded: poll it alone (lane 0), backing off,
            // then read the window again
            const int j = __builtin_ctzll(waiting & upto);
            const unsigned long long* e = &status[base - j];
            uint32_t nap = 1;
            for (;;) {
                if (++spins >= kLookBackSpins) {
                    if (lane == 0) atomicOr(&ctl->flags, kFlagStall);
                    break;
                }
                for (uint32_t k = 0; k < nap; ++k) __builtin_amdgcn_s_sleep(8);
                nap = nap < 16u ? 2u * nap : 16u;
                unsigned long long w = 0;
                if (lane == 0) w = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(w >> 62)) != 0u) break;
            }
            continue;
        }
        const unsigned long long mine = ((upto >> lane) & 1ull) ? (v & kStatusValue) : 0ull;
        acc += wave_sum_u64(mine);
        if (inclusive) break;
        base -= 64;
    }
    if (lane == 0)
        __hip_atomic_store(&status[chunk], kInclusive | (acc + size), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return acc;
}

// CRC-32 (reflected polynomial 0xEDB88320, as zlib computes it) of the
// header's first 92 bytes, once per encode, on the last chunk's path.  The
// wave first builds the byte table in LDS (lane l: entries l, l + 64,
// l + 128, l + 192, eight bit steps each), then one lane takes a byte per
// table read: 92 dependent LDS reads instead of 736 dependent bit steps.
__device__ __forceinline__ void crc_table_wave(uint32_t* t) {
    const uint32_t lane = threadIdx.x & 63u;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        uint32_t c = lane + 64u * k;
#pragma unroll
        for (int j = 0; j < 8; ++j) c = (c >> 1) ^ ((c & 1u) ? 0xEDB88320u : 0u);
        t[lane + 64u * k] = c;
    }
}

__device__ uint32_t header_crc32(const uint8_t* b, const uint32_t* t) {
    uint32_t c = 0xFFFFFFFFu;
    for (uint32_t i = 0; i < kHeaderCrcOffset; ++i) c = t[(c ^ b[i]) & 0xFFu] ^ (c >> 8);
    return ~c;
}

// A chunk's nw words from its slot to their place in the stream, by one
// wave: the words start at src (4-byte aligned) or, when `odd`, half a dword
// after it; out_dw dwords are written (a multiple of 2), the words past nw
// as zeros.  Each lane moves 16 bytes per step and issues the loads of
// kCopyBatch steps before their stores, so that few round trips to memory
// sit on the wave's path (the slot is long out of L2 by the end of the
// chunk).  Reads may run up to 4 dwords past the slot into the workspace's
// next region; those words are past nw and masked.
constexpr int kCopyBatch = 4;

__device__ __forceinline__ void copy_words(const uint32_t* __restrict__ src, bool odd, uint32_t nw,
                                           uint32_t* __restrict__ dst, uint32_t out_dw) {
    const uint32_t lane = threadIdx.x & 63u;
    for (uint32_t base = 0; base < out_dw; base += 256u * kCopyBatch) {
        uint4 a[kCopyBatch];
        uint32_t e[kCopyBatch];
#pragma unroll
        for (int b = 0; b < kCopyBatch; ++b) {
            const uint32_t j = base + 256u * b + 4u * lane;          // first output dword of this step
            if (j < out_dw) {
                a[b] = *reinterpret_cast<const uint4*>(src + j);
                e[b] = src[j + 4];
            }
        }
#pragma unroll
        for (int b = 0; b < kCopyBatch; ++b) {
            const uint32_t j = base + 256u * b + 4u * lane;
            if (j >= out_dw) continue;
            uint32_t o[4] = {a[b].x, a[b].y, a[b].z, a[b].w};
            if (odd) {
                o[0] = __builtin_amdgcn_alignbit(a[b].y, a[b].x, 16);
                o[1] = __builtin_amdgcn_alignbit(a[b].z, a[b].y, 16);
                o[2] = __builtin_amdgcn_alignbit(a[b].w, a[b].z, 16);
                o[3] = __builtin_amdgcn_alignbit(e[b], a[b].w, 16);
            }
            // words past nw are padding
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wi = 2u * (j + q);                    // first word of dword q
                if (wi >= nw) o[q] = 0u;
                else if (wi + 1 >= nw) o[q] &= 0xFFFFu;
            }
            if (j + 4 <= out_dw) *reinterpret_cast<uint4*>(dst + j) = make_uint4(o[0], o[1], o[2], o[3]);
            else *reinterpret_cast<uint2*>(dst + j) = make_uint2(o[0], o[1]);
        }
    }
}

// SPLIT: every (plane, channel) has its own split of the Gaussian budget
// (the pair table in LDS instead of the mixture table).
template <int KV, int MU, bool SPLIT>
__global__ void __launch_bounds__(kEncodeBlock) k_encode(EncodeArgs a) {
    __shared__ __align__(16) uint32_t s_tab[SPLIT ? 2 * kTableWordsPadded : kTableWordsPadded];
    __shared__ uint32_t s_small[KV == kE4M3 ? kE4Words : 1];
    __shared__ unsigned long long s_head[kHeaderBytes / 8];        // the last chunk's header
    __shared__ uint32_t s_crc[256];                                // the last chunk's CRC-32 table
    if constexpr (KV == kE4M3) build_e4_lds(s_small, a.prefix);
    if constexpr (SPLIT) fill_pairs_lds(reinterpret_cast<uint2*>(s_tab), a.split.a, a.split.b);
    else copy_to_lds(s_tab, a.table, static_cast<uint32_t>(kTableBytes / 16));

    const uint32_t lane = threadIdx.x & 63u;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * (kEncodeBlock / 64) + wave;
    if (chunk >= a.geom.n_chunks) return;
    const ChunkPos cp = chunk_pos(a.geom, chunk);
    const uint32_t D = static_cast<uint32_t>(a.geom.channels);

    const float sigma = a.sigma[cp.srow * D + cp.k * 64 + lane];
    float inv24 = __frcp_rn(sigma) * 16777216.0f;
    if (__ballot(!sigma_ok(sigma))) {
        if (lane == 0) atomicOr(&a.ctl->flags, kFlagBadSigma);
        inv24 = 16777216.0f;
    }
    const Model base{s_tab, a.prefix, s_small, a.eslots, a.tn + a.tw};
    // a weight above w_n + w_w is refused (as a bad sigma); the budget is
    // capped meanwhile, so the chunk still codes within its slot
    const auto m = [&]() {
        if constexpr (SPLIT) {
            const uint32_t w = a.split.words[cp.g * D + cp.k * 64 + lane];
            if (__ballot(w > a.split.w_gauss) && lane == 0) atomicOr(&a.ctl->flags, kFlagBadSigma);
            const uint32_t tn = split_narrow_budget(w, a.split.t_all, base.htot);
            return SplitModel{base, tn, base.htot - tn};
        } else {
            return base;
        }
    }();

    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    // the chunk's rows of KV and mu as buffers (a chunk's rows span fewer than
    // 2^31 bytes)
    const int64_t row0 = (cp.g * a.geom.tokens + cp.t0) * static_cast<int64_t>(D) + cp.k * 64;
    const __amdgpu_buffer_rsrc_t kvb = buffer_rsrc(static_cast<const KB*>(a.kv) + row0, cp.len * D * sizeof(KB));
    const __amdgpu_buffer_rsrc_t mub = buffer_rsrc(static_cast<const MT*>(a.mu) + row0, cp.len * D * sizeof(MT));
    uint16_t* __restrict__ slot = a.slots + static_cast<uint64_t>(chunk) * a.slot_words;

    PushState st{static_cast<uint32_t>(kL), kLHi, static_cast<uint32_t>(a.slot_words)};
    int t = static_cast<int>(cp.len) - 1;
    uint32_t kr[kEncodeBatch], mr[kEncodeBatch];         // the next batch's rows, read a batch ahead
    if (t >= kEncodeBatch - 1) load_rows<KV, MU, kEncodeBatch>(t, kr, mr, kvb, mub, D, lane);
    for (; t >= kEncodeBatch - 1; t -= kEncodeBatch)
        encode_batch_ahead<KV, MU, kEncodeBatch>(kr, mr, t - kEncodeBatch, st, kvb, mub, D, lane, inv24, m, slot);
    for (; t >= 0; --t) encode_batch<KV, MU, 1>(t, st, kvb, mub, D, lane, inv24, m, slot);

    // the chunk's place in the stream: the sizes of the chunks before it
    const uint32_t nw = static_cast<uint32_t>(a.slot_words) - st.wp;
    const unsigned long long size = chunk_bytes(nw);
    const unsigned long long beg = look_back(a.status, chunk, size, a.ctl);
    const uint64_t n = static_cast<uint64_t>(a.geom.n_chunks);
    const uint64_t pay_off = kHeaderBytes + 8ull * (n + 1);
    const bool dir_fits = pay_off <= a.out_capacity;
    if (pay_off + beg + size <= a.out_capacity) {
        // the 64 final states, then the words from the slot (this wave's own
        // stores: wait for them before reading them back in other lanes),
        // zero padded to 8 bytes
        uint8_t* dst = a.out + pay_off + beg;
        reinterpret_cast<unsigned long long*>(dst)[lane] = (static_cast<unsigned long long>(st.xh) << 32) | st.xl;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        copy_words(reinterpret_cast<const uint32_t*>(slot) + (st.wp >> 1), (st.wp & 1u) != 0, nw,
                   reinterpret_cast<uint32_t*>(dst + kStateBytes), static_cast<uint32_t>((size - kStateBytes) / 4));
    } else if (lane == 0) {
        atomicOr(&a.ctl->flags, kFlagCapacity);
    }
    unsigned long long* dir = reinterpret_cast<unsigned long long*>(a.out + kHeaderBytes);
    if (lane == 0 && dir_fits) dir[chunk] = beg;
    if (static_cast<uint64_t>(chunk) + 1 == n) {
        crc_table_wave(s_crc);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");      // the table's stores before its reads
    }
    if (static_cast<uint64_t>(chunk) + 1 == n && lane == 0) {
        // the last chunk knows the payload size: directory end, header (with
        // the side-information checksum of the kernel before and its CRC),
        // and the workspace's copy of the header (also when the stream does
        // not fit, for the size it needed)
        const unsigned long long total = beg + size;
        a.ctl->total_payload = total;
        if (dir_fits) dir[n] = total;
        for (int i = 0; i < kHeaderBytes / 8; ++i) __builtin_memcpy(&s_head[i], a.header.bytes + 8 * i, 8);
        s_head[72 / 8] = total;
        s_head[80 / 8] = a.ctl->side_hash;
        const uint32_t crc = header_crc32(reinterpret_cast<const uint8_t*>(s_head), s_crc);
        s_head[kHeaderCrcOffset / 8] =
            (s_head[kHeaderCrcOffset / 8] & 0xFFFFFFFFull) | (static_cast<unsigned long long>(crc) << 32);
        for (int i = 0; i < kHeaderBytes / 8; ++i) {
            if (a.out_capacity >= static_cast<uint64_t>(kHeaderBytes)) reinterpret_cast<unsigned long long*>(a.out)[i] = s_head[i];
            reinterpret_cast<unsigned long long*>(a.header_copy)[i] = s_head[i];
        }
    }
}

hipError_t launch_encode(const EncodeArgs& a, int kv_dtype, int mu_dtype, hipStream_t s) {
    constexpr int waves = kEncodeBlock / 64;
    const uint64_t blocks = (static_cast<uint64_t>(a.geom.n_chunks) + waves - 1) / waves;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(kEncodeBlock);
    const bool sp = a.split.words != nullptr;
#define KVC_ENC(K, U)                                                                \
    do {                                                                             \
        if (sp) hipLaunchKernelGGL((k_encode<K, U, true>), grid, block, 0, s, a);    \
        else hipLaunchKernelGGL((k_encode<K, U, false>), grid, block, 0, s, a);      \
    } while (0)
    if (kv_dtype == kBF16 && mu_dtype == kBF16) KVC_ENC(kBF16, kBF16);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) KVC_ENC(kBF16, kF32);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) KVC_ENC(kE4M3, kBF16);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) KVC_ENC(kE4M3, kF32);
    else return hipErrorInvalidValue;
#undef KVC_ENC
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// decoder: one wave per chunk, tokens first to last.
//
// The rANS target t = x mod 2^31 lies either in the Gaussian range
// [0, T_n + T_w), where the symbol s is the one with G(s) <= t < G(s+1), or
// in the floor-and-escape range above it, where s is the one with
// Q(s) <= t - T_n - T_w < Q(s+1); Q does not depend on the lane's model.
//
// Gaussian range: the aim inverts the mixture table through a table of z at
// log-spaced distances of t from the nearer end of the range (so the tails,
// where G is flat in z, are resolved as finely as the bulk), takes the cell
// the aimed position mu + z sigma falls in, and evaluates G exactly at that
// cell's two edges, as the encoder does.  A cell that does not bracket t is
// moved one symbol towards it and checked again; what still misses is
// searched by the whole wave.  Floor-and-escape range: a bucket table of Q
// (built per call from the prefix) brackets s, and a per-lane binary search
// over the exact prefix finishes it.  The symbol found never depends on the
// aim, only the cost of finding it.
// ---------------------------------------------------------------------------
constexpr int kDecodeBlock = 1024;
constexpr int kDecodeBatch = 12;

// Aim table: z(d), the position at which the interpolated mixture table
// reaches d, is linear between the knots d_j = 2^(j >> 6) (1 + (j & 63) / 64);
// entry j holds the line's intercept and slope (z = c_j + k_j d on
// [d_j, d_{j+1})), so that the float32 bits of d give the entry (exponent
// and top mantissa bits) and one fused multiply-add gives z.  Distances
// stay below 2^31 (one entry at 2^31 takes float rounding).
constexpr int kAimMantBits = 6;
constexpr uint32_t kAimFracBits = 23 - kAimMantBits;
constexpr int kAimEntries = (31 << kAimMantBits) + 1;

__device__ __forceinline__ double table_inverse(const uint32_t* s_tab, double d) {
    uint32_t lo = 0, hi = kTablePoints;                 // largest k with H[k] <= d
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (static_cast<double>(s_tab[mid]) <= d) lo = mid;
        else hi = mid;
    }
    if (lo >= static_cast<uint32_t>(kTablePoints - 1)) return kTableZMax;
    const double fr = (d - s_tab[lo]) / static_cast<double>(s_tab[lo + 1] - s_tab[lo]);
    return (lo + fr) / 256.0 - kTableZMax;
}

__device__ __forceinline__ double aim_knot(int j) {
    return ldexp(1.0 + static_cast<double>(j & ((1 << kAimMantBits) - 1)) / (1 << kAimMantBits), j >> kAimMantBits);
}

__device__ __forceinline__ void build_aim_lds(float2* s_aim, const uint32_t* s_tab) {
    for (int j = threadIdx.x; j < kAimEntries; j += blockDim.x) {
        const double d0 = aim_knot(j), d1 = aim_knot(j + 1);
        const double z0 = table_inverse(s_tab, d0), z1 = table_inverse(s_tab, d1);
        const double k = (z1 - z0) / (d1 - d0);
        s_aim[j] = make_float2(static_cast<float>(z0 - k * d0), static_cast<float>(k));
    }
    __syncthreads();
}

static_assert(kTableEntries <= static_cast<int>(kTableWordsPadded) && kTableWordsPadded % 4 == 0, "table padding");
static_assert(2 * (kAimEntries + 1) == static_cast<int>(kAimFloats) && kAimFloats % 4 == 0, "aim table size");

// One workgroup: the mixture table for (tn, tw), padded with its last
// entry, and (when aim is given) the aim table built from it, plus one
// zero pair that pads it to 16 bytes.
__global__ void __launch_bounds__(1024) k_coder_tables(PhiTables phi, uint32_t tn, uint32_t tw,
                                                       uint32_t* __restrict__ table, float* __restrict__ aim) {
    __shared__ uint32_t s_tab[kTableEntries];
    __shared__ float2 s_aim[kAimEntries];
    build_table_lds(s_tab, phi, tn, tw);
    for (int k = threadIdx.x; k < static_cast<int>(kTableWordsPadded); k += blockDim.x)
        table[k] = s_tab[k < kTableEntries ? k : kTableEntries - 1];
    if (aim == nullptr) return;
    build_aim_lds(s_aim, s_tab);
    for (int k = threadIdx.x; k <= kAimEntries; k += blockDim.x) {
        aim[2 * k] = k < kAimEntries ? s_aim[k].x : 0.0f;
        aim[2 * k + 1] = k < kAimEntries ? s_aim[k].y : 0.0f;
    }
}

hipError_t launch_coder_tables(const PhiTables& phi, uint32_t tn, uint32_t tw, uint32_t* table, float* aim,
                               hipStream_t s) {
    hipLaunchKernelGGL(k_coder_tables, dim3(1), dim3(1024), 0, s, phi, tn, tw, table, aim);
    return hipGetLastError();
}

// z where the mixture table reaches t (t < htot), from the distance to the
// nearer end of the range; the upper half mirrors the lower one (the table
// is symmetric to within 2 units).
__device__ __forceinline__ float aim_z(uint32_t t, uint32_t htot, const float2* s_aim) {
    const uint32_t u = htot - t;
    const bool upper = u < t;
    // the distance to the nearer end, at least 1: the median of t, u and 1
    uint32_t d;
    __asm__("v_med3_u32 %0, %1, %2, 1" : "=v"(d) : "v"(t), "v"(u));
    const float df = static_cast<float>(d);
    // d >= 1: the exponent field starts at 127; the table is addressed from
    // a base biased by that many octaves (the LDS address wraps back)
    uint32_t j;
    __asm__("v_bfe_u32 %0, %1, %2, 15" : "=v"(j) : "v"(__float_as_uint(df)), "i"(kAimFracBits));
    const float2 e = (s_aim - (127u << kAimMantBits))[j];
    const float z = __fmaf_rn(df, e.y, e.x);
    return upper ? -z : z;
}

// A decoder candidate is held as a word whose upper half is the bf16
// pattern (the lower half is ignored) and, for e4m3, as the pattern itself.
// Nearest bf16 value to x, x clamped to [-max, max]: half a bf16 step added
// to the float32 bits (ties away from zero; the candidate only starts the
// search, so the tie rule does not matter), whose upper half is the pattern.
__device__ __forceinline__ uint32_t nearest_bf16(float x) {
    const float lim = __uint_as_float(0x7F7F0000u);
    const uint32_t u = __float_as_uint(__builtin_amdgcn_fmed3f(x, -lim, lim));
    return u + 0x8000u;
}

// e4m3fn pattern of the value nearest x, x clamped to [-448, 448]:
// subnormal steps of 2^-9 below 2^-6, three mantissa bits above.
__device__ __forceinline__ uint32_t nearest_e4m3(float x) {
    const float c = __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f);
    const uint32_t u = __float_as_uint(c);
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(__builtin_fabsf(c) * 512.0f));
    const uint32_t nrm = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    return (a < 0x3C800000u ? sub : nrm) | ((u >> 24) & 0x80u);
}

template <int KV>
__device__ __forceinline__ uint32_t nearest_candidate(float x) {
    if constexpr (KV == kBF16) return nearest_bf16(x);
    else return nearest_e4m3(x);
}

// Candidate of the ordered index s, and the bit pattern of a candidate.
template <int KV>
__device__ __forceinline__ uint32_t candidate_of_index(uint32_t s) {
    if constexpr (KV == kBF16) {
        // s >= 0x8000: pattern s ^ 0x8000; below: 0xFFFF - s = s ^ 0xFFFF
        const uint32_t below = ((s >> 15) & 1u) - 1u;
        return (s ^ 0x8000u ^ (below & 0x7FFFu)) << 16;
    } else {
        return bits_of_order<KV>(s);
    }
}

template <int KV>
__device__ __forceinline__ uint32_t candidate_bits(uint32_t cand) {
    if constexpr (KV == kBF16) return cand >> 16;
    else return cand;
}

// A candidate symbol with its exact CDF terms: G at both cell edges and
// the count of its floor-and-escape slots, Q(s + 1) - Q(s), where
// Q(b) = b + prefix[b].
struct Cell {
    uint32_t g0, g1, qf;
};

// Ordered index of a candidate (bf16: pattern in the upper half).
template <int KV>
__device__ __forceinline__ uint32_t index_of_candidate(uint32_t cand) {
    if constexpr (KV == kBF16) return order_of_bits<kBF16>(cand >> 16);
    else return order_of_bits<KV>(cand);
}

// Cell of the bf16 candidate kw (pattern in the upper half).  The outer edge (away from zero) is the
// pattern's magnitude plus half a step, the inner edge the magnitude minus
// half a step (0 for +-0).  With a bf16 mean the +-max cells may keep
// their finite outer edge (the mean lies at least half a step inside it, so
// z saturates at +-24 as for an infinite edge, sigma <= 2^96); with an fp32
// mean it becomes infinite, as the format defines.  Inf and NaN patterns
// reach here only from the escape lookup, and their G terms are replaced
// by the caller (every edge of theirs is infinite).  The escape slot count
// comes from the escape count table, at the pattern's entry.
template <int MU, class M>
__device__ __forceinline__ Cell eval_bf16(uint32_t kw, float mu, float inv24, const M& m) {
    const uint32_t sign = kw & 0x80000000u;
    uint32_t ob = (kw & 0xFFFF0000u) | 0x8000u;
    const uint32_t ib = __builtin_elementwise_max(__builtin_elementwise_sub_sat(ob, 0x10000u), sign);
    if constexpr (MU == kF32) ob = (kw & 0x7FFF0000u) == 0x7F7F0000u ? (sign | 0x7F800000u) : ob;
    const uint32_t ha = m.h(z_fixed(__uint_as_float(ib), mu, inv24));
    const uint32_t hb = m.h(z_fixed(__uint_as_float(ob), mu, inv24));
    Cell c;
    c.g0 = __builtin_elementwise_min(ha, hb);
    c.g1 = __builtin_elementwise_max(ha, hb);
    c.qf = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(m.ecount) + ((kw >> 14) & 0x3FFFCu));
    return c;
}

// Cell of the e4m3 pattern kb: edges and prefix from the LDS copies.
template <class M>
__device__ __forceinline__ Cell eval_e4m3(uint32_t kb, float mu, float inv24, const M& m) {
    Cell c;
    const uint32_t s = order_of_bits<kE4M3>(kb);
    c.g0 = m.h(z_fixed(e4_edge(m.small, s), mu, inv24));
    c.g1 = m.h(z_fixed(e4_edge(m.small, s + 1u), mu, inv24));
    c.qf = 1u + (m.small[s + 1u] - m.small[s]);
    return c;
}

template <int KV, int MU, class M>
__device__ __forceinline__ Cell eval_cell(uint32_t kb, float mu, float inv24, const M& m) {
    if constexpr (KV == kBF16) return eval_bf16<MU>(kb, mu, inv24, m);
    else return eval_e4m3(kb, mu, inv24, m);
}

// bf16 edge b (any b in 0..N) as a position: magnitude |b - 32768| * 2^16 -
// 2^15 (0 for the edge between -0 and +0), negative below b = 32768; at
// and beyond the outer edges of -max / +max the position is infinite for
// an fp32 mean; a bf16 mean may keep the finite outer edge (see eval_bf16),
// beyond which the pattern is pinned to Inf.
template <int MU>
__device__ __forceinline__ float edge_from_index_bf16(uint32_t b) {
    const uint32_t a = b >= 32768u ? b - 32768u : 32768u - b;
    uint32_t mag = __builtin_elementwise_sub_sat(a << 16, 0x8000u);    // a <= 32768
    if constexpr (MU == kBF16) mag = mag < 0x7F800000u ? mag : 0x7F800000u;
    else mag = mag < 0x7F7F8000u ? mag : 0x7F800000u;
    return __uint_as_float(mag | (b < 32768u ? 0x80000000u : 0u));
}

// G(b), the mixture-table term of the CDF at edge b, for the
// wave-cooperative search (bf16 edge from the index; e4m3 edge from LDS).
template <int KV, int MU, class M>
__device__ __forceinline__ uint32_t gauss_probe(uint32_t b, float mu, float inv24, const M& m) {
    if constexpr (KV == kBF16) return m.h(z_fixed(edge_from_index_bf16<MU>(b), mu, inv24));
    else return m.h(z_fixed(e4_edge(m.small, b), mu, inv24));
}

// Probe offsets for the first cooperative round: 1, 2, 3, ... then growing
// geometrically to 65535 over the 63 probing lanes.
__device__ __forceinline__ uint32_t geo_offset(int lane) {
    const float g = __builtin_amdgcn_exp2f(static_cast<float>(lane) * (16.0f / 62.0f));
    const uint32_t o = static_cast<uint32_t>(g);
    return o > static_cast<uint32_t>(lane + 1) ? o : static_cast<uint32_t>(lane + 1);
}

// Gaussian-range slot the aim did not bracket: the whole wave resolves
// every lane with `need` set, one lane at a time.  [lo, hi) brackets the
// lane's symbol with G(lo) = glo <= target < G(hi) = ghi; `up` tells which
// end is the known near one (lo if up).  Every lane probes with the
// searched lane's mean, scale and model (with a per-channel split, its
// budgets).  Returns s.
template <int KV, int MU, class M>
__device__ __forceinline__ uint32_t coop_gauss(bool need, uint32_t target, float mu, float inv24, bool up, uint32_t lo,
                                               uint32_t hi, uint32_t glo, uint32_t ghi, const M& m, uint32_t geo,
                                               uint32_t s_in) {
    const int lane = threadIdx.x & 63;
    uint32_t s_out = s_in;
    uint64_t pend = __ballot(need);
    while (pend) {
        const int L = __builtin_ctzll(pend);
        pend &= pend - 1;
        const uint32_t t = __builtin_amdgcn_readlane(target, L);
        const float mL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu), L));
        const float iL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv24), L));
        const bool upL = __builtin_amdgcn_readlane(static_cast<int>(up), L) != 0;
        const M mdl = m.of_lane(L);                      // lane L's budgets on every lane
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
            const uint32_t c = gauss_probe<KV, MU>(valid ? p : a, mL, iL, mdl);
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
        (void)ga;
        (void)gb;
        if (lane == L) s_out = a;
    }
    return s_out;
}

// Bucket table of the static part Q(b) = b + prefix[b] of the CDF: with
// s_j the largest s < N with Q(s) <= j * 2^shift, entry j holds, first,
// s_j in its high 16 bits and s_j's bit pattern in its low 16 (so entries
// order as their symbols, and an entry gives the decoder's candidate word
// of s_j at once), then Q(s_j).  A slot y in the floor-and-escape range has
// its symbol in [s_(y >> shift), s_((y >> shift) + 1)].  The shift is the
// smallest that keeps the table within kEscapeBucketsMax entries.

// Escape slot table: entry p of the bf16 pattern p, with s its ordered
// index, holds T_n + T_w + Q(s) and Q(s + 1) - Q(s), Q(b) = b + prefix[b];
// the escape count table holds Q(s + 1) - Q(s) alone.  Either output may be
// null.  One thread per pattern; the grid covers the 65536 patterns exactly.

// The symbol of escape offset y within [lo, hi]: binary search for the
// largest s with Q(s) = s + prefix[s] <= y (e4m3: the LDS prefix), with
// Q(lo) = qlo on entry; qlo leaves holding Q of the result.
template <int KV>
__device__ __forceinline__ uint32_t escape_symbol(uint32_t lo, uint32_t hi, uint32_t y, uint32_t& qlo, const Model& m) {
    while (__ballot(lo < hi)) {
        if (lo < hi) {
            const uint32_t mid = (lo + hi + 1u) >> 1;
            uint32_t qm;
            if constexpr (KV == kBF16) qm = mid + m.prefix[mid];
            else qm = mid + m.small[mid];
            if (qm <= y) {
                lo = mid;
                qlo = qm;
            } else {
                hi = mid - 1u;
            }
        }
    }
    return lo;
}

// Candidate word of the floor-and-escape slot y for every lane with `need`
// set, and q = Q(s) of its symbol s: the bucket table narrows the symbol to
// [lo, hi] and, when lo = hi, gives the candidate word and Q(s) at once; a
// per-lane binary search over Q(b) = b + prefix[b] finishes the rest.
// Indices stay in [0, N) whatever the prefix holds.
struct EscapeHit {
    uint32_t cand, q;
};
struct alignas(4) U32Quad {
    uint32_t a, b, c, d;
};

template <int KV>
__device__ __forceinline__ EscapeHit escape_candidate(bool need, uint32_t y, const uint32_t* base, uint32_t boff,
                                                      uint32_t shift, const Model& m) {
    // entries j and j + 1 (j <= the last bucket but one) in one read; a
    // lane without `need` keeps them equal.  Entries order as their symbols.
    // The table starts boff bytes after base; the sum stays in the vector
    // offset, so no second scalar base is kept for it.
    uint32_t e0 = 0, e1 = 0, q = 0;
    if (need) {
        uint32_t off = ((y >> shift) << 3) + boff;
        __asm__("" : "+v"(off));
        const U32Quad v = *reinterpret_cast<const U32Quad*>(reinterpret_cast<const char*>(base) + off);
        e0 = v.a;
        q = v.b;
        e1 = v.c;
    }
    if (__ballot(e0 < e1)) {
        // a bucket that starts within a run of symbols: search it
        const bool search = e0 < e1;
        const uint32_t s = escape_symbol<KV>(e0 >> 16, e1 >> 16, y, q, m);
        if (search) e0 = (s << 16) | candidate_bits<KV>(candidate_of_index<KV>(s));
    }
    if constexpr (KV == kBF16) return EscapeHit{e0 << 16, q};
    else return EscapeHit{e0 & 0xFFFFu, q};
}

// Stream words of a chunk, staged through a per-wave LDS ring of two
// 128-word blocks plus a copy of the first block after the second, so that
// the 128 words from any position of the ring on are contiguous.  The
// block after next is loaded into registers (one dword per lane) as soon as
// a block is entered and written to the ring when the one before it is
// left, so no global read sits on the serial decode chain.  A refill read
// is one LDS access at a wave-uniform base plus the lane's rank.
constexpr int kRingDwords = 192;
struct WordRing {
    __amdgpu_buffer_rsrc_t words;      // the chunk's word area (reads past its end give 0)
    uint32_t* ring;                    // this wave's kRingDwords dwords of LDS
    uint32_t base;                     // first word of the block being read
    uint32_t ahead;                    // this lane's dword of block base/128 + 2

    __device__ __forceinline__ uint32_t load(uint32_t block, uint32_t lane) const {
        // the whole offset in the vector operand, where the range check applies
        return __builtin_amdgcn_raw_buffer_load_b32(words, (block * 64u + lane) * 4u, 0, 0);
    }
    __device__ __forceinline__ void init(uint32_t lane) {
        base = 0;
        const uint32_t b0 = load(0, lane);
        ring[lane] = b0;
        ring[128u + lane] = b0;
        ring[64u + lane] = load(1, lane);
        ahead = load(2, lane);
    }
    // words p .. p + 127 start here (base <= p < base + 128; p wave-uniform)
    __device__ __forceinline__ const uint16_t* at(uint32_t p) const {
        return reinterpret_cast<const uint16_t*>(ring) + (p & 255u);
    }
    __device__ __forceinline__ void advance(uint32_t rp, uint32_t lane) {
        if (rp >= base + 128u) {                       // wave-uniform
            // the block just left (slot of base) takes the block after next
            if ((base >> 7) & 1u) {
                ring[64u + lane] = ahead;
            } else {
                ring[lane] = ahead;
                ring[128u + lane] = ahead;
            }
            base += 128u;
            ahead = load((base >> 7) + 2u, lane);
        }
    }
};

// Cache policy of the decoder's row stores (each row written once):
// non-temporal, decode 1.6% faster on the 8B-shaped cache.  The streamed
// reads keep the default policy: non-temporal reads gained nothing more
// there and made the decoder 9% slower on small calls whose inputs stay in
// the last-level cache, and non-temporal word-slot stores made the encoder
// 12% slower.
constexpr int kNonTemporal = 2;

constexpr uint32_t kPageWindow = 32;      // block-table entries a paged-decode wave keeps in LDS

// Store of one decoded row element: the row's byte address is wave-uniform
// (scalar registers) and the lane's byte offset a 32-bit vector register,
// widened next to the store so that the compiler selects the scalar-base
// form (no 64-bit address arithmetic per store).  A bf16 candidate word
// holds the pattern in its high half (a high-half 16-bit store).
// Non-temporal: each row is written once.  Plain stores rather than inline
// assembly, so that the compiler sees the address registers and covers them
// in its hazard handling.
template <int KV>
__device__ __forceinline__ void store_row(uint64_t row, uint32_t lane_off, uint32_t cand) {
    __asm__("" : "+v"(lane_off));
    using GChar = __attribute__((address_space(1))) char;
    GChar* p = reinterpret_cast<GChar*>(row) + lane_off;
    if constexpr (KV == kBF16) {
        using G16 = __attribute__((address_space(1))) uint16_t;
        __builtin_nontemporal_store(static_cast<uint16_t>(cand >> 16), reinterpret_cast<G16*>(p));
    } else {
        using G8 = __attribute__((address_space(1))) uint8_t;
        __builtin_nontemporal_store(static_cast<uint8_t>(cand), reinterpret_cast<G8*>(p));
    }
}

// SPLIT: every (plane, channel) has its own split of the Gaussian budget:
// the pair table in LDS instead of the mixture table, and the lane's own
// Newton steps after the call's aim (SplitModel::aim).
template <int KV, int MU, bool PAGED, bool SPLIT>
__global__ void __launch_bounds__(kDecodeBlock) __attribute__((amdgpu_num_sgpr(80))) k_decode(DecodeArgs a) {
    __shared__ __align__(16) uint32_t s_tab[SPLIT ? 2 * kTableWordsPadded : kTableWordsPadded];
    __shared__ __align__(16) float2 s_aim[kAimEntries + 1];
    __shared__ uint32_t s_ring[kDecodeBlock / 64][kRingDwords];
    __shared__ uint32_t s_small[KV == kE4M3 ? kE4Words : 1];
    __shared__ int32_t s_pages[PAGED ? kDecodeBlock / 64 : 1][PAGED ? kPageWindow : 1];
    if constexpr (KV == kE4M3) build_e4_lds(s_small, a.prefix);      // exact prefix + edges
    if constexpr (SPLIT) fill_pairs_lds(reinterpret_cast<uint2*>(s_tab), a.split.a, a.split.b);
    else copy_to_lds(s_tab, a.table, static_cast<uint32_t>(kTableBytes / 16));
    copy_to_lds(s_aim, a.aim, static_cast<uint32_t>(kAimBytes / 16));
    const uint32_t htot = a.tn + a.tw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * (kDecodeBlock / 64) + wave;
    if (chunk >= a.geom.n_chunks) return;
    // nothing is decoded when the stream's header is not the one the call
    // was set up with, a block-table entry is bad (paged output), or the
    // side information is not the encoder's (the same in every wave)
    if ((a.ctl->flags & (kFlagHeader | kFlagBadPage)) || a.ctl->side_hash != a.expect_hash) {
        if (chunk == 0 && lane == 0 && a.ctl->side_hash != a.expect_hash) atomicOr(&a.ctl->flags, kFlagMismatch);
        return;
    }
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
    WordRing win{buffer_rsrc(base + kStateBytes, avail * 2u), s_ring[wave], 0u, 0u};
    win.init(static_cast<uint32_t>(lane));

    const float sigma = a.sigma[cp.srow * D + cp.k * 64 + lane];
    float inv24 = __frcp_rn(sigma) * 16777216.0f;
    float sg = sigma;
    if (__ballot(!sigma_ok(sigma))) {
        if (lane == 0) atomicOr(&a.ctl->flags, kFlagBadSigma);
        inv24 = 16777216.0f;
        sg = 1.0f;
    }
    constexpr uint32_t kN = Alphabet<KV>::kSize;
    const Model plain{s_tab, a.prefix, s_small, nullptr, htot, a.ecount};
    // (a weight the encoder would refuse cannot pass the side-information
    // check; the capped budgets keep every lane's table within range)
    const auto m = [&]() {
        if constexpr (SPLIT) {
            const uint32_t w = a.split.words[cp.g * D + cp.k * 64 + lane];
            const uint32_t tn = split_narrow_budget(w, a.split.t_all, htot);
            return SplitModel{plain, tn, htot - tn};
        } else {
            return plain;
        }
    }();
    const uint32_t geo = geo_offset(lane);
    // bf16: the bucket table follows the escape count table (one base
    // address for both)
    const uint32_t* bucket_base = KV == kBF16 ? a.ecount : a.buckets;
    const uint32_t bucket_off = KV == kBF16 ? static_cast<uint32_t>(kEscapeCountBytes) : 0u;

    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    // this chunk's rows of mu and of the output as buffers: lane offset in a
    // vector register, row offset in a scalar one
    const int64_t row0 = (cp.g * a.geom.tokens + cp.t0) * static_cast<int64_t>(D) + cp.k * 64;
    const uint32_t rows_bytes = cp.len * D * static_cast<uint32_t>(sizeof(MT));
    const __amdgpu_buffer_rsrc_t mub = buffer_rsrc(static_cast<const MT*>(a.mu) + row0, rows_bytes);
    const __amdgpu_buffer_rsrc_t outb =
        buffer_rsrc(static_cast<KB*>(a.kv_out) + row0, cp.len * D * static_cast<uint32_t>(sizeof(KB)));
    const uint64_t out_base = reinterpret_cast<uint64_t>(static_cast<KB*>(a.kv_out) + row0);
    const uint32_t mu_lane = static_cast<uint32_t>(lane) * static_cast<uint32_t>(sizeof(MT));
    const uint32_t kv_lane = static_cast<uint32_t>(lane) * static_cast<uint32_t>(sizeof(KB));

    // paged output: page_row is the byte address of the current token's row
    // (this chunk's 64 channels of head h), a token further each step; at a
    // page boundary the next entry of the sequence's table row names the
    // page.  Every entry the call reads was checked before the launch
    // (by the prologue; the decode does nothing when one is bad).  The wave
    // stages kPageWindow entries of its table row at a time in LDS, so a
    // page boundary reads LDS rather than waiting on a global read (whose
    // wait would also cover the row stores in flight).  Reads of the pool
    // pointer and of table entries come back in vector registers and are
    // moved to scalar ones, where the stores take their base address.
    uint64_t page_row = 0, page_base = 0;
    const int32_t* page_entry = nullptr;                 // the window's first entry
    uint32_t page_left = 0, tok_bytes = 0, page_bytes = 0;
    uint32_t page_slot = 0;                              // the current page's entry in the window
    uint32_t cols_left = 0;                              // checked entries from page_entry on
    auto fill_window = [&]() {
        const uint32_t n = cols_left < kPageWindow ? cols_left : kPageWindow;
        if (static_cast<uint32_t>(lane) < n) s_pages[wave][lane] = page_entry[lane];
        __builtin_amdgcn_wave_barrier();
    };
    auto page_at = [&](uint32_t row) -> uint64_t {
        const uint32_t e = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(s_pages[wave][page_slot]));
        return page_base + uint64_t(e) * page_bytes + uint64_t(row) * tok_bytes;
    };
    if constexpr (PAGED) {
        const int64_t per_kv = int64_t(a.paged.batch) * a.paged.heads;
        const int64_t lk = cp.g / per_kv;                       // layer * 2 + kv
        const uint32_t bh = static_cast<uint32_t>(cp.g - lk * per_kv);
        const uint32_t b = bh / a.paged.heads, h = bh - b * a.paged.heads;
        const uint64_t pool = reinterpret_cast<uint64_t>(a.paged.pools[lk]);
        // (the builtin returns int: each half is taken as unsigned before widening)
        const uint32_t pool_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(pool)));
        const uint32_t pool_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(pool >> 32)));
        tok_bytes = a.paged.heads * D * static_cast<uint32_t>(sizeof(KB));      // below 2^32 (checked by the caller)
        page_bytes = a.paged.page_tokens * tok_bytes;
        page_base = ((uint64_t(pool_hi) << 32) | pool_lo) + (h * D + cp.k * 64u) * static_cast<uint32_t>(sizeof(KB));
        const uint32_t page_i = cp.t0 / a.paged.page_tokens;
        const uint32_t in_page = cp.t0 - page_i * a.paged.page_tokens;
        page_entry = a.paged.block_table + int64_t(b) * a.paged.max_pages + page_i;
        cols_left = static_cast<uint32_t>((a.geom.tokens + a.paged.page_tokens - 1) / a.paged.page_tokens) - page_i;
        fill_window();
        page_left = a.paged.page_tokens - in_page;
        page_row = page_at(in_page);
    }

    uint32_t rp = 0;
    unsigned long long misses = 0;                   // wave-uniform

    // predictor-mean rows as raw bits (the last row stands in for rows past
    // the chunk's end, which are not decoded; the buffer does not
    // range-check the row offset)
    using MRaw = typename std::conditional<MU == kBF16, uint16_t, uint32_t>::type;
    auto load_mu = [&](uint32_t t) -> MRaw {
        const uint32_t roff = (t < cp.len ? t : cp.len - 1) * D * static_cast<uint32_t>(sizeof(MT));
        if constexpr (MU == kBF16) return __builtin_amdgcn_raw_buffer_load_b16(mub, mu_lane, roff, 0);
        else return __builtin_amdgcn_raw_buffer_load_b32(mub, mu_lane, roff, 0);
    };
    auto mu_of = [](MRaw r) -> float {
        return MU == kBF16 ? __uint_as_float(static_cast<uint32_t>(r) << 16) : __uint_as_float(static_cast<uint32_t>(r));
    };
    MRaw nxt[kDecodeBatch];

    // One symbol of every lane: row t of the chunk, predictor mean mu.  The
    // first step of a batch loads the means of the next batch right after
    // its escape count table read: the vector memory counter is in order, so
    // this step's wait for that read does not include them and the next
    // step's does.
    auto step = [&](uint32_t t, float mu, bool first) {
        const uint32_t target = static_cast<uint32_t>(x) & (kM - 1u);
        // candidate: the cell the aim lands in, with its exact CDF terms
        float za = aim_z(target, htot, s_aim);
        if constexpr (SPLIT) za = m.aim(za, target);
        uint32_t kb = nearest_candidate<KV>(__fmaf_rn(za, sg, mu));
        const bool is_esc = target >= htot;
        const uint64_t esc = __ballot(is_esc);
        uint32_t qs = 0;                                 // Q(s) of an escape lane's symbol
        if (esc) {
            // floor-and-escape slots: the symbol comes from the lookup
            misses += __popcll(esc);
            const EscapeHit h = escape_candidate<KV>(is_esc, target - htot, bucket_base, bucket_off, a.bucket_shift, m);
            if (is_esc) kb = h.cand;
            qs = h.q;
        }
        Cell c = eval_cell<KV, MU>(kb, mu, inv24, m);
        if (first) {
            __asm__ volatile("" : : : "memory");
#pragma unroll
            for (int u = 0; u < kDecodeBatch; ++u) nxt[u] = load_mu(t + kDecodeBatch + u);
        }
        if (esc) {
            // a floor-and-escape slot has rank f_G(s) + (y - Q(s)): the
            // symbol's slots are taken to start at T_n + T_w + Q(s) - f_G(s)
            // (G terms of Inf and NaN, whose edges are all infinite, set first)
            if (is_esc) {
                __asm__ volatile("");                    // keep this a branch (rarely taken)
                if constexpr (KV == kBF16) {
                    const bool special = (kb & 0x7F800000u) == 0x7F800000u;    // Inf, NaN
                    if (__ballot(special)) {
                        __asm__ volatile("");            // a branch: Inf and NaN are rare
                        if (special) c.g0 = c.g1 = (kb & 0x80000000u) ? 0u : htot;
                    }
                }
                const uint32_t fg = c.g1 - c.g0;
                c.g1 = htot + qs;
                c.g0 = c.g1 - fg;
            }
        }
        // in the cell when target - G0 < G1 - G0 (unsigned: below G0 wraps)
        uint64_t need = __ballot(target - c.g0 >= c.g1 - c.g0) & ~esc;
        if (need) {
            // Gaussian slots outside the aimed cell: one symbol towards the
            // target first (G(0) = 0 <= target < G(N) = htot), then the
            // wave-cooperative search
            misses += __popcll(need);
            bool hit = ((need >> lane) & 1ull) == 0ull;
            if (!hit) {
                const uint32_t s0 = index_of_candidate<KV>(kb);
                kb = candidate_of_index<KV>(target < c.g0 ? s0 - 1u : s0 + 1u);
                c = eval_cell<KV, MU>(kb, mu, inv24, m);
                hit = target - c.g0 < c.g1 - c.g0;
            }
            need = __ballot(!hit);
            if (need) {
                const bool up = target >= c.g1;
                const uint32_t s1 = index_of_candidate<KV>(kb);
                const uint32_t sym = coop_gauss<KV, MU>(!hit, target, mu, inv24, up, up ? s1 + 1u : 0u,
                                                        up ? kN : s1, up ? c.g1 : 0u, up ? htot : c.g0, m, geo, s1);
                if (!hit) {
                    kb = candidate_of_index<KV>(sym);
                    c = eval_cell<KV, MU>(kb, mu, inv24, m);
                }
            }
        }
        // x = f (x >> 31) + rank, f = f_G + Q(s + 1) - Q(s); x < 2^63, so
        // x >> 31 fits 32 bits
        const uint32_t f = (c.g1 - c.g0) + c.qf;
        // the symbol is final: store it right after this step's wait for its
        // escape count table read (f is an input of the store only to hold it
        // there).
        // The vector memory counter is in order and counts stores: a store
        // issued before that wait would be waited for too, and one issued
        // in the next step would hold up the next wait.
        const uint32_t ooff = t * D * static_cast<uint32_t>(sizeof(KB));
        // f is a false input of the stored value, which holds the store there
        uint32_t kst = kb;
        __asm__ volatile("" : "+v"(kst) : "v"(f));
        if constexpr (PAGED) {
            store_row<KV>(page_row, kv_lane, kst);
            page_row += tok_bytes;
            if (--page_left == 0 && t + 1u < cp.len) {  // the next token starts a page
                if (++page_slot == kPageWindow) {        // (a checked entry follows the window)
                    page_entry += kPageWindow;
                    cols_left -= kPageWindow;
                    fill_window();
                    page_slot = 0;
                }
                page_left = a.paged.page_tokens;
                page_row = page_at(0);
            }
        } else if constexpr (KV == kBF16) {
            store_row<KV>(out_base + ooff, kv_lane, kst);
        } else {
            __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(kst), outb, kv_lane, ooff, kNonTemporal);
        }
        x = static_cast<unsigned long long>(f) * static_cast<uint32_t>(x >> kLog2M) + (target - c.g0);

        // refill: a lane takes one word when x < 2^47 and a second one when
        // it is still below 2^47 after that (x < 2^31 before); round one
        // holds one word per taking lane in lane order, round two the second
        // words
        uint32_t xh = static_cast<uint32_t>(x >> 32), xl = static_cast<uint32_t>(x);
        const bool take1 = xh < kLHi;
        const uint64_t m1 = __ballot(take1);
        const uint32_t w1 = win.at(rp)[lane_rank(m1)];
        const uint32_t sh = __builtin_amdgcn_alignbit(xh, xl, 16);
        xl = take1 ? (xl << 16) | w1 : xl;
        xh = take1 ? sh : xh;
        rp += __popcll(m1);
        const uint64_t m2 = __ballot(xh < kLHi);
        if (m2) {
            const bool take2 = xh < kLHi;
            const uint32_t w2 = win.at(rp)[lane_rank(m2)];
            const uint32_t sh2 = __builtin_amdgcn_alignbit(xh, xl, 16);
            xl = take2 ? (xl << 16) | w2 : xl;
            xh = take2 ? sh2 : xh;
            rp += __popcll(m2);
        }
        x = (static_cast<unsigned long long>(xh) << 32) | xl;
        win.advance(rp, static_cast<uint32_t>(lane));
    };

    // full batches: the means of the next batch are loaded while this one
    // decodes, so no HBM read sits on the serial chain; a non-finite mean
    // counts as 0
    const uint32_t full = cp.len - cp.len % kDecodeBatch;
#pragma unroll
    for (int u = 0; u < kDecodeBatch; ++u) nxt[u] = load_mu(u);
    for (uint32_t t0 = 0; t0 < full; t0 += kDecodeBatch) {
        float mus[kDecodeBatch];
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) mus[u] = mu_of(nxt[u]);
        uint64_t odd = 0;
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) odd |= __ballot(!__builtin_isfinite(mus[u]));
        if (odd) {
#pragma unroll
            for (int u = 0; u < kDecodeBatch; ++u) mus[u] = __builtin_isfinite(mus[u]) ? mus[u] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) step(t0 + u, mus[u], u == 0);
    }
    for (uint32_t t = full; t < cp.len; ++t) {
        const float mu = mu_of(load_mu(t));
        step(t, __builtin_isfinite(mu) ? mu : 0.0f, false);
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
    if (lane == 0 && misses) atomicAdd(&a.ctl->misses, misses);
}

// Every block-table entry a paged decode reads (rows 0..batch-1, columns
// 0..used-1) must name a page of the pool; one that does not sets the flag
// the decoder reads before its first store.

template <bool PAGED, bool SPLIT>
hipError_t launch_decode_as(const DecodeArgs& a, int kv_dtype, int mu_dtype, dim3 grid, dim3 block, hipStream_t s) {
    if (kv_dtype == kBF16 && mu_dtype == kBF16) hipLaunchKernelGGL((k_decode<kBF16, kBF16, PAGED, SPLIT>), grid, block, 0, s, a);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) hipLaunchKernelGGL((k_decode<kBF16, kF32, PAGED, SPLIT>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) hipLaunchKernelGGL((k_decode<kE4M3, kBF16, PAGED, SPLIT>), grid, block, 0, s, a);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) hipLaunchKernelGGL((k_decode<kE4M3, kF32, PAGED, SPLIT>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int mu_dtype, bool paged, hipStream_t s) {
    constexpr int waves = kDecodeBlock / 64;
    const uint64_t blocks = (static_cast<uint64_t>(a.geom.n_chunks) + waves - 1) / waves;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(kDecodeBlock);
    if (a.split.words != nullptr)
        return paged ? launch_decode_as<true, true>(a, kv_dtype, mu_dtype, grid, block, s)
                     : launch_decode_as<false, true>(a, kv_dtype, mu_dtype, grid, block, s);
    return paged ? launch_decode_as<true, false>(a, kv_dtype, mu_dtype, grid, block, s)
                 : launch_decode_as<false, false>(a, kv_dtype, mu_dtype, grid, block, s);
}

// ---------------------------------------------------------------------------
// sigma calibration: workgroups of 4 waves per (plane, sigma block, 64-channel
// group), each over a contiguous split of the block's reps x tokens rows;
// float64 sums in a fixed order, so the result does not depend on
// scheduling.  Non-finite residuals carry no scale information and are
// skipped.
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

// Pass 1: block (plane, sigma block and 64-channel group, split) sums the
// squared residuals of a contiguous range of the block's reps x tokens rows
// (rep-major; a sigma block of `block` tokens, the last one shorter).  Its 4 waves
// take every 4th row; each lane keeps one channel's float64 sum in row order
// and the waves are added in wave order, so the partial does not depend on
// scheduling.  Rows are loaded 4 at a time to keep loads in flight.
constexpr int kCalibBlock = 256;
constexpr int kCalibWaves = kCalibBlock / 64;
constexpr int kCalibUnroll = 4;

template <int KV, int MU>
__global__ void __launch_bounds__(kCalibBlock) k_calibrate_part(const void* kv_, const void* mu_, int64_t reps,
                                                                int64_t planes, int64_t tokens, int64_t channels,
                                                                int64_t block, int64_t nb,
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
    // (plane, sigma block) pair: the block's tokens [t_lo, t_lo + len)
    const int64_t vp = blockIdx.x / groups;
    const int64_t p = vp / nb;
    const int64_t t_lo = (vp - p * nb) * block;
    const int64_t len = tokens - t_lo < block ? tokens - t_lo : block;
    const int64_t d = (blockIdx.x % groups) * 64 + lane;
    const int64_t splits = gridDim.y, s = blockIdx.y;
    const int64_t rows = reps * len;
    const int64_t r1 = rows * (s + 1) / splits;
    int64_t r = rows * s / splits + wave;
    int64_t rep = r / len, t = r - rep * len;            // advanced by carries below
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
                const int64_t off = ((rep * planes + p) * tokens + t_lo + t) * channels + d;
                kb[u] = kv[off];
                mb[u] = mu[off];
            }
            r += kCalibWaves;
            t += kCalibWaves;
            while (t >= len) {
                t -= len;
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
        part[s * planes * nb * channels + vp * channels + d] = CalibPart{sum, u};
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

int64_t calibrate_splits(int64_t reps, int64_t pairs, int64_t block) {
    int64_t sp = (4096 + pairs - 1) / pairs;             // about 4096 blocks in all
    sp = sp < 1 ? 1 : (sp > kCalibSplitsMax ? kCalibSplitsMax : sp);
    const int64_t rows = reps * block;
    return sp > rows ? rows : sp;
}

hipError_t launch_calibrate(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps,
                            int64_t planes, int64_t tokens, int64_t channels, int64_t block_tokens,
                            float sigma_floor, float* sigma_out, CalibPart* part, hipStream_t s) {
    // block_tokens = 0 or >= tokens: one block of every token
    const int64_t blk = (block_tokens == 0 || block_tokens > tokens) ? tokens : block_tokens;
    const int64_t nb = (tokens + blk - 1) / blk;
    const int64_t pairs = planes * nb * (channels / 64);
    const int64_t splits = calibrate_splits(reps, pairs, blk);
    const dim3 grid(static_cast<uint32_t>(pairs), static_cast<uint32_t>(splits)), block(kCalibBlock);
    if (kv_dtype == kBF16 && mu_dtype == kBF16)
        hipLaunchKernelGGL((k_calibrate_part<kBF16, kBF16>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels,
                           blk, nb, part);
    else if (kv_dtype == kBF16 && mu_dtype == kF32)
        hipLaunchKernelGGL((k_calibrate_part<kBF16, kF32>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels,
                           blk, nb, part);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16)
        hipLaunchKernelGGL((k_calibrate_part<kE4M3, kBF16>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels,
                           blk, nb, part);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32)
        hipLaunchKernelGGL((k_calibrate_part<kE4M3, kF32>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels,
                           blk, nb, part);
    else return hipErrorInvalidValue;
    const int64_t n = planes * nb * channels;
    hipLaunchKernelGGL(k_calibrate_final, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s, part, splits,
                       n, sigma_floor, sigma_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// rate-fitted sigma: for each candidate sigma_j = max(floor, base * (1 - j/32)),
// the integer code length of the held-out data under the coder's own CDF,
// sum of 2^16 (31 - e) - LOG2[m] over f = C(s+1) - C(s) (e the top bit of f,
// m the 8 bits below it); the least sum wins, the first j on a tie.  Sums of
// integers: the result does not depend on the order of summation.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t code_len_q16(uint32_t f, const uint32_t* log2_tab) {
    const uint32_t lz = __builtin_clz(f);                    // f >= 1: 31 - top bit
    const uint32_t m = ((f << lz) >> 23) & 0xFFu;
    return lz * 65536u - log2_tab[m];
}

template <int KV, int MU>
__global__ void __launch_bounds__(kCalibBlock) k_rate_cost(const void* kv_, const void* mu_, int64_t reps,
                                                           int64_t planes, int64_t tokens, int64_t channels,
                                                           int64_t block, int64_t nb, const float* __restrict__ base,
                                                           float sigma_floor, const uint32_t* __restrict__ table,
                                                           const uint32_t* __restrict__ prefix,
                                                           unsigned long long* __restrict__ part) {
    __shared__ __align__(16) uint32_t s_tab[kTableWordsPadded];
    __shared__ uint32_t s_log[256];
    __shared__ unsigned long long s_sum[kCalibWaves][64];
    for (uint32_t i = threadIdx.x; i < 256u; i += blockDim.x)
        s_log[i] = static_cast<uint32_t>(floor(65536.0 * log2(1.0 + i / 256.0) + 0.5));
    copy_to_lds(s_tab, table, static_cast<uint32_t>(kTableBytes / 16));     // and the barrier
    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    const KB* __restrict__ kv = static_cast<const KB*>(kv_);
    const MT* __restrict__ mu = static_cast<const MT*>(mu_);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t groups = channels / 64;
    const int64_t vp = blockIdx.x / groups;                   // (plane, sigma block) pair
    const int64_t p = vp / nb;
    const int64_t t_lo = (vp - p * nb) * block;
    const int64_t len = tokens - t_lo < block ? tokens - t_lo : block;
    const int64_t d = (blockIdx.x % groups) * 64 + lane;
    const int64_t splits = gridDim.y, s = blockIdx.y;
    const uint32_t j = blockIdx.z;
    const int64_t n = planes * nb * channels;
    // the candidate: 1 - j/32 is exact in float32
    const float k = static_cast<float>(32u - j) * 0.03125f;
    const float sg = fmaxf(__fmul_rn(base[vp * channels + d], k), sigma_floor);
    const float inv24 = __frcp_rn(sg) * 16777216.0f;
    const Model m{s_tab, prefix, nullptr};
    const int64_t rows = reps * len;
    const int64_t r1 = rows * (s + 1) / splits;
    unsigned long long acc = 0;
    for (int64_t r = rows * s / splits + wave; r < r1; r += kCalibWaves) {
        const int64_t rep = r / len, t = r - rep * len;
        const int64_t off = ((rep * planes + p) * tokens + t_lo + t) * channels + d;
        const uint32_t sym = order_of_bits<KV>(kv[off]);
        const float mv = mu_value<MU>(mu[off]);
        const uint32_t f = cdf_at<KV>(sym + 1u, mv, inv24, m) - cdf_at<KV>(sym, mv, inv24, m);
        acc += code_len_q16(f, s_log);
    }
    s_sum[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        unsigned long long t = 0;
        for (int w = 0; w < kCalibWaves; ++w) t += s_sum[w][lane];
        part[(static_cast<int64_t>(j) * splits + s) * n + vp * channels + d] = t;
    }
}

// One thread per (plane, sigma block, channel): the candidate with the least
// code length; sigma_io holds the base on entry and the fitted sigma after.
__global__ void k_rate_pick(const unsigned long long* __restrict__ part, int64_t splits, int64_t n, float sigma_floor,
                            float* __restrict__ sigma_io) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    unsigned long long best = ~0ull;
    uint32_t best_j = 0;
    for (uint32_t j = 0; j < static_cast<uint32_t>(kRateSteps); ++j) {
        unsigned long long c = 0;
        for (int64_t s = 0; s < splits; ++s) c += part[(static_cast<int64_t>(j) * splits + s) * n + i];
        if (c < best) {
            best = c;
            best_j = j;
        }
    }
    const float k = static_cast<float>(32u - best_j) * 0.03125f;
    sigma_io[i] = fmaxf(__fmul_rn(sigma_io[i], k), sigma_floor);
}

hipError_t launch_rate_fit(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps, int64_t planes,
                           int64_t tokens, int64_t channels, int64_t block_tokens, float sigma_floor,
                           const uint32_t* table, const uint32_t* prefix, float* sigma_io, unsigned long long* part,
                           hipStream_t s) {
    const int64_t blk = (block_tokens == 0 || block_tokens > tokens) ? tokens : block_tokens;
    const int64_t nb = (tokens + blk - 1) / blk;
    const int64_t pairs = planes * nb * (channels / 64);
    const int64_t splits = calibrate_splits(reps, pairs, blk);
    const dim3 grid(static_cast<uint32_t>(pairs), static_cast<uint32_t>(splits), kRateSteps), block(kCalibBlock);
#define KVC_RATE(K, U)                                                                                          \
    hipLaunchKernelGGL((k_rate_cost<K, U>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels, blk, nb, \
                       sigma_io, sigma_floor, table, prefix, part)
    if (kv_dtype == kBF16 && mu_dtype == kBF16) KVC_RATE(kBF16, kBF16);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) KVC_RATE(kBF16, kF32);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) KVC_RATE(kE4M3, kBF16);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) KVC_RATE(kE4M3, kF32);
    else return hipErrorInvalidValue;
#undef KVC_RATE
    const int64_t n = planes * nb * channels;
    hipLaunchKernelGGL(k_rate_pick, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s, part, splits, n,
                       sigma_floor, sigma_io);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// per-channel split: for each candidate narrow weight w_j = max(W - 200 j,
// 0), W = w_n + w_w, j < kSplitSteps, the integer code length of the
// held-out data with every lane's budgets split by w_j (the same sum as
// the rate-fitted sigma); the least sum wins, the first j on a tie.  One
// workgroup per (plane, 64-channel group) and split of the rows evaluates
// every candidate: the two cell edges' table entries are read once per
// scalar and combined with each candidate's budgets.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t split_candidate(uint32_t j, uint32_t w_gauss) {
    const uint32_t d = static_cast<uint32_t>(kSplitStepBp) * j;
    return w_gauss > d ? w_gauss - d : 0u;
}

// The lane table's interpolated value from its two pair-table entries (u:
// the table position, its 16 low bits the interpolation weight).
__device__ __forceinline__ uint32_t interp_pairs(uint2 p0, uint2 p1, uint32_t u, uint32_t tn, uint32_t tw) {
    const uint32_t a = mul_shr31(tn, p0.x) + mul_shr31(tw, p0.y);
    const uint32_t c = mul_shr31(tn, p1.x) + mul_shr31(tw, p1.y);
    return a + interp_step(c - a, u);
}

template <int KV, int MU>
__global__ void __launch_bounds__(kCalibBlock) k_split_cost(const void* kv_, const void* mu_, int64_t reps,
                                                            int64_t planes, int64_t tokens, int64_t channels,
                                                            int64_t blk, int64_t nb, const float* __restrict__ sigma,
                                                            SplitArgs sp, uint32_t htot,
                                                            const uint32_t* __restrict__ prefix,
                                                            unsigned long long* __restrict__ part) {
    __shared__ __align__(16) uint2 s_ab[kTableWordsPadded];
    __shared__ uint32_t s_log[256];
    __shared__ unsigned long long s_sum[kCalibWaves][64];
    for (uint32_t i = threadIdx.x; i < 256u; i += blockDim.x)
        s_log[i] = static_cast<uint32_t>(floor(65536.0 * log2(1.0 + i / 256.0) + 0.5));
    fill_pairs_lds(s_ab, sp.a, sp.b);                            // and the barrier
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
    const int64_t n = planes * channels;
    uint32_t tn[kSplitSteps];
#pragma unroll
    for (int j = 0; j < kSplitSteps; ++j) tn[j] = split_narrow_budget(split_candidate(j, sp.w_gauss), sp.t_all, htot);
    unsigned long long acc[kSplitSteps];
#pragma unroll
    for (int j = 0; j < kSplitSteps; ++j) acc[j] = 0;
    const int64_t rows = reps * tokens;
    const int64_t r1 = rows * (s + 1) / splits;
    for (int64_t r = rows * s / splits + wave; r < r1; r += kCalibWaves) {
        const int64_t rep = r / tokens, t = r - rep * tokens;
        const int64_t off = ((rep * planes + p) * tokens + t) * channels + d;
        const uint32_t sym = order_of_bits<KV>(kv[off]);
        const float mv = mu_value<MU>(mu[off]);
        const float inv24 = __frcp_rn(sigma[(p * nb + t / blk) * channels + d]) * 16777216.0f;
        const uint32_t u0 = static_cast<uint32_t>(z_fixed(edge<KV>(sym), mv, inv24) + kQMax);
        const uint32_t u1 = static_cast<uint32_t>(z_fixed(edge<KV>(sym + 1u), mv, inv24) + kQMax);
        const uint2 a0 = s_ab[u0 >> 16], a1 = s_ab[(u0 >> 16) + 1];
        const uint2 b0 = s_ab[u1 >> 16], b1 = s_ab[(u1 >> 16) + 1];
        const uint32_t qf = 1u + prefix[sym + 1u] - prefix[sym];
#pragma unroll
        for (int j = 0; j < kSplitSteps; ++j) {
            const uint32_t h0 = interp_pairs(a0, a1, u0, tn[j], htot - tn[j]);
            const uint32_t h1 = interp_pairs(b0, b1, u1, tn[j], htot - tn[j]);
            acc[j] += code_len_q16(h1 - h0 + qf, s_log);
        }
    }
#pragma unroll
    for (int j = 0; j < kSplitSteps; ++j) {
        s_sum[wave][lane] = acc[j];
        __syncthreads();
        if (wave == 0) {
            unsigned long long t = 0;
            for (int w = 0; w < kCalibWaves; ++w) t += s_sum[w][lane];
            part[(static_cast<int64_t>(j) * splits + s) * n + p * channels + d] = t;
        }
        __syncthreads();
    }
}

// One thread per (plane, channel): the candidate with the least code length.
__global__ void k_split_pick(const unsigned long long* __restrict__ part, int64_t splits, int64_t n, uint32_t w_gauss,
                             uint32_t* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    unsigned long long best = ~0ull;
    uint32_t best_j = 0;
    for (uint32_t j = 0; j < static_cast<uint32_t>(kSplitSteps); ++j) {
        unsigned long long c = 0;
        for (int64_t s = 0; s < splits; ++s) c += part[(static_cast<int64_t>(j) * splits + s) * n + i];
        if (c < best) {
            best = c;
            best_j = j;
        }
    }
    out[i] = split_candidate(best_j, w_gauss);
}

hipError_t launch_split_fit(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps, int64_t planes,
                            int64_t tokens, int64_t channels, int64_t block_tokens, const float* sigma,
                            const SplitArgs& sp, uint32_t htot, const uint32_t* prefix, uint32_t* out,
                            unsigned long long* part, hipStream_t s) {
    const int64_t blk = (block_tokens == 0 || block_tokens > tokens) ? tokens : block_tokens;
    const int64_t nb = (tokens + blk - 1) / blk;
    const int64_t pairs = planes * (channels / 64);
    const int64_t splits = calibrate_splits(reps, pairs, tokens);
    const dim3 grid(static_cast<uint32_t>(pairs), static_cast<uint32_t>(splits)), block(kCalibBlock);
#define KVC_SPLIT(K, U)                                                                                       \
    hipLaunchKernelGGL((k_split_cost<K, U>), grid, block, 0, s, kv, mu, reps, planes, tokens, channels, blk, nb, \
                       sigma, sp, htot, prefix, part)
    if (kv_dtype == kBF16 && mu_dtype == kBF16) KVC_SPLIT(kBF16, kBF16);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) KVC_SPLIT(kBF16, kF32);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) KVC_SPLIT(kE4M3, kBF16);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) KVC_SPLIT(kE4M3, kF32);
    else return hipErrorInvalidValue;
#undef KVC_SPLIT
    const int64_t n = planes * channels;
    hipLaunchKernelGGL(k_split_pick, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s, part, splits, n,
                       sp.w_gauss, out);
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

// F(b) - F(a) for the Student-t narrow part, truncated to [-24, 24] and
// renormalised (as its table is), a <= b.
__device__ __forceinline__ double t_mass(double a, double b, int nu) {
    a = fmax(a, -static_cast<double>(kTableZMax));
    b = fmin(b, static_cast<double>(kTableZMax));
    if (!(a < b)) return 0.0;
    const double span = 1.0 - 2.0 * student_t_cdf(-static_cast<double>(kTableZMax), nu);
    const double m = a > 0.0 ? student_t_cdf(-a, nu) - student_t_cdf(-b, nu) : student_t_cdf(b, nu) - student_t_cdf(a, nu);
    return m / span;
}

// SPLIT: each (plane, channel) with its own split of the Gaussian weight
// (budgets from the pair table; the float model's weights w_c and
// w_n + w_w - w_c).
template <int KV, int MU, bool SPLIT>
__global__ void __launch_bounds__(256) k_estimate(EstimateArgs a) {
    __shared__ __align__(16) uint32_t s_tab[SPLIT ? 2 * kTableWordsPadded : kTableEntries];
    __shared__ double s_red[2][4];
    if constexpr (SPLIT) fill_pairs_lds(reinterpret_cast<uint2*>(s_tab), a.split.a, a.split.b);
    else build_table_lds(s_tab, a.phi, a.tn, a.tw);
    using KB = typename Alphabet<KV>::Bits;
    using MT = typename MuT<MU>::T;
    const KB* __restrict__ kv = static_cast<const KB*>(a.kv);
    const MT* __restrict__ mup = static_cast<const MT*>(a.mu);
    const Model base{s_tab, a.prefix, nullptr, nullptr, a.tn + a.tw};
    const int64_t D = a.geom.channels, T = a.geom.tokens;
    const int64_t n = a.geom.planes * T * D;
    double wn = a.w_narrow_bp / 1e4, ww = a.w_wide_bp / 1e4;
    const double we = 1.0 - wn - ww;
    double acc_i = 0.0, acc_f = 0.0;
    bool bad = false;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t d = i % D;
        const int64_t g = i / (T * D);
        const int64_t tc = (i / D - g * T) / a.geom.chunk_tokens;
        const float sg = a.sigma[(g * a.geom.sigma_blocks + (a.geom.sigma_tc ? tc / a.geom.sigma_tc : 0)) * D + d];
        const float inv24 = __frcp_rn(sg) * 16777216.0f;
        const float mu = mu_value<MU>(mup[i]);
        const uint32_t s = order_of_bits<KV>(kv[i]);
        const auto model = [&]() {
            if constexpr (SPLIT) {
                const uint32_t w = a.split.words[g * D + d];
                bad |= w > a.split.w_gauss;
                wn = w / 1e4;
                ww = a.split.w_gauss / 1e4 - wn;
                const uint32_t tn = split_narrow_budget(w, a.split.t_all, base.htot);
                return SplitModel{base, tn, base.htot - tn};
            } else {
                return base;
            }
        }();
        const uint32_t c0 = cdf_at<KV>(s, mu, inv24, model);
        const uint32_t c1 = cdf_at<KV>(s + 1, mu, inv24, model);
        acc_i += 31.0 - log2(static_cast<double>(c1 - c0));
        const double lo = edge<KV>(s), hi = edge<KV>(s + 1);
        const double m = mu, sd = sg;
        const double narrow = a.narrow_dof ? t_mass((lo - m) / sd, (hi - m) / sd, static_cast<int>(a.narrow_dof))
                                           : gauss_mass((lo - m) / sd, (hi - m) / sd);
        double q = wn * narrow + ww * gauss_mass((lo - m) / (3.0 * sd), (hi - m) / (3.0 * sd));
        if (a.te) q += we * static_cast<double>(a.prefix[s + 1] - a.prefix[s]) / a.te;
        const double b = -log2(q);
        acc_f += (b < 64.0) ? b : 64.0;
    }
    acc_i = wave_sum_f64(acc_i);
    acc_f = wave_sum_f64(acc_f);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (__ballot(bad) && lane == 0) atomicOr(&a.ctl->flags, kFlagBadSigma);
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
    const bool sp = a.split.words != nullptr;
#define KVC_EST(K, U)                                                                  \
    do {                                                                               \
        if (sp) hipLaunchKernelGGL((k_estimate<K, U, true>), grid, block, 0, s, a);    \
        else hipLaunchKernelGGL((k_estimate<K, U, false>), grid, block, 0, s, a);      \
    } while (0)
    if (kv_dtype == kBF16 && mu_dtype == kBF16) KVC_EST(kBF16, kBF16);
    else if (kv_dtype == kBF16 && mu_dtype == kF32) KVC_EST(kBF16, kF32);
    else if (kv_dtype == kE4M3 && mu_dtype == kBF16) KVC_EST(kE4M3, kBF16);
    else if (kv_dtype == kE4M3 && mu_dtype == kF32) KVC_EST(kE4M3, kF32);
    else return hipErrorInvalidValue;
#undef KVC_EST
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
    const Model model{s_tab, prefix, nullptr};
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

namespace kvc {

// ---------------------------------------------------------------------------
// Per-device cache of the coder tables: the mixture table and the decoder's
// aim table depend only on the budgets (T_n, T_w) and the narrow part, not
// on the data, so each combination a process uses is built once per device
// (a kernel and a synchronisation of the calling stream, on first use) and
// only read afterwards.  A call whose combination finds no free slot builds
// its tables in its own workspace as before.
// ---------------------------------------------------------------------------
constexpr int kTabCacheSlots = 8;
__device__ __align__(16) uint32_t g_tab_cache[kTabCacheSlots][kTableWordsPadded];
__device__ __align__(16) float g_aim_cache[kTabCacheSlots][kAimFloats];

namespace {
struct TabKey {
    uint32_t tn, tw, dof;
    bool used;
};
std::mutex g_tab_mutex;
TabKey g_tab_keys[kMaxDevices][kTabCacheSlots];
uint32_t* g_tab_dev[kMaxDevices];
float* g_aim_dev[kMaxDevices];
}  // namespace

bool cached_coder_tables(uint32_t tn, uint32_t tw, uint32_t narrow_dof, const PhiTables& phi, hipStream_t s,
                         const uint32_t** table, const float** aim, hipError_t* err) {
    *err = hipSuccess;
    int dev = 0;
    if ((*err = hipGetDevice(&dev)) != hipSuccess) return false;
    if (dev < 0 || dev >= kMaxDevices) return false;
    std::lock_guard<std::mutex> lock(g_tab_mutex);
    if (!g_tab_dev[dev]) {
        void* pt = nullptr;
        void* pa = nullptr;
        if ((*err = hipGetSymbolAddress(&pt, HIP_SYMBOL(g_tab_cache))) != hipSuccess) return false;
        if ((*err = hipGetSymbolAddress(&pa, HIP_SYMBOL(g_aim_cache))) != hipSuccess) return false;
        g_tab_dev[dev] = static_cast<uint32_t*>(pt);
        g_aim_dev[dev] = static_cast<float*>(pa);
    }
    int slot = -1;
    for (int i = 0; i < kTabCacheSlots && slot < 0; ++i) {
        const TabKey& k = g_tab_keys[dev][i];
        if (k.used && k.tn == tn && k.tw == tw && k.dof == narrow_dof) slot = i;
    }
    if (slot < 0) {
        for (int i = 0; i < kTabCacheSlots && slot < 0; ++i)
            if (!g_tab_keys[dev][i].used) slot = i;
        if (slot < 0) return false;                    // full: the caller builds its own
        uint32_t* t = g_tab_dev[dev] + static_cast<size_t>(slot) * kTableWordsPadded;
        float* a = g_aim_dev[dev] + static_cast<size_t>(slot) * kAimFloats;
        if ((*err = launch_coder_tables(phi, tn, tw, t, a, s)) != hipSuccess) return false;
        if ((*err = hipStreamSynchronize(s)) != hipSuccess) return false;
        g_tab_keys[dev][slot] = TabKey{tn, tw, narrow_dof, true};
    }
    *table = g_tab_dev[dev] + static_cast<size_t>(slot) * kTableWordsPadded;
    *aim = g_aim_dev[dev] + static_cast<size_t>(slot) * kAimFloats;
    return true;
}

// ---------------------------------------------------------------------------
// Per-call preparation in one launch: workgroups take one role each by
// index range — the side-information checksum (with the decoder's header
// comparison), the bf16 escape slot or count table, the escape bucket
// table, the reset of the encoder's look-back entries, and the check of a
// paged decode's block table.  The control block was cleared by the launch
// before.
// ---------------------------------------------------------------------------
template <int KV>
__global__ void __launch_bounds__(256) k_prologue(PrologueArgs a) {
    uint32_t b = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    if (b < a.hash_blocks) {
        if (a.head != nullptr && b == 0 && tid < kHeaderBytes / 8) {
            unsigned long long w, e;
            __builtin_memcpy(&w, a.head + 8 * tid, 8);
            __builtin_memcpy(&e, a.expect.bytes + 8 * tid, 8);
            if (w != e) atomicOr(&a.ctl->flags, kFlagHeader);
        }
        __shared__ unsigned long long s_part[4];
        const unsigned long long golden = 0x9E3779B97F4A7C15ull;
        const uint64_t n1 = a.n_sigma, n = a.n_sigma + a.n_prefix;
        const uint64_t stride = static_cast<uint64_t>(a.hash_blocks) * 256u;
        unsigned long long acc = 0;
        for (uint64_t j = static_cast<uint64_t>(b) * 256u + tid; j < n; j += stride) {
            unsigned long long i, w, tag;
            if (j < n1) { i = j; w = a.sigma_words[j]; tag = 1; }
            else { i = j - n1; w = a.prefix_words[j - n1]; tag = 2; }
            acc += mix64(((i << 32) | w) + tag * golden);
        }
        acc = wave_sum_u64(acc);
        if ((tid & 63u) == 0) s_part[tid >> 6] = acc;
        __syncthreads();
        if (tid == 0) {
            const unsigned long long sum = s_part[0] + s_part[1] + s_part[2] + s_part[3];
            if (sum) atomicAdd(&a.ctl->side_hash, sum);
        }
        return;
    }
    b -= a.hash_blocks;
    if (b < a.slot_blocks) {
        // one thread per bf16 pattern p, s its ordered index
        const uint32_t p = b * 256u + tid;
        const uint32_t s = order_of_bits<kBF16>(p);
        const uint32_t p0 = a.prefix[s], p1 = a.prefix[s + 1u];
        if (a.eslots) a.eslots[p] = make_uint2(a.htot + s + p0, 1u + (p1 - p0));
        if (a.ecount) a.ecount[p] = 1u + (p1 - p0);
        return;
    }
    b -= a.slot_blocks;
    if (b < a.bucket_blocks) {
        const uint32_t j = b * 256u + tid;
        if (j >= a.n_buckets) return;
        const unsigned long long y = static_cast<unsigned long long>(j) << a.bucket_shift;
        uint32_t lo = 0, hi = a.n_sym - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1u) >> 1;
            if (static_cast<unsigned long long>(mid) + a.prefix[mid] <= y) lo = mid;
            else hi = mid - 1u;
        }
        a.buckets[j] = make_uint2((lo << 16) | candidate_bits<KV>(candidate_of_index<KV>(lo)), lo + a.prefix[lo]);
        return;
    }
    b -= a.bucket_blocks;
    if (b < a.zero_blocks) {
        const uint64_t stride = static_cast<uint64_t>(a.zero_blocks) * 256u;
        for (uint64_t i = static_cast<uint64_t>(b) * 256u + tid; i < a.n_zero; i += stride) a.zero[i] = 0ull;
        return;
    }
    b -= a.zero_blocks;
    if (b < a.page_blocks) {
        const int64_t i = static_cast<int64_t>(b) * 256 + tid;
        if (i >= a.pages.batch * a.pages_used) return;
        const int32_t e = a.pages.block_table[(i / a.pages_used) * a.pages.max_pages + i % a.pages_used];
        if (e < 0 || int64_t(e) >= a.pages.num_pages) atomicOr(&a.ctl->flags, kFlagBadPage);
    }
}

hipError_t launch_prologue(PrologueArgs a, int kv_dtype, hipStream_t s) {
    const uint64_t n = a.n_sigma + a.n_prefix;
    uint64_t hb = (n + 255) / 256;
    a.hash_blocks = static_cast<uint32_t>(hb < 1 ? 1 : (hb > 64 ? 64 : hb));
    a.slot_blocks = (a.eslots || a.ecount) ? 65536u / 256u : 0u;
    a.bucket_blocks = a.buckets ? (a.n_buckets + 255u) / 256u : 0u;
    uint64_t zb = (a.n_zero + 255) / 256;
    a.zero_blocks = a.zero ? static_cast<uint32_t>(zb < 1 ? 1 : (zb > 1024 ? 1024 : zb)) : 0u;
    const int64_t np = a.pages.block_table ? int64_t(a.pages.batch) * a.pages_used : 0;
    a.page_blocks = static_cast<uint32_t>((np + 255) / 256);
    const uint32_t blocks = a.hash_blocks + a.slot_blocks + a.bucket_blocks + a.zero_blocks + a.page_blocks;
    if (kv_dtype == kBF16) hipLaunchKernelGGL(k_prologue<kBF16>, dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_prologue<kE4M3>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvc
