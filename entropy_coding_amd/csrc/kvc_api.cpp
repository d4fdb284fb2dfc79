// C ABI of libkvc (declared in include/kvc.h): argument validation, stream
// header and directory bookkeeping, workspace layout, kernel launches and
// the single status read-back per call.  Every step of the coder itself
// runs in the kernels of kvc_kernels.hip.
#include "kvc.h"

#include <hip/hip_runtime_api.h>

#include <cfloat>
#include <cstring>

#include "kvc_internal.hpp"

namespace {

using kvc::ChunkGeom;
using kvc::Control;

constexpr uint32_t kLog2M = 31;
constexpr uint32_t kLog2L = 47;
constexpr uint32_t kWordBits = 16;
constexpr uint32_t kLanes = 64;
constexpr uint32_t kVersion = 4;   // stream format version (split slot ranges, floor of z * 2^24, header CRC)
constexpr uint32_t kMaxChunkTokens = 1u << 20;
constexpr int64_t kMaxScalars = int64_t(1) << 40;
// decode workspace: control block, the escape count table, the escape
// bucket table (two u32 per entry; right after the count table, where the
// bf16 decoder expects it), the mixture table and the aim table
constexpr uint64_t kDecodeCountOffset = 256;
constexpr uint64_t kDecodeBucketOffset = kDecodeCountOffset + kvc::kEscapeCountBytes;
constexpr uint64_t kDecodeTableOffset = 786944;
constexpr uint64_t kDecodeAimOffset = kDecodeTableOffset + 49408;
static_assert(kDecodeBucketOffset + 8 * kvc::kEscapeBucketsMax <= kDecodeTableOffset &&
                  kDecodeTableOffset % 256 == 0 && kDecodeTableOffset + kvc::kTableBytes <= kDecodeAimOffset &&
                  kDecodeAimOffset + kvc::kAimBytes <= KVC_DECODE_WORKSPACE_BYTES,
              "decode workspace layout");

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

bool kv_dtype_ok(int32_t t) { return t == KVC_BF16 || t == KVC_E4M3; }
bool mu_dtype_ok(int32_t t) { return t == KVC_BF16 || t == KVC_F32; }

uint32_t alphabet(int32_t kv) { return kv == KVC_BF16 ? 65536u : 256u; }

bool budgets(int32_t kv, uint32_t wn, uint32_t ww, uint32_t* tn, uint32_t* tw, uint32_t* te) {
    if (!kv_dtype_ok(kv) || wn > 10000u || ww > 10000u || wn + ww > 10000u) return false;
    const uint64_t t = (uint64_t(1) << kLog2M) - alphabet(kv);
    *tn = static_cast<uint32_t>(t * wn / 10000u);
    *tw = static_cast<uint32_t>(t * ww / 10000u);
    *te = static_cast<uint32_t>(t - *tn - *tw);
    return true;
}

// Shape rules shared by encoder and decoder.  sigma_block_tokens: 0 (one
// sigma per plane and channel) or B, one sigma per block of B tokens; a
// chunk must lie within one block, so B is a multiple of the chunk length
// unless one block covers every token.
bool geometry(int64_t planes, int64_t tokens, int64_t channels, uint32_t chunk_tokens, uint32_t sigma_block_tokens,
              ChunkGeom* g) {
    if (planes < 1 || tokens < 1 || channels < 64 || channels % 64) return false;
    if (planes > kMaxScalars || tokens > kMaxScalars || channels > kMaxScalars) return false;
    if (planes * tokens > kMaxScalars / channels) return false;
    if (chunk_tokens < 1 || chunk_tokens > kMaxChunkTokens) return false;
    const bool blocks = sigma_block_tokens != 0 && int64_t(sigma_block_tokens) < tokens;
    if (blocks && sigma_block_tokens % chunk_tokens) return false;
    const int64_t n_blocks = blocks ? (tokens + sigma_block_tokens - 1) / sigma_block_tokens : 1;
    if (planes * n_blocks * channels >= (int64_t(1) << 32)) return false;   // sigma words indexable
    // a chunk's rows span chunk_tokens * channels scalars of up to 4 bytes: byte offsets fit 31 bits
    if (int64_t(chunk_tokens) * channels >= (int64_t(1) << 29)) return false;
    g->planes = planes;
    g->tokens = tokens;
    g->channels = channels;
    g->chunk_tokens = chunk_tokens;
    g->n_tok_chunks = static_cast<uint32_t>((tokens + chunk_tokens - 1) / chunk_tokens);
    g->n_groups = static_cast<uint32_t>(channels / 64);
    g->sigma_tc = blocks ? sigma_block_tokens / chunk_tokens : 0u;
    g->n_chunks = planes * int64_t(g->n_tok_chunks) * int64_t(g->n_groups);
    g->sigma_blocks = n_blocks;
    return true;
}

// Words of sigma: [planes][sigma blocks][channels].
uint64_t sigma_words(const ChunkGeom& g) {
    return uint64_t(g.planes) * uint64_t(g.sigma_blocks) * uint64_t(g.channels);
}

// Words of the side buffer: sigma, then (with a per-channel split) the
// narrow weight of every (plane, channel).
uint64_t side_words(const ChunkGeom& g, uint32_t channel_split) {
    return sigma_words(g) + (channel_split ? uint64_t(g.planes) * uint64_t(g.channels) : 0u);
}

// The kernels' view of a per-channel split (no split: words null).
kvc::SplitArgs split_args(uint32_t channel_split, const ChunkGeom& g, const float* d_side, int32_t kv_dtype,
                          uint32_t w_narrow_bp, uint32_t w_wide_bp, const kvc::PhiTables& phi) {
    kvc::SplitArgs a;
    if (!channel_split) return a;
    a.words = reinterpret_cast<const uint32_t*>(d_side) + sigma_words(g);
    a.a = phi.a;
    a.b = phi.b;
    a.t_all = static_cast<uint32_t>((uint64_t(1) << kLog2M) - alphabet(kv_dtype));
    a.w_gauss = w_narrow_bp + w_wide_bp;
    return a;
}

// Default chunk length.  Each chunk is one wave and MI355X holds 8,192 of
// them at once (256 CUs x 32 waves), so a call runs in rounds of 8,192
// chunks, each round as long as one chunk.  Among the lengths
// ceil(T / k) from at most 1024 tokens down to 256 (or T when shorter), the
// default takes the one with the least rounds x (length + 9): the time of
// the call, plus a per-chunk allowance for the final states (about 47 bits
// per lane) and the per-chunk set-up.  Ties go to the longer chunk; of the
// lengths that give the same chunks per plane, the shortest costs least,
// so the choice is always some ceil(T / k).
constexpr int64_t kWaveSlots = 256 * 32;
constexpr int64_t kChunkMax = 1024, kChunkFloor = 256, kChunkAllowance = 9;

uint32_t default_chunk_tokens(int64_t planes, int64_t tokens, int64_t channels, uint32_t sigma_block_tokens) {
    if (tokens <= 0) return 1;
    if (planes <= 0 || channels < 64) return static_cast<uint32_t>(tokens < kChunkMax ? tokens : kChunkMax);
    const int64_t groups = channels / 64;
    // with sigma blocks shorter than the tokens, only divisors of the block
    // length (so that no chunk straddles two blocks)
    const int64_t blk = (sigma_block_tokens != 0 && int64_t(sigma_block_tokens) < tokens) ? sigma_block_tokens : 0;
    const int64_t span = blk ? blk : tokens;
    const int64_t top = span < kChunkMax ? span : kChunkMax;
    int64_t floor_len = span < kChunkFloor ? span : kChunkFloor;
    if (blk) {
        // no divisor of B in [floor, top]: the largest divisor below
        bool any = false;
        for (int64_t len = top; len >= floor_len && !any; --len) any = blk % len == 0;
        if (!any) floor_len = 1;
    }
    int64_t best_len = 0, best_cost = -1;
    for (int64_t len = top; len >= floor_len; --len) {          // at most 1024 lengths
        if (blk && blk % len) continue;
        const int64_t chunks = planes * ((tokens + len - 1) / len) * groups;
        const int64_t cost = ((chunks + kWaveSlots - 1) / kWaveSlots) * (len + kChunkAllowance);
        if (best_cost < 0 || cost < best_cost) {
            best_len = len;
            best_cost = cost;
        }
    }
    return static_cast<uint32_t>(best_len);
}

bool params_geometry(const kvc_params* p, ChunkGeom* g) {
    if (!p || !kv_dtype_ok(p->kv_dtype) || !mu_dtype_ok(p->mu_dtype)) return false;
    if (p->narrow_dof > uint32_t(kvc::kNarrowDofMax) || p->channel_split > 1) return false;
    uint32_t tc = p->chunk_tokens;
    if (tc == 0) tc = default_chunk_tokens(p->planes, p->tokens, p->channels, p->sigma_block_tokens);
    return geometry(p->planes, p->tokens, p->channels, tc, p->sigma_block_tokens, g);
}

// Workspace of the encoder: control block (and the header copy), the
// look-back entries of the chunk sizes, one word slot per chunk sized for
// two words per scalar (the worst case), then the per-call mixture and
// escape slot tables.  A slot is written and read back by its chunk's wave
// alone, never reused within a call.
struct EncodeLayout {
    uint64_t status, slots, table, eslots, total, slot_words, max_stream;
};

EncodeLayout encode_layout(const ChunkGeom& g) {
    EncodeLayout l;
    const uint64_t n = static_cast<uint64_t>(g.n_chunks);
    l.slot_words = round_up(2ull * kLanes * g.chunk_tokens, 4);
    l.status = 256;
    l.slots = round_up(l.status + n * 8, 256);
    l.table = round_up(l.slots + n * l.slot_words * 2, 256);
    l.eslots = round_up(l.table + kvc::kTableBytes, 256);
    l.total = l.eslots + kvc::kEscapeSlotsBytes;
    l.max_stream = KVC_HEADER_BYTES + 8 * (n + 1) + n * (kLanes * 8 + l.slot_words * 2);
    return l;
}

void put16(uint8_t* b, int off, uint16_t v) { std::memcpy(b + off, &v, 2); }
void put32(uint8_t* b, int off, uint32_t v) { std::memcpy(b + off, &v, 4); }
void put64(uint8_t* b, int off, uint64_t v) { std::memcpy(b + off, &v, 8); }
uint16_t get16(const uint8_t* b, int off) { uint16_t v; std::memcpy(&v, b + off, 2); return v; }
uint32_t get32(const uint8_t* b, int off) { uint32_t v; std::memcpy(&v, b + off, 4); return v; }
uint64_t get64(const uint8_t* b, int off) { uint64_t v; std::memcpy(&v, b + off, 8); return v; }

// KVC-1 header; payload size (offset 72) and side hash (offset 80) are
// filled in on the device.
kvc::StreamHeader make_header(const kvc_params* p, const ChunkGeom& g, uint32_t tn, uint32_t tw, uint32_t te) {
    kvc::StreamHeader h;
    std::memset(h.bytes, 0, sizeof(h.bytes));
    std::memcpy(h.bytes, "KVC1", 4);
    put16(h.bytes, 4, kVersion);
    put16(h.bytes, 6, KVC_HEADER_BYTES);
    h.bytes[8] = static_cast<uint8_t>(p->kv_dtype);
    h.bytes[9] = static_cast<uint8_t>(p->mu_dtype);
    h.bytes[10] = kLog2M;
    h.bytes[11] = kLog2L;
    h.bytes[12] = kWordBits;
    h.bytes[13] = kLanes;
    h.bytes[14] = static_cast<uint8_t>(p->narrow_dof);
    h.bytes[15] = static_cast<uint8_t>(p->channel_split);
    put32(h.bytes, 16, p->w_narrow_bp);
    put32(h.bytes, 20, p->w_wide_bp);
    put32(h.bytes, 24, tn);
    put32(h.bytes, 28, tw);
    put32(h.bytes, 32, te);
    put32(h.bytes, 36, g.chunk_tokens);
    put64(h.bytes, 40, static_cast<uint64_t>(g.planes));
    put64(h.bytes, 48, static_cast<uint64_t>(g.tokens));
    put64(h.bytes, 56, static_cast<uint64_t>(g.channels));
    put64(h.bytes, 64, static_cast<uint64_t>(g.n_chunks));
    put32(h.bytes, 88, p->sigma_block_tokens);
    return h;
}

// CRC-32 (reflected polynomial 0xEDB88320, initial value and final xor
// 0xFFFFFFFF: the zlib / gzip / PNG checksum), bit by bit.
uint32_t crc32(const uint8_t* b, size_t n) {
    uint32_t c = 0xFFFFFFFFu;
    for (size_t i = 0; i < n; ++i) {
        c ^= b[i];
        for (int k = 0; k < 8; ++k) c = (c >> 1) ^ ((c & 1u) ? 0xEDB88320u : 0u);
    }
    return ~c;
}

int parse_header(const uint8_t* b, kvc_params* p, ChunkGeom* g, uint64_t* payload, uint64_t* hash) {
    if (std::memcmp(b, "KVC1", 4) != 0 || get16(b, 4) != kVersion || get16(b, 6) != KVC_HEADER_BYTES)
        return KVC_ERR_CORRUPT;
    if (get32(b, kvc::kHeaderCrcOffset) != crc32(b, kvc::kHeaderCrcOffset)) return KVC_ERR_CORRUPT;
    if (b[10] != kLog2M || b[11] != kLog2L || b[12] != kWordBits || b[13] != kLanes ||
        b[14] > kvc::kNarrowDofMax || b[15] > 1)
        return KVC_ERR_CORRUPT;
    kvc_params q;
    std::memset(&q, 0, sizeof(q));
    q.kv_dtype = b[8];
    q.mu_dtype = b[9];
    q.w_narrow_bp = get32(b, 16);
    q.w_wide_bp = get32(b, 20);
    q.chunk_tokens = get32(b, 36);
    q.planes = static_cast<int64_t>(get64(b, 40));
    q.tokens = static_cast<int64_t>(get64(b, 48));
    q.channels = static_cast<int64_t>(get64(b, 56));
    q.sigma_block_tokens = get32(b, 88);
    q.narrow_dof = b[14];
    q.channel_split = b[15];
    uint32_t tn, tw, te;
    if (!kv_dtype_ok(q.kv_dtype) || !mu_dtype_ok(q.mu_dtype) ||
        !budgets(q.kv_dtype, q.w_narrow_bp, q.w_wide_bp, &tn, &tw, &te))
        return KVC_ERR_CORRUPT;
    if (tn != get32(b, 24) || tw != get32(b, 28) || te != get32(b, 32)) return KVC_ERR_CORRUPT;
    if (get64(b, 40) > uint64_t(kMaxScalars) || get64(b, 48) > uint64_t(kMaxScalars) ||
        get64(b, 56) > uint64_t(kMaxScalars))
        return KVC_ERR_CORRUPT;
    if (q.chunk_tokens == 0 || !geometry(q.planes, q.tokens, q.channels, q.chunk_tokens, q.sigma_block_tokens, g))
        return KVC_ERR_CORRUPT;
    if (get64(b, 64) != static_cast<uint64_t>(g->n_chunks)) return KVC_ERR_CORRUPT;
    for (int i = kvc::kHeaderCrcOffset + 4; i < KVC_HEADER_BYTES; ++i)
        if (b[i]) return KVC_ERR_CORRUPT;
    *payload = get64(b, 72);
    *hash = get64(b, 80);
    if (p) *p = q;
    return KVC_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_DEVICE; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Element alignment of KV / mu / sigma / prefix buffers.
bool data_aligned(int32_t kv_dtype, int32_t mu_dtype, const void* kv, const void* mu, const void* sigma,
                  const void* prefix) {
    return aligned(kv, kv_dtype == KVC_BF16 ? 2 : 1) && aligned(mu, mu_dtype == KVC_F32 ? 4 : 2) &&
           aligned(sigma, 4) && aligned(prefix, 4);
}

// Optional stage timing with HIP events on the call's stream; inert when
// the caller passes no output array.
class StageTimer {
  public:
    StageTimer(float* out, int stages, hipStream_t s) : out_(out), n_(stages), s_(s) {
        if (!out_) return;
        for (int i = 0; i <= n_ && ok_; ++i) ok_ = hipEventCreate(&ev_[i]) == hipSuccess;
    }
    ~StageTimer() {
        if (!out_) return;
        for (int i = 0; i <= n_; ++i)
            if (ev_[i]) (void)hipEventDestroy(ev_[i]);
    }
    void mark(int i) {
        if (out_ && ok_) ok_ = hipEventRecord(ev_[i], s_) == hipSuccess;
    }
    // after the stream has been synchronised
    void read() {
        if (!out_) return;
        for (int i = 0; i < n_; ++i) {
            float ms = -1.0f;
            if (ok_ && hipEventElapsedTime(&ms, ev_[i], ev_[i + 1]) != hipSuccess) ms = -1.0f;
            out_[i] = ms;
        }
    }

  private:
    float* out_;
    int n_;
    hipStream_t s_;
    bool ok_ = true;
    hipEvent_t ev_[8] = {};
};

}  // namespace

extern "C" {

int kvc_version(void) { return static_cast<int>(kVersion); }

const char* kvc_status_string(int status) {
    switch (status) {
        case KVC_OK: return "ok";
        case KVC_ERR_INVALID: return "invalid argument";
        case KVC_ERR_CAPACITY: return "buffer too small";
        case KVC_ERR_CORRUPT: return "corrupt stream";
        case KVC_ERR_MISMATCH: return "side information does not match the stream";
        case KVC_ERR_DEVICE: return "device error";
        default: return "unknown status";
    }
}

int kvc_phi_tables(uint32_t* h_narrow, uint32_t* h_wide) {
    if (!h_narrow || !h_wide) return KVC_ERR_INVALID;
    kvc::host_phi_tables(h_narrow, h_wide);
    return KVC_OK;
}

int kvc_narrow_table(uint32_t narrow_dof, uint32_t* h_out) {
    if (!h_out || narrow_dof > uint32_t(kvc::kNarrowDofMax)) return KVC_ERR_INVALID;
    kvc::host_narrow_table(narrow_dof, h_out);
    return KVC_OK;
}

int kvc_encode_sizes(const kvc_params* p, uint64_t* h_max_stream_bytes, uint64_t* h_workspace_bytes) {
    ChunkGeom g;
    if (!params_geometry(p, &g)) return KVC_ERR_INVALID;
    uint32_t tn, tw, te;
    if (!budgets(p->kv_dtype, p->w_narrow_bp, p->w_wide_bp, &tn, &tw, &te)) return KVC_ERR_INVALID;
    const EncodeLayout l = encode_layout(g);
    if (h_max_stream_bytes) *h_max_stream_bytes = l.max_stream;
    if (h_workspace_bytes) *h_workspace_bytes = l.total;
    return KVC_OK;
}

int kvc_encode(const kvc_params* p, const void* d_kv, const void* d_mu, const float* d_sigma,
               const uint32_t* d_prefix, void* d_out, uint64_t out_capacity, uint64_t* h_out_bytes,
               void* h_header_out, void* d_workspace, uint64_t workspace_bytes, void* stream,
               kvc_encode_info* h_info) {
    ChunkGeom g;
    if (!params_geometry(p, &g) || !d_kv || !d_mu || !d_sigma || !d_out || !d_workspace) return KVC_ERR_INVALID;
    if (!h_out_bytes && (h_header_out || h_info)) return KVC_ERR_INVALID;   // host outputs need the sync
    uint32_t tn, tw, te;
    if (!budgets(p->kv_dtype, p->w_narrow_bp, p->w_wide_bp, &tn, &tw, &te)) return KVC_ERR_INVALID;
    if (te && !d_prefix) return KVC_ERR_INVALID;
    if (!data_aligned(p->kv_dtype, p->mu_dtype, d_kv, d_mu, d_sigma, d_prefix) || !aligned(d_out, 8) ||
        !aligned(d_workspace, 256))
        return KVC_ERR_INVALID;
    const EncodeLayout l = encode_layout(g);
    if (workspace_bytes < l.total) return KVC_ERR_CAPACITY;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const kvc::PhiTables phi = kvc::device_phi_tables(&e, p->narrow_dof);
    if (e != hipSuccess) return KVC_ERR_DEVICE;

    uint8_t* ws = static_cast<uint8_t*>(d_workspace);
    Control* ctl = reinterpret_cast<Control*>(ws);
    const uint32_t* prefix = te ? d_prefix : nullptr;
    // the mixture table: the device's cached one, else built here
    const uint32_t* table = nullptr;
    const float* no_aim = nullptr;
    if (!kvc::cached_coder_tables(tn, tw, p->narrow_dof, phi, s, &table, &no_aim, &e)) {
        if (e != hipSuccess) return KVC_ERR_DEVICE;
        table = reinterpret_cast<const uint32_t*>(ws + l.table);
        if ((e = kvc::launch_coder_tables(phi, tn, tw, reinterpret_cast<uint32_t*>(ws + l.table), nullptr, s)) !=
            hipSuccess)
            return KVC_ERR_DEVICE;
    }
    StageTimer timer(h_info ? h_info->stage_ms : nullptr, KVC_ENCODE_STAGES, s);
    if ((e = kvc::launch_clear_control(ctl, s)) != hipSuccess) return KVC_ERR_DEVICE;
    timer.mark(0);
    kvc::PrologueArgs pa;
    pa.sigma_words = reinterpret_cast<const uint32_t*>(d_sigma);
    pa.n_sigma = side_words(g, p->channel_split);
    pa.prefix_words = prefix;
    pa.n_prefix = prefix ? alphabet(p->kv_dtype) + 1u : 0u;
    pa.prefix = prefix ? prefix : phi.zero;
    pa.htot = tn + tw;
    if (p->kv_dtype == KVC_BF16) pa.eslots = reinterpret_cast<uint2*>(ws + l.eslots);
    pa.zero = reinterpret_cast<unsigned long long*>(ws + l.status);
    pa.n_zero = uint64_t(g.n_chunks);
    pa.ctl = ctl;
    if ((e = kvc::launch_prologue(pa, p->kv_dtype, s)) != hipSuccess) return KVC_ERR_DEVICE;

    kvc::EncodeArgs ea;
    ea.geom = g;
    ea.kv = d_kv;
    ea.mu = d_mu;
    ea.sigma = d_sigma;
    ea.prefix = prefix ? prefix : phi.zero;          // kernels read a prefix unconditionally
    ea.tn = tn;
    ea.tw = tw;
    ea.table = table;
    ea.eslots = reinterpret_cast<const uint32_t*>(ws + l.eslots);
    ea.slots = reinterpret_cast<uint16_t*>(ws + l.slots);
    ea.slot_words = l.slot_words;
    ea.status = reinterpret_cast<unsigned long long*>(ws + l.status);
    ea.out = static_cast<uint8_t*>(d_out);
    ea.out_capacity = out_capacity;
    ea.header = make_header(p, g, tn, tw, te);
    ea.header_copy = ws + kvc::kHeaderCopyOffset;
    ea.split = split_args(p->channel_split, g, d_sigma, p->kv_dtype, p->w_narrow_bp, p->w_wide_bp, phi);
    ea.ctl = ctl;
    timer.mark(1);
    if ((e = kvc::launch_encode(ea, p->kv_dtype, p->mu_dtype, s)) != hipSuccess) return KVC_ERR_DEVICE;
    timer.mark(2);
    if (!h_out_bytes) return KVC_OK;                  // asynchronous: kvc_encode_result reads the outcome
    const int st = kvc_encode_result(d_workspace, stream, h_out_bytes, h_header_out);
    timer.read();
    return st;
}

int kvc_encode_result(const void* d_workspace, void* stream, uint64_t* h_out_bytes, void* h_header_out) {
    if (!d_workspace || !h_out_bytes || !aligned(d_workspace, 256)) return KVC_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t blk[kvc::kHeaderCopyOffset + KVC_HEADER_BYTES];
    if (hipMemcpyAsync(blk, d_workspace, sizeof(blk), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return KVC_ERR_DEVICE;
    Control host;
    std::memcpy(&host, blk, sizeof(host));
    const uint8_t* head = blk + kvc::kHeaderCopyOffset;
    // the workspace's header copy is written also when the stream did not
    // fit, so the size it needed is known then too
    kvc_params q;
    ChunkGeom g;
    uint64_t payload = 0, hash = 0;
    if (host.flags & kvc::kFlagStall) return KVC_ERR_DEVICE;
    if (host.flags & kvc::kFlagBadSigma) return KVC_ERR_INVALID;
    if (parse_header(head, &q, &g, &payload, &hash) != KVC_OK || payload != host.total_payload)
        return KVC_ERR_DEVICE;
    *h_out_bytes = KVC_HEADER_BYTES + 8ull * uint64_t(g.n_chunks + 1) + payload;
    if (host.flags & kvc::kFlagCapacity) return KVC_ERR_CAPACITY;
    if (h_header_out) std::memcpy(h_header_out, head, KVC_HEADER_BYTES);
    return KVC_OK;
}

int kvc_stream_info(const void* h_header, uint64_t header_bytes, kvc_params* h_params, uint64_t* h_stream_bytes) {
    if (!h_header || header_bytes < KVC_HEADER_BYTES) return KVC_ERR_INVALID;
    ChunkGeom g;
    uint64_t payload = 0, hash = 0;
    const int st = parse_header(static_cast<const uint8_t*>(h_header), h_params, &g, &payload, &hash);
    if (st != KVC_OK) return st;
    if (h_stream_bytes) *h_stream_bytes = KVC_HEADER_BYTES + 8ull * uint64_t(g.n_chunks + 1) + payload;
    return KVC_OK;
}

}  // extern "C"

namespace {

// Sizes in bytes of one element of each dtype.
uint64_t kv_size(int32_t t) { return t == KVC_BF16 ? 2u : 1u; }
uint64_t mu_size(int32_t t) { return t == KVC_F32 ? 4u : 2u; }

// kvc_decode_async and kvc_decode_paged_async: the output is d_kv_out, or
// the paged pools when `paged` is not null.  Everything is checked on the
// host against the header the caller holds before anything is launched;
// the kernels compare the device stream's header with it.
// What a decode call needs, from its host-side checks alone (no device call).
struct DecodePlan {
    kvc_params p;
    ChunkGeom g;
    uint64_t payload = 0, hash = 0, dir_bytes = 0;
    uint32_t tn = 0, tw = 0, te = 0, n_sym = 0;
    const uint32_t* prefix = nullptr;
    kvc::PagedOut po{};
};

// Every check a decode makes before touching the device: arguments, the
// header (CRC included), the stream's length against it, and every caller
// buffer against what it describes.
int decode_check(const void* h_header, const void* d_in, uint64_t in_bytes, const void* d_mu, uint64_t mu_bytes,
                 const float* d_sigma, uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                 void* d_kv_out, uint64_t kv_out_bytes, const kvc_paged_kv* paged, const void* d_workspace,
                 uint64_t workspace_bytes, DecodePlan* plan) {
    if (!h_header || !d_in || !d_mu || !d_sigma || (!d_kv_out && !paged) || !d_workspace) return KVC_ERR_INVALID;
    if (workspace_bytes < KVC_DECODE_WORKSPACE_BYTES) return KVC_ERR_CAPACITY;
    if (!aligned(d_in, 8) || !aligned(d_workspace, 256) || !aligned(d_sigma, 4) || !aligned(d_prefix, 4) ||
        !aligned(d_kv_out, 2) || !aligned(d_mu, 2))
        return KVC_ERR_INVALID;
    if (paged) {
        if (!paged->d_pools || !paged->d_block_table || !aligned(paged->d_pools, 8) ||
            !aligned(paged->d_block_table, 4) || paged->page_tokens < 1 || paged->batch < 1 || paged->heads < 1 ||
            paged->batch > 0x7FFFFFFF || paged->heads > 0x7FFFFFFF || paged->num_pages < 1 ||
            paged->num_pages > 0x7FFFFFFF || paged->max_pages < 1 || paged->max_pages > kMaxScalars ||
            paged->batch * paged->max_pages > kMaxScalars || paged->n_pools < 1 || paged->n_pools > kMaxScalars ||
            paged->reserved != 0)
            return KVC_ERR_INVALID;
    }
    kvc_params& p = plan->p;
    ChunkGeom& g = plan->g;
    int st = parse_header(static_cast<const uint8_t*>(h_header), &p, &g, &plan->payload, &plan->hash);
    if (st != KVC_OK) return st;
    plan->dir_bytes = 8ull * uint64_t(g.n_chunks + 1);
    if (in_bytes < KVC_HEADER_BYTES + plan->dir_bytes || in_bytes - KVC_HEADER_BYTES - plan->dir_bytes != plan->payload)
        return KVC_ERR_CORRUPT;
    if (!budgets(p.kv_dtype, p.w_narrow_bp, p.w_wide_bp, &plan->tn, &plan->tw, &plan->te)) return KVC_ERR_CORRUPT;
    if (plan->te && !d_prefix) return KVC_ERR_INVALID;
    plan->prefix = plan->te ? d_prefix : nullptr;
    if (!data_aligned(p.kv_dtype, p.mu_dtype, d_kv_out, d_mu, d_sigma, d_prefix)) return KVC_ERR_INVALID;
    // the caller's buffers must hold what the header describes
    const uint64_t n = uint64_t(g.planes) * uint64_t(g.tokens) * uint64_t(g.channels);
    plan->n_sym = alphabet(p.kv_dtype);
    if (mu_bytes / mu_size(p.mu_dtype) < n || sigma_bytes / 4u < side_words(g, p.channel_split))
        return KVC_ERR_INVALID;
    if (plan->prefix && prefix_bytes / 4u < uint64_t(plan->n_sym) + 1u) return KVC_ERR_INVALID;
    if (!paged && kv_out_bytes / kv_size(p.kv_dtype) < n) return KVC_ERR_INVALID;
    kvc::PagedOut& po = plan->po;
    if (paged) {
        // planes ordered (layer, kv, batch, head), one pool per (layer, kv);
        // every token's page inside the table's rows; every pool holds
        // num_pages pages of page_tokens rows of heads x channels elements
        const int64_t per_kv = paged->batch * paged->heads;
        if (g.planes % (2 * per_kv) != 0 || g.planes / per_kv != paged->n_pools) return KVC_ERR_INVALID;
        if (paged->max_pages < (g.tokens + paged->page_tokens - 1) / paged->page_tokens) return KVC_ERR_INVALID;
        const uint64_t page_bytes = uint64_t(paged->heads) * uint64_t(g.channels) * kv_size(p.kv_dtype) *
                                    uint64_t(paged->page_tokens);
        if (page_bytes >= (uint64_t(1) << 32)) return KVC_ERR_INVALID;        // a page's bytes fit 32 bits
        if (paged->pool_bytes / page_bytes < uint64_t(paged->num_pages)) return KVC_ERR_INVALID;
        po.pools = paged->d_pools;
        po.block_table = paged->d_block_table;
        po.max_pages = paged->max_pages;
        po.num_pages = paged->num_pages;
        po.page_tokens = paged->page_tokens;
        po.heads = static_cast<uint32_t>(paged->heads);
        po.batch = static_cast<uint32_t>(paged->batch);
    }
    return KVC_OK;
}

int decode_launch(const void* h_header, const void* d_in, uint64_t in_bytes, const void* d_mu, uint64_t mu_bytes,
                  const float* d_sigma, uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                  void* d_kv_out, uint64_t kv_out_bytes, const kvc_paged_kv* paged, void* d_workspace,
                  uint64_t workspace_bytes, void* stream, float* stage_ms) {
    DecodePlan plan;
    int st = decode_check(h_header, d_in, in_bytes, d_mu, mu_bytes, d_sigma, sigma_bytes, d_prefix, prefix_bytes,
                          d_kv_out, kv_out_bytes, paged, d_workspace, workspace_bytes, &plan);
    if (st != KVC_OK) return st;
    const kvc_params& p = plan.p;
    const ChunkGeom& g = plan.g;
    const uint32_t tn = plan.tn, tw = plan.tw, te = plan.te, n_sym = plan.n_sym;
    const uint32_t* prefix = plan.prefix;
    const uint64_t dir_bytes = plan.dir_bytes, payload = plan.payload, hash = plan.hash;
    const kvc::PagedOut& po = plan.po;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const kvc::PhiTables phi = kvc::device_phi_tables(&e, p.narrow_dof);
    if (e != hipSuccess) return KVC_ERR_DEVICE;

    Control* ctl = static_cast<Control*>(d_workspace);
    // escape bucket table after the control block: the smallest shift that
    // keeps ((N + T_e - 1) >> shift) + 2 entries within the table
    const uint64_t q_total = uint64_t(n_sym) + te;
    uint32_t shift = 0;
    while (((q_total - 1) >> shift) + 2 > kvc::kEscapeBucketsMax) ++shift;
    const uint32_t n_buckets = static_cast<uint32_t>(((q_total - 1) >> shift) + 2);
    uint32_t* buckets = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(d_workspace) + kDecodeBucketOffset);
    uint8_t* ws = static_cast<uint8_t*>(d_workspace);
    // the mixture and aim tables: the device's cached ones, else built here
    const uint32_t* table = nullptr;
    const float* aim = nullptr;
    if (!kvc::cached_coder_tables(tn, tw, p.narrow_dof, phi, s, &table, &aim, &e)) {
        if (e != hipSuccess) return KVC_ERR_DEVICE;
        table = reinterpret_cast<const uint32_t*>(ws + kDecodeTableOffset);
        aim = reinterpret_cast<const float*>(ws + kDecodeAimOffset);
        if ((e = kvc::launch_coder_tables(phi, tn, tw, reinterpret_cast<uint32_t*>(ws + kDecodeTableOffset),
                                          reinterpret_cast<float*>(ws + kDecodeAimOffset), s)) != hipSuccess)
            return KVC_ERR_DEVICE;
    }
    StageTimer timer(stage_ms, KVC_DECODE_STAGES, s);
    if ((e = kvc::launch_clear_control(ctl, s)) != hipSuccess) return KVC_ERR_DEVICE;
    timer.mark(0);
    kvc::PrologueArgs pa;
    pa.sigma_words = reinterpret_cast<const uint32_t*>(d_sigma);
    pa.n_sigma = side_words(g, p.channel_split);
    pa.prefix_words = prefix;
    pa.n_prefix = prefix ? n_sym + 1u : 0u;
    pa.head = static_cast<const uint8_t*>(d_in);
    std::memcpy(pa.expect.bytes, h_header, KVC_HEADER_BYTES);
    pa.prefix = prefix ? prefix : phi.zero;
    pa.htot = tn + tw;
    if (p.kv_dtype == KVC_BF16) pa.ecount = reinterpret_cast<uint32_t*>(ws + kDecodeCountOffset);
    pa.buckets = reinterpret_cast<uint2*>(buckets);
    pa.n_sym = n_sym;
    pa.bucket_shift = shift;
    pa.n_buckets = n_buckets;
    if (paged) {
        pa.pages = po;
        pa.pages_used = (g.tokens + po.page_tokens - 1) / po.page_tokens;
    }
    pa.ctl = ctl;
    if ((e = kvc::launch_prologue(pa, p.kv_dtype, s)) != hipSuccess) return KVC_ERR_DEVICE;
    timer.mark(1);
    const uint8_t* in = static_cast<const uint8_t*>(d_in);
    kvc::DecodeArgs da;
    da.geom = g;
    da.directory = reinterpret_cast<const unsigned long long*>(in + KVC_HEADER_BYTES);
    da.payload = in + KVC_HEADER_BYTES + dir_bytes;
    da.payload_bytes = payload;
    da.mu = d_mu;
    da.sigma = d_sigma;
    da.prefix = prefix ? prefix : phi.zero;
    da.tn = tn;
    da.tw = tw;
    da.table = table;
    da.aim = aim;
    da.buckets = buckets;
    da.bucket_shift = shift;
    da.ecount = reinterpret_cast<const uint32_t*>(ws + kDecodeCountOffset);
    da.kv_out = d_kv_out;
    da.paged = po;
    da.expect_hash = hash;
    da.split = split_args(p.channel_split, g, d_sigma, p.kv_dtype, p.w_narrow_bp, p.w_wide_bp, phi);
    da.ctl = ctl;
    if ((e = kvc::launch_decode(da, p.kv_dtype, p.mu_dtype, paged != nullptr, s)) != hipSuccess) return KVC_ERR_DEVICE;
    timer.mark(2);
    if (stage_ms) {
        // stage times need the stream finished: the caller synchronises
        // through kvc_decode_result right after
        if (hipStreamSynchronize(s) != hipSuccess) return KVC_ERR_DEVICE;
        timer.read();
    }
    return KVC_OK;
}

// Status of a decode from its control block (after the stream has finished).
int decode_status(const Control& host) {
    if (host.flags & kvc::kFlagHeader) return KVC_ERR_CORRUPT;
    if (host.flags & kvc::kFlagMismatch) return KVC_ERR_MISMATCH;
    if (host.flags & (kvc::kFlagBadSigma | kvc::kFlagBadPage)) return KVC_ERR_INVALID;
    if (host.flags & kvc::kFlagCorrupt) return KVC_ERR_CORRUPT;
    return KVC_OK;
}

}  // namespace

extern "C" {

int kvc_decode_async(const void* h_header, const void* d_in, uint64_t in_bytes, const void* d_mu, uint64_t mu_bytes,
                     const float* d_sigma, uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                     void* d_kv_out, uint64_t kv_out_bytes, void* d_workspace, uint64_t workspace_bytes,
                     void* stream) {
    if (!d_kv_out) return KVC_ERR_INVALID;
    return decode_launch(h_header, d_in, in_bytes, d_mu, mu_bytes, d_sigma, sigma_bytes, d_prefix, prefix_bytes,
                         d_kv_out, kv_out_bytes, nullptr, d_workspace, workspace_bytes, stream, nullptr);
}

int kvc_decode_result(const void* d_workspace, void* stream, kvc_decode_info* h_info) {
    if (!d_workspace || !aligned(d_workspace, 256)) return KVC_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Control host;
    if (hipMemcpyAsync(&host, d_workspace, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return KVC_ERR_DEVICE;
    if (h_info) h_info->fallback_symbols = host.misses;
    return decode_status(host);
}

int kvc_decode(const void* h_header, const void* d_in, uint64_t in_bytes, const void* d_mu, uint64_t mu_bytes,
               const float* d_sigma, uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
               void* d_kv_out, uint64_t kv_out_bytes, void* d_workspace, uint64_t workspace_bytes, void* stream,
               kvc_decode_info* h_info) {
    if (!d_kv_out) return KVC_ERR_INVALID;
    const int st = decode_launch(h_header, d_in, in_bytes, d_mu, mu_bytes, d_sigma, sigma_bytes, d_prefix,
                                 prefix_bytes, d_kv_out, kv_out_bytes, nullptr, d_workspace, workspace_bytes, stream,
                                 h_info ? h_info->stage_ms : nullptr);
    if (st != KVC_OK) return st;
    return kvc_decode_result(d_workspace, stream, h_info);
}

int kvc_decode_noalloc(const void* h_header, const void* d_in, uint64_t in_bytes, const void* d_mu,
                       uint64_t mu_bytes, const float* d_sigma, uint64_t sigma_bytes, const uint32_t* d_prefix,
                       uint64_t prefix_bytes, void* d_kv_out, uint64_t kv_out_bytes, void* stream) {
    static_assert(kvc::kNoAllocScratchBytes >= KVC_DECODE_WORKSPACE_BYTES, "scratch holds a decode workspace");
    if (!d_kv_out) return KVC_ERR_INVALID;
    hipError_t e = hipSuccess;
    void* ws = kvc::noalloc_scratch(&e);
    if (e != hipSuccess || !ws) return KVC_ERR_DEVICE;
    // the decoder's workspace does not grow with the stream; a layout that
    // needed more than the scratch holds would be refused here
    if (KVC_DECODE_WORKSPACE_BYTES > kvc::kNoAllocScratchBytes) return KVC_ERR_CAPACITY;
    const int st = decode_launch(h_header, d_in, in_bytes, d_mu, mu_bytes, d_sigma, sigma_bytes, d_prefix,
                                 prefix_bytes, d_kv_out, kv_out_bytes, nullptr, ws, kvc::kNoAllocScratchBytes, stream,
                                 nullptr);
    if (st != KVC_OK) return st;
    return kvc_decode_result(ws, stream, nullptr);
}

int kvc_reload(int64_t n, const void* const* h_streams, const uint64_t* h_stream_bytes, const void* d_mu,
               uint64_t mu_stride, const float* d_sigma, uint64_t sigma_stride, const uint32_t* d_prefix,
               uint64_t prefix_bytes, void* d_kv_out, uint64_t kv_stride, void* d_staging, uint64_t staging_bytes,
               void* d_workspace, uint64_t workspace_bytes, void* stream, void* copy_stream, int64_t* h_failed) {
    if (h_failed) *h_failed = -1;
    if (n < 1 || !h_streams || !h_stream_bytes || !d_mu || !d_sigma || !d_kv_out || !d_staging || !d_workspace ||
        !aligned(d_staging, 256) || !aligned(d_workspace, 256))
        return KVC_ERR_INVALID;
    if (workspace_bytes / KVC_DECODE_WORKSPACE_BYTES < uint64_t(n)) return KVC_ERR_CAPACITY;
    // two staging halves, each 256-byte aligned; every stream must fit one.
    // Every layer passes the decode's host checks (its header read in host
    // memory, its buffers) before anything is copied or launched.
    const uint64_t half = (staging_bytes / 2) & ~uint64_t(255);
    for (int64_t l = 0; l < n; ++l) {
        int st = KVC_OK;
        if (!h_streams[l] || h_stream_bytes[l] < KVC_HEADER_BYTES) st = KVC_ERR_CORRUPT;
        else if (h_stream_bytes[l] > half) st = KVC_ERR_CAPACITY;
        if (st == KVC_OK) {
            DecodePlan plan;
            st = decode_check(h_streams[l], static_cast<uint8_t*>(d_staging) + (l & 1) * half, h_stream_bytes[l],
                              static_cast<const uint8_t*>(d_mu) + uint64_t(l) * mu_stride, mu_stride,
                              reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(d_sigma) +
                                                             uint64_t(l) * sigma_stride),
                              sigma_stride, d_prefix, prefix_bytes,
                              static_cast<uint8_t*>(d_kv_out) + uint64_t(l) * kv_stride, kv_stride, nullptr,
                              static_cast<uint8_t*>(d_workspace) + uint64_t(l) * KVC_DECODE_WORKSPACE_BYTES,
                              KVC_DECODE_WORKSPACE_BYTES, &plan);
        }
        if (st != KVC_OK) {
            if (h_failed) *h_failed = l;
            return st;
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
    hipEvent_t copied[2] = {}, consumed[2] = {};
    int st = KVC_OK;
    for (int i = 0; i < 2 && st == KVC_OK; ++i)
        if (hipEventCreateWithFlags(&copied[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&consumed[i], hipEventDisableTiming) != hipSuccess)
            st = KVC_ERR_DEVICE;
    uint8_t* stage = static_cast<uint8_t*>(d_staging);
    uint8_t* ws = static_cast<uint8_t*>(d_workspace);
    int64_t queued = 0;
    for (int64_t l = 0; l < n && st == KVC_OK; ++l) {
        const int h = static_cast<int>(l & 1);
        uint8_t* buf = stage + h * half;
        // the half is free once the decode two layers back has read it
        if (l >= 2 && hipStreamWaitEvent(cs, consumed[h], 0) != hipSuccess) { st = KVC_ERR_DEVICE; break; }
        if (hipMemcpyAsync(buf, h_streams[l], h_stream_bytes[l], hipMemcpyHostToDevice, cs) != hipSuccess ||
            hipEventRecord(copied[h], cs) != hipSuccess || hipStreamWaitEvent(s, copied[h], 0) != hipSuccess) {
            st = KVC_ERR_DEVICE;
            break;
        }
        const uint8_t* mu = static_cast<const uint8_t*>(d_mu) + uint64_t(l) * mu_stride;
        const uint8_t* sg = reinterpret_cast<const uint8_t*>(d_sigma) + uint64_t(l) * sigma_stride;
        uint8_t* out = static_cast<uint8_t*>(d_kv_out) + uint64_t(l) * kv_stride;
        // the header is read in host memory: no device round trip
        st = decode_launch(h_streams[l], buf, h_stream_bytes[l], mu, mu_stride, reinterpret_cast<const float*>(sg),
                           sigma_stride, d_prefix, prefix_bytes, out, kv_stride, nullptr,
                           ws + uint64_t(l) * KVC_DECODE_WORKSPACE_BYTES, KVC_DECODE_WORKSPACE_BYTES, stream, nullptr);
        if (st != KVC_OK) {
            if (h_failed) *h_failed = l;
            break;
        }
        if (hipEventRecord(consumed[h], s) != hipSuccess) st = KVC_ERR_DEVICE;
        ++queued;
    }
    // whatever was queued finishes before the events go and the statuses are read
    if (hipStreamSynchronize(s) != hipSuccess || hipStreamSynchronize(cs) != hipSuccess) st = KVC_ERR_DEVICE;
    for (int i = 0; i < 2; ++i) {
        if (copied[i]) (void)hipEventDestroy(copied[i]);
        if (consumed[i]) (void)hipEventDestroy(consumed[i]);
    }
    for (int64_t l = 0; l < queued && st == KVC_OK; ++l) {
        const int ls = kvc_decode_result(ws + uint64_t(l) * KVC_DECODE_WORKSPACE_BYTES, stream, nullptr);
        if (ls != KVC_OK) {
            st = ls;
            if (h_failed) *h_failed = l;
        }
    }
    return st;
}

int kvc_decode_paged(const void* h_header, const void* d_in, uint64_t in_bytes, const void* d_mu, uint64_t mu_bytes,
                     const float* d_sigma, uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                     const kvc_paged_kv* h_paged, void* d_workspace, uint64_t workspace_bytes, void* stream,
                     kvc_decode_info* h_info) {
    if (!h_paged) return KVC_ERR_INVALID;
    const int st = decode_launch(h_header, d_in, in_bytes, d_mu, mu_bytes, d_sigma, sigma_bytes, d_prefix,
                                 prefix_bytes, nullptr, 0, h_paged, d_workspace, workspace_bytes, stream,
                                 h_info ? h_info->stage_ms : nullptr);
    if (st != KVC_OK) return st;
    return kvc_decode_result(d_workspace, stream, h_info);
}

int kvc_calibrate_sigma(const void* d_kv, const void* d_mu, int32_t kv_dtype, int32_t mu_dtype, int64_t reps,
                        int64_t planes, int64_t tokens, int64_t channels, float sigma_floor, float* d_sigma_out,
                        void* d_workspace, uint64_t workspace_bytes, void* stream) {
    return kvc_calibrate_sigma_blocks(d_kv, d_mu, kv_dtype, mu_dtype, reps, planes, tokens, channels, 0, sigma_floor,
                                      d_sigma_out, d_workspace, workspace_bytes, stream);
}

int kvc_calibrate_sigma_blocks(const void* d_kv, const void* d_mu, int32_t kv_dtype, int32_t mu_dtype, int64_t reps,
                               int64_t planes, int64_t tokens, int64_t channels, int64_t block_tokens,
                               float sigma_floor, float* d_sigma_out, void* d_workspace, uint64_t workspace_bytes,
                               void* stream) {
    if (!d_kv || !d_mu || !d_sigma_out || !kv_dtype_ok(kv_dtype) || !mu_dtype_ok(mu_dtype)) return KVC_ERR_INVALID;
    if (block_tokens < 0) return KVC_ERR_INVALID;
    if (!data_aligned(kv_dtype, mu_dtype, d_kv, d_mu, d_sigma_out, nullptr)) return KVC_ERR_INVALID;
    if (reps < 1 || planes < 1 || tokens < 1 || channels < 64 || channels % 64) return KVC_ERR_INVALID;
    if (reps > kMaxScalars || planes > kMaxScalars || tokens > kMaxScalars || channels > kMaxScalars)
        return KVC_ERR_INVALID;
    if (reps * tokens > kMaxScalars / channels || reps * tokens * channels > kMaxScalars / planes)
        return KVC_ERR_INVALID;
    const int64_t n_blocks = (block_tokens == 0 || block_tokens >= tokens) ? 1 : (tokens + block_tokens - 1) / block_tokens;
    if (planes * n_blocks * (channels / 64) > 0x7FFFFFFF) return KVC_ERR_INVALID;
    if (!(sigma_floor > 0.0f) || !(sigma_floor <= FLT_MAX)) return KVC_ERR_INVALID;
    // partial sums: one CalibPart per (split, plane, block, channel), at most 64 splits
    static_assert(sizeof(kvc::CalibPart) * kvc::kCalibSplitsMax == 1024, "workspace formula");
    if (!d_workspace || !aligned(d_workspace, 256) || planes * n_blocks * channels > kMaxScalars / 1024 ||
        workspace_bytes < KVC_CALIBRATE_WORKSPACE_BYTES(planes * n_blocks, channels))
        return KVC_ERR_INVALID;
    return finish(kvc::launch_calibrate(d_kv, d_mu, kv_dtype, mu_dtype, reps, planes, tokens, channels,
                                        n_blocks == 1 ? 0 : block_tokens, sigma_floor, d_sigma_out,
                                        static_cast<kvc::CalibPart*>(d_workspace), static_cast<hipStream_t>(stream)));
}

int kvc_calibrate_sigma_rate(const void* d_kv, const void* d_mu, int32_t kv_dtype, int32_t mu_dtype, int64_t reps,
                             int64_t planes, int64_t tokens, int64_t channels, int64_t block_tokens, float sigma_floor,
                             uint32_t w_narrow_bp, uint32_t w_wide_bp, uint32_t narrow_dof, const uint32_t* d_prefix,
                             float* d_sigma_out, void* d_workspace, uint64_t workspace_bytes, void* stream) {
    uint32_t tn, tw, te;
    if (!budgets(kv_dtype, w_narrow_bp, w_wide_bp, &tn, &tw, &te) || (te && !d_prefix) || !aligned(d_prefix, 4))
        return KVC_ERR_INVALID;
    if (narrow_dof > uint32_t(kvc::kNarrowDofMax)) return KVC_ERR_INVALID;
    // every candidate sigma must be a valid sigma of the format
    if (!(sigma_floor >= 0x1p-96f) || !(sigma_floor <= 0x1p96f)) return KVC_ERR_INVALID;
    if (block_tokens < 0 || tokens < 1 || planes < 1 || channels < 64) return KVC_ERR_INVALID;
    const int64_t n_blocks = (block_tokens == 0 || block_tokens >= tokens) ? 1 : (tokens + block_tokens - 1) / block_tokens;
    if (planes > kMaxScalars / n_blocks || planes * n_blocks > kMaxScalars / channels) return KVC_ERR_INVALID;
    const uint64_t n = uint64_t(planes * n_blocks) * uint64_t(channels);
    const uint64_t rms_bytes = KVC_CALIBRATE_WORKSPACE_BYTES(planes * n_blocks, channels);
    const uint64_t cost_bytes = n * uint64_t(kvc::kRateSteps) * uint64_t(kvc::kCalibSplitsMax) * 8u;
    if (!d_workspace || workspace_bytes < KVC_CALIBRATE_RATE_WORKSPACE_BYTES(planes * n_blocks, channels))
        return KVC_ERR_INVALID;
    static_assert(kvc::kRateSteps * kvc::kCalibSplitsMax * 8 == 12800, "workspace formula");
    int st = kvc_calibrate_sigma_blocks(d_kv, d_mu, kv_dtype, mu_dtype, reps, planes, tokens, channels, block_tokens,
                                        sigma_floor, d_sigma_out, d_workspace, rms_bytes, stream);
    if (st != KVC_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const kvc::PhiTables phi = kvc::device_phi_tables(&e, narrow_dof);
    if (e != hipSuccess) return KVC_ERR_DEVICE;
    uint8_t* ws = static_cast<uint8_t*>(d_workspace);
    auto* part = reinterpret_cast<unsigned long long*>(ws + rms_bytes);
    auto* table = reinterpret_cast<uint32_t*>(ws + round_up(rms_bytes + cost_bytes, 256));
    if ((e = kvc::launch_coder_tables(phi, tn, tw, table, nullptr, s)) != hipSuccess) return KVC_ERR_DEVICE;
    return finish(kvc::launch_rate_fit(d_kv, d_mu, kv_dtype, mu_dtype, reps, planes, tokens, channels,
                                       n_blocks == 1 ? 0 : block_tokens, sigma_floor, table,
                                       te ? d_prefix : phi.zero, d_sigma_out, part, s));
}

int kvc_calibrate_split(const void* d_kv, const void* d_mu, int32_t kv_dtype, int32_t mu_dtype, int64_t reps,
                        int64_t planes, int64_t tokens, int64_t channels, int64_t block_tokens, const float* d_sigma,
                        uint32_t w_narrow_bp, uint32_t w_wide_bp, uint32_t narrow_dof, const uint32_t* d_prefix,
                        uint32_t* d_split_out, void* d_workspace, uint64_t workspace_bytes, void* stream) {
    uint32_t tn, tw, te;
    if (!budgets(kv_dtype, w_narrow_bp, w_wide_bp, &tn, &tw, &te) || !mu_dtype_ok(mu_dtype) || (te && !d_prefix))
        return KVC_ERR_INVALID;
    if (narrow_dof > uint32_t(kvc::kNarrowDofMax)) return KVC_ERR_INVALID;
    if (!d_kv || !d_mu || !d_sigma || !d_split_out || !d_workspace) return KVC_ERR_INVALID;
    if (!data_aligned(kv_dtype, mu_dtype, d_kv, d_mu, d_sigma, d_prefix) || !aligned(d_split_out, 4) ||
        !aligned(d_workspace, 256))
        return KVC_ERR_INVALID;
    if (reps < 1 || block_tokens < 0 || tokens < 1 || planes < 1 || channels < 64 || channels % 64)
        return KVC_ERR_INVALID;
    if (planes > kMaxScalars / channels || reps > kMaxScalars / (planes * channels) ||
        tokens > kMaxScalars / (reps * planes * channels))
        return KVC_ERR_INVALID;
    // one workgroup per (plane, 64-channel group); the workspace size formula in range
    if (planes * (channels / 64) > 0x7FFFFFFF || planes * channels > kMaxScalars / 8192) return KVC_ERR_INVALID;
    if (workspace_bytes < KVC_CALIBRATE_SPLIT_WORKSPACE_BYTES(planes, channels)) return KVC_ERR_INVALID;
    static_assert(kvc::kSplitSteps * kvc::kCalibSplitsMax * 8 == 8192, "workspace formula");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const kvc::PhiTables phi = kvc::device_phi_tables(&e, narrow_dof);
    if (e != hipSuccess) return KVC_ERR_DEVICE;
    kvc::SplitArgs sp;
    sp.a = phi.a;
    sp.b = phi.b;
    sp.t_all = static_cast<uint32_t>((uint64_t(1) << kLog2M) - alphabet(kv_dtype));
    sp.w_gauss = w_narrow_bp + w_wide_bp;
    return finish(kvc::launch_split_fit(d_kv, d_mu, kv_dtype, mu_dtype, reps, planes, tokens, channels,
                                        block_tokens >= tokens ? 0 : block_tokens, d_sigma, sp, tn + tw,
                                        te ? d_prefix : phi.zero, d_split_out,
                                        static_cast<unsigned long long*>(d_workspace), s));
}

int kvc_build_marginal(const void* d_samples, int32_t dtype, uint64_t n, uint32_t w_narrow_bp,
                       uint32_t w_wide_bp, uint32_t* d_prefix_out, void* stream) {
    uint32_t tn, tw, te;
    if (!d_prefix_out || !budgets(dtype, w_narrow_bp, w_wide_bp, &tn, &tw, &te)) return KVC_ERR_INVALID;
    if (n > 0 && !d_samples) return KVC_ERR_INVALID;
    if (!aligned(d_samples, dtype == KVC_BF16 ? 2 : 1) || !aligned(d_prefix_out, 4)) return KVC_ERR_INVALID;
    if (n >= (uint64_t(1) << 32) - (uint64_t(1) << 16)) return KVC_ERR_INVALID;
    return finish(kvc::launch_marginal(d_samples, dtype, n, te, d_prefix_out, static_cast<hipStream_t>(stream)));
}

int kvc_estimate_bits(const kvc_params* p, const void* d_kv, const void* d_mu, const float* d_sigma,
                      const uint32_t* d_prefix, double* h_bits_out, void* d_workspace, uint64_t workspace_bytes,
                      void* stream) {
    ChunkGeom g;
    if (!params_geometry(p, &g) || !d_kv || !d_mu || !d_sigma || !h_bits_out || !d_workspace)
        return KVC_ERR_INVALID;
    if (workspace_bytes < KVC_ESTIMATE_WORKSPACE_BYTES) return KVC_ERR_CAPACITY;
    if (!data_aligned(p->kv_dtype, p->mu_dtype, d_kv, d_mu, d_sigma, d_prefix) || !aligned(d_workspace, 8))
        return KVC_ERR_INVALID;
    uint32_t tn, tw, te;
    if (!budgets(p->kv_dtype, p->w_narrow_bp, p->w_wide_bp, &tn, &tw, &te)) return KVC_ERR_INVALID;
    if (te && !d_prefix) return KVC_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const kvc::PhiTables phi = kvc::device_phi_tables(&e, p->narrow_dof);
    if (e != hipSuccess) return KVC_ERR_DEVICE;
    Control* ctl = static_cast<Control*>(d_workspace);
    if ((e = kvc::launch_clear_control(ctl, s)) != hipSuccess) return KVC_ERR_DEVICE;
    kvc::EstimateArgs a;
    a.geom = g;
    a.kv = d_kv;
    a.mu = d_mu;
    a.sigma = d_sigma;
    a.prefix = te ? d_prefix : phi.zero;
    a.tn = tn;
    a.tw = tw;
    a.te = te;
    a.w_narrow_bp = p->w_narrow_bp;
    a.w_wide_bp = p->w_wide_bp;
    a.narrow_dof = p->narrow_dof;
    a.phi = phi;
    a.split = split_args(p->channel_split, g, d_sigma, p->kv_dtype, p->w_narrow_bp, p->w_wide_bp, phi);
    a.ctl = ctl;
    if ((e = kvc::launch_estimate(a, p->kv_dtype, p->mu_dtype, s)) != hipSuccess) return KVC_ERR_DEVICE;
    Control host;
    if ((e = hipMemcpyAsync(&host, ctl, sizeof(host), hipMemcpyDeviceToHost, s)) != hipSuccess) return KVC_ERR_DEVICE;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return KVC_ERR_DEVICE;
    if (host.flags & kvc::kFlagBadSigma) return KVC_ERR_INVALID;
    const double n = static_cast<double>(g.planes) * static_cast<double>(g.tokens) * static_cast<double>(g.channels);
    h_bits_out[0] = host.bits[0] / n;
    h_bits_out[1] = host.bits[1] / n;
    return KVC_OK;
}

int kvc_cdf_table(int32_t kv_dtype, int32_t mu_dtype, uint32_t w_narrow_bp, uint32_t w_wide_bp, uint32_t narrow_dof,
                  const void* d_mu, const float* d_sigma, int64_t pairs, const uint32_t* d_prefix, uint32_t* d_out,
                  void* stream) {
    uint32_t tn, tw, te;
    if (!mu_dtype_ok(mu_dtype) || !budgets(kv_dtype, w_narrow_bp, w_wide_bp, &tn, &tw, &te)) return KVC_ERR_INVALID;
    if (narrow_dof > uint32_t(kvc::kNarrowDofMax)) return KVC_ERR_INVALID;
    if (pairs < 1 || pairs > (int64_t(1) << 24) || !d_mu || !d_sigma || !d_out) return KVC_ERR_INVALID;
    if (te && !d_prefix) return KVC_ERR_INVALID;
    if (!data_aligned(kv_dtype, mu_dtype, nullptr, d_mu, d_sigma, d_prefix) || !aligned(d_out, 4))
        return KVC_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const kvc::PhiTables phi = kvc::device_phi_tables(&e, narrow_dof);
    if (e != hipSuccess) return KVC_ERR_DEVICE;
    // sigma is checked on the host, a block at a time
    bool ok = true;
    float hs[1024];
    for (int64_t i0 = 0; i0 < pairs && ok; i0 += 1024) {
        const int64_t m = (pairs - i0 < 1024) ? pairs - i0 : 1024;
        e = hipMemcpyAsync(hs, d_sigma + i0, sizeof(float) * static_cast<size_t>(m), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return KVC_ERR_DEVICE;
        for (int64_t i = 0; i < m; ++i) {
            const float sg = hs[i];
            if (!(sg >= 0x1p-96f && sg <= 0x1p96f)) ok = false;
        }
    }
    if (!ok) return KVC_ERR_INVALID;
    e = kvc::launch_cdf_table(kv_dtype, mu_dtype, tn, tw, d_mu, d_sigma, pairs, te ? d_prefix : phi.zero, d_out,
                              phi, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return finish(e);
}

}  // extern "C"
