// Host-side interface between the C ABI (kvc_api.cpp) and the kernels
// (kvc_kernels.hip): plain structs of device pointers and sizes, and the
// launch functions.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kvc {

// Status bits the kernels raise in the workspace flag word.
enum : uint32_t {
    kFlagBadSigma = 1u,
    kFlagCorrupt = 2u,
    kFlagCapacity = 4u,
    kFlagBadPage = 8u,                  // a block-table entry outside the page pool
    kFlagMismatch = 16u,                // decode: sigma / prefix checksum differs from the header's
    kFlagHeader = 32u,                  // decode: the device stream's header differs from the host copy
    kFlagStall = 64u,                   // encode: a chunk size was not published in time (never expected)
};

// Control block at the head of every workspace (cleared by a kernel),
// followed by a copy of the stream header (encode: written with the
// stream; read back by kvc_encode_result).
struct Control {
    uint32_t flags;
    uint32_t pad;
    unsigned long long side_hash;       // sum of mixed side-information words
    unsigned long long total_payload;   // payload bytes of the stream
    double bits[2];                     // estimate sums (integer model, float model)
    unsigned long long misses;          // decoder: symbols found by the fallback search
    unsigned long long reserved[2];
};
static_assert(sizeof(Control) == 64, "control block size");
constexpr uint64_t kHeaderCopyOffset = 64;           // header copy in the workspace, after Control
constexpr uint32_t kHeaderCrcOffset = 92;            // CRC-32 of header bytes [0, 92) at [92, 96)

struct ChunkGeom {
    int64_t planes, tokens, channels;
    uint32_t chunk_tokens;
    uint32_t n_tok_chunks;              // ceil(tokens / chunk_tokens)
    uint32_t n_groups;                  // channels / 64
    uint32_t sigma_tc;                  // token chunks per sigma block; 0: one sigma block per plane
    int64_t n_chunks;
    int64_t sigma_blocks;               // sigma blocks per plane (sigma is [planes][sigma_blocks][channels])
};

// Per-device Phi base tables (kTablePoints entries each).
struct PhiTables {
    const uint32_t* a;                  // round(2^31 Phi(z_k))
    const uint32_t* b;                  // round(2^31 Phi(z_k / 3))
    const uint32_t* zero;               // 65,537 zeros: the escape prefix of a model without one
};

// Per-call coder tables in global memory (launch_coder_tables), copied into
// LDS by every workgroup of the coding kernels: the mixture table (12,290
// words, padded to 12,292) and the decoder's aim table (float pairs).
constexpr uint32_t kTableWordsPadded = 12292;
constexpr uint64_t kTableBytes = 4ull * kTableWordsPadded;
constexpr uint32_t kAimFloats = 2 * 1986;          // 1985 pairs and a zero pair
constexpr uint64_t kAimBytes = 4ull * kAimFloats;

struct StreamHeader {
    uint8_t bytes[128];
};

// A per-channel split of the Gaussian budget: words[g * channels + c] is
// the narrow weight (basis points) of plane g, channel c; the kernels form
// the pair table (A[k], B[k]) in LDS from the base tables a, b and each
// lane's budgets from t_all = M - N and htot = T_n + T_w.  words null: the
// call's own weights everywhere.
struct SplitArgs {
    const uint32_t* words = nullptr;
    const uint32_t* a = nullptr;        // the narrow part's base table (kPhiPoints entries)
    const uint32_t* b = nullptr;        // the wide part's base table
    uint32_t t_all = 0;
    uint32_t w_gauss = 0;               // w_n + w_w: the largest narrow weight accepted
};

struct EncodeArgs {
    ChunkGeom geom;
    const void* kv;
    const void* mu;
    const float* sigma;
    const uint32_t* prefix;             // escape prefix; the zero table when there is no escape part
    uint32_t tn, tw;
    const uint32_t* table;              // the mixture table (launch_coder_tables)
    const uint32_t* eslots;             // bf16: the escape slot table (launch_prologue)
    uint16_t* slots;                    // per-chunk word slots, filled from the end
    uint64_t slot_words;                // words per slot (2 per scalar, multiple of 4)
    unsigned long long* status;         // [n_chunks] chunk sizes for the look-back, zeroed
    uint8_t* out;                       // the stream
    uint64_t out_capacity;
    StreamHeader header;                // the stream header but for payload size, checksum and CRC
    uint8_t* header_copy;               // the workspace's copy of the finished header
    SplitArgs split;
    Control* ctl;
};

// Decoded rows written straight into paged KV pools: pool (layer, kv) is
// [num_pages][page_tokens][heads][channels]; plane g = ((layer * 2 + kv) *
// batch + b) * heads + h keeps token t at page block_table[b][t /
// page_tokens], row t % page_tokens.
struct PagedOut {
    void* const* pools;                 // [layers * 2] pool base pointers
    const int32_t* block_table;         // [batch][max_pages]
    int64_t max_pages, num_pages;
    uint32_t page_tokens, heads;
    uint32_t batch, pad;
};

struct DecodeArgs {
    ChunkGeom geom;
    const uint8_t* payload;             // first payload byte of the stream
    const unsigned long long* directory;
    uint64_t payload_bytes;
    const void* mu;
    const float* sigma;
    const uint32_t* prefix;
    uint32_t tn, tw;
    const uint32_t* table;              // the mixture table (launch_coder_tables)
    const float* aim;                   // the aim table, kAimFloats floats
    const uint32_t* buckets;            // escape bucket table (launch_prologue)
    uint32_t bucket_shift;
    const uint32_t* ecount;             // bf16: the escape count table (launch_prologue),
                                        // with the bucket table right after it
    void* kv_out;                       // contiguous output [planes][tokens][channels], or
    PagedOut paged;                     // the paged output (launch_decode with paged = true)
    unsigned long long expect_hash;     // the header's side-information checksum
    SplitArgs split;
    Control* ctl;
};

struct EstimateArgs {
    ChunkGeom geom;
    const void* kv;
    const void* mu;
    const float* sigma;
    const uint32_t* prefix;
    uint32_t tn, tw, te;
    uint32_t w_narrow_bp, w_wide_bp;
    uint32_t narrow_dof;                // 0: Gaussian narrow part; nu: Student's t (float model)
    PhiTables phi;
    SplitArgs split;
    Control* ctl;
};

// The allocation-free decode's scratch: a fixed device array of
// kNoAllocScratchBytes per device; its device address (taken once per
// device), or null with *err set.
constexpr uint64_t kNoAllocScratchBytes = 917504;
void* noalloc_scratch(hipError_t* err);

// Phi base tables: computed once on the host, copied to each device.
constexpr int kPhiPoints = 12289;
PhiTables device_phi_tables(hipError_t* err);
void host_phi_tables(uint32_t* a, uint32_t* b);   // kPhiPoints entries each
// The narrow part's base table: Phi (narrow_dof = 0) or Student's t with
// narrow_dof = 1..kNarrowDofMax degrees of freedom, truncated to [-24, 24]
// and renormalised.  The device tables with `a` set to it.
constexpr int kNarrowDofMax = 16;
PhiTables device_phi_tables(hipError_t* err, uint32_t narrow_dof);
void host_narrow_table(uint32_t narrow_dof, uint32_t* a);   // kPhiPoints entries

hipError_t launch_clear_control(Control* ctl, hipStream_t s);
// The mixture table for budgets (tn, tw) into `table` (kTableBytes) and,
// when `aim` is not null, the decoder's aim table (kAimBytes).
hipError_t launch_coder_tables(const PhiTables& phi, uint32_t tn, uint32_t tw, uint32_t* table, float* aim,
                               hipStream_t s);
hipError_t launch_encode(const EncodeArgs& a, int kv_dtype, int mu_dtype, hipStream_t s);
// Per-call preparation in one launch (after launch_clear_control): the
// side-information checksum of sigma_words and prefix_words (and, with head
// not null, the comparison of the device stream's header with `expect`);
// the bf16 escape slot table (eslots) and/or escape count table (ecount)
// from `prefix`; the escape bucket table (buckets); zeroing n_zero words at
// zero; the check of pages_used columns of a paged decode's block table.
// Null outputs skip their part; the block counts are filled in by the launch.
struct PrologueArgs {
    const uint32_t* sigma_words = nullptr;
    uint64_t n_sigma = 0;
    const uint32_t* prefix_words = nullptr;   // the checksum's prefix words (null without an escape part)
    uint64_t n_prefix = 0;
    const uint8_t* head = nullptr;
    StreamHeader expect{};
    const uint32_t* prefix = nullptr;         // the prefix the tables read (the zero table without one)
    uint32_t htot = 0;
    uint2* eslots = nullptr;
    uint32_t* ecount = nullptr;
    uint2* buckets = nullptr;
    uint32_t n_sym = 0, bucket_shift = 0, n_buckets = 0;
    unsigned long long* zero = nullptr;
    uint64_t n_zero = 0;
    PagedOut pages{};                         // block_table null: no check
    int64_t pages_used = 0;
    Control* ctl = nullptr;
    uint32_t hash_blocks = 0, slot_blocks = 0, bucket_blocks = 0, zero_blocks = 0, page_blocks = 0;
};
hipError_t launch_prologue(PrologueArgs a, int kv_dtype, hipStream_t s);
// The mixture and aim tables of (tn, tw, narrow_dof) from the per-device
// cache, built there on first use (synchronising s once); false when the
// cache is full (then the caller builds them itself) or on an error (*err).
bool cached_coder_tables(uint32_t tn, uint32_t tw, uint32_t narrow_dof, const PhiTables& phi, hipStream_t s,
                         const uint32_t** table, const float** aim, hipError_t* err);

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int mu_dtype, bool paged, hipStream_t s);

// Bucket table of Q(b) = b + prefix[b] for the decoder's floor-and-escape
// lookup, two u32 per entry: entry j = ((s_j << 16) | pattern of s_j,
// Q(s_j)), where s_j is the largest s < n_sym with Q(s) <= j << shift
// (entries order as their symbols).
constexpr uint32_t kEscapeBucketsMax = 65538;

// Escape slot table of the bf16 alphabet, indexed by bit pattern p (s its
// ordered index): entry p = (T_n + T_w + Q(s), Q(s + 1) - Q(s)), two u32,
// so the encoder finds the start and the count of a symbol's
// floor-and-escape slots in one read.  The escape count table holds the
// count alone (one u32 per pattern) for the decoder, which needs the start
// only for slots in the floor-and-escape range, where the bucket table
// gives it.  Either output may be null.
constexpr uint64_t kEscapeSlotsBytes = 65536ull * 8;
constexpr uint64_t kEscapeCountBytes = 65536ull * 4;

// sigma calibration: float64 partial sums per (split, plane, channel)
struct CalibPart {
    double sum;
    unsigned long long used;
};
constexpr int64_t kCalibSplitsMax = 64;
int64_t calibrate_splits(int64_t reps, int64_t pairs, int64_t block);
// sigma per (plane, block of block_tokens tokens, channel); block_tokens = 0
// (or >= tokens): one block of every token
hipError_t launch_calibrate(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps,
                            int64_t planes, int64_t tokens, int64_t channels, int64_t block_tokens,
                            float sigma_floor, float* sigma_out, CalibPart* part, hipStream_t s);
// Rate-fitted sigma: sigma_io (the base on entry) becomes, per (plane,
// block, channel), the candidate max(floor, base (1 - j/32)), j < kRateSteps,
// with the least integer code length under the mixture table `table`
// (launch_coder_tables) and the escape prefix.  part: kRateSteps x splits x
// (planes x blocks x channels) u64.
constexpr int kRateSteps = 25;
hipError_t launch_rate_fit(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps, int64_t planes,
                           int64_t tokens, int64_t channels, int64_t block_tokens, float sigma_floor,
                           const uint32_t* table, const uint32_t* prefix, float* sigma_io, unsigned long long* part,
                           hipStream_t s);
// Per-channel split: out[plane][channel] becomes the candidate narrow
// weight max(w_gauss - kSplitStepBp j, 0), j < kSplitSteps, with the least
// integer code length of the held-out data under sigma (per block of
// block_tokens tokens when not 0) and the escape prefix.  part: kSplitSteps
// x splits x (planes x channels) u64.
constexpr int kSplitSteps = 16;
constexpr uint32_t kSplitStepBp = 200;
hipError_t launch_split_fit(const void* kv, const void* mu, int kv_dtype, int mu_dtype, int64_t reps, int64_t planes,
                            int64_t tokens, int64_t channels, int64_t block_tokens, const float* sigma,
                            const SplitArgs& sp, uint32_t htot, const uint32_t* prefix, uint32_t* out,
                            unsigned long long* part, hipStream_t s);
hipError_t launch_marginal(const void* samples, int dtype, uint64_t n, uint32_t te,
                           uint32_t* prefix_out, hipStream_t s);
hipError_t launch_estimate(const EstimateArgs& a, int kv_dtype, int mu_dtype, hipStream_t s);
hipError_t launch_cdf_table(int kv_dtype, int mu_dtype, uint32_t tn, uint32_t tw,
                            const void* mu, const float* sigma, int64_t pairs,
                            const uint32_t* prefix, uint32_t* out, PhiTables phi,
                            hipStream_t s);

}  // namespace kvc
