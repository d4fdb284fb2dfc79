/*
 * kvc.h -- C ABI of libkvc, a lossless KV-cache entropy coder for MI355X (gfx950).
 *
 * The method ("speculative KV coding"): both ends of a KV transfer rebuild a
 * predictor mean mu and a frozen, calibrated per-(kv, head, channel) sigma;
 * every KV scalar is arithmetic-coded under the mixture
 *     q = 0.95 N(mu, sigma^2) + 0.03 N(mu, (3 sigma)^2) + 0.02 p_hat,
 * p_hat being the empirical marginal over the BF16 (or e4m3) alphabet, and
 * the decoder rebuilds KV exactly from the bits and (mu, sigma).
 * Sources: wiki page "Speculative KV Coding" (aisparkup.com), sections
 * "pipeline", "predictor choice" and "mixture distribution"; blog post
 * "推测性KV编码：用预测模型实现缓存无损压缩4倍" (blog.hotdry.top), sections
 * "engineering choice of predictor" and "application scenarios and
 * deployment parameters".
 *
 * The byte stream is format KVC-1: integer mixture CDF with total 2^31 and
 * every frequency >= 1, 64-bit-state rANS with 16-bit words, 64 interleaved
 * lanes (one per channel) per chunk of up to chunk_tokens tokens, a chunk
 * directory for random access, and a checksum of the side information.
 *
 * Conventions for every call:
 *   - Pointers named d_* are DEVICE pointers owned by the caller; pointers
 *     named h_* are HOST pointers.  The library never allocates memory and
 *     never frees caller memory; scratch comes from a caller workspace.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is queued on it; calls that return a host value synchronise
 *     that stream once before returning; the *_async calls queue the work
 *     and return at once, their outcome read later by the *_result call
 *     (one synchronisation), so that many calls can be queued, on one stream
 *     or several, with no host round trip between them.
 *   - Layouts are row-major: KV and mu are [planes][tokens][channels] with
 *     channels fastest; sigma is [planes][channels] float32; the marginal
 *     prefix is uint32[N + 1] (N = 65536 for bf16, 256 for e4m3).
 *   - Every call returns a kvc_status; no exception crosses the ABI.  On an
 *     error, outputs are undefined (but never written out of bounds).
 *   - Concurrent calls on different streams are safe (each with its own
 *     workspace).  The state the library keeps, per device, lives in static
 *     device arrays (no allocation): the base CDF tables, copied on first
 *     use, and the mixture and decoder tables of every (weights, narrow
 *     part) a process uses (up to 8), built on first use by a kernel on the
 *     calling stream, which that first call synchronises; all of them are
 *     only read afterwards.  kvc_decode_noalloc's scratch is the one
 *     exception, see there.
 *   - Graph capture: once a call with the same weights and narrow part has
 *     run on the device (so its tables exist), kvc_encode without a size
 *     pointer and kvc_decode_async only launch kernels (the control block is
 *     cleared by a kernel, not a memset) and may be captured in a HIP graph
 *     and replayed; their *_result calls synchronise and stay outside it.
 */
#ifndef KVC_H
#define KVC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_INVALID = -1,   /* bad argument, shape, dtype, weights or sigma   */
    KVC_ERR_CAPACITY = -2,  /* output buffer or workspace too small           */
    KVC_ERR_CORRUPT = -3,   /* stream malformed or damaged                    */
    KVC_ERR_MISMATCH = -4,  /* sigma / prefix differ from the encoder's       */
    KVC_ERR_DEVICE = -5     /* a HIP call failed                              */
} kvc_status;

enum { KVC_BF16 = 0, KVC_E4M3 = 1, KVC_F32 = 2 };   /* E4M3 = OCP float8 e4m3fn */

#define KVC_HEADER_BYTES 128
#define KVC_DECODE_WORKSPACE_BYTES 917504   /* control block, escape tables, coder tables */
#define KVC_ESTIMATE_WORKSPACE_BYTES 256
#define KVC_ENCODE_STAGES 2
#define KVC_DECODE_STAGES 2

/* Optional per-call measurements (pass NULL to skip; costs a few events). */
typedef struct kvc_encode_info {
    float stage_ms[KVC_ENCODE_STAGES];  /* GPU time of: side-information checksum
                                           and per-call tables, coding kernel
                                           (which also places every chunk at its
                                           final offset)                          */
} kvc_encode_info;

typedef struct kvc_decode_info {
    float stage_ms[KVC_DECODE_STAGES];  /* GPU time of: side-information checksum
                                           and per-call tables, decoding kernel   */
    uint32_t reserved;
    uint64_t fallback_symbols;          /* symbols not found by the aim: slots in
                                           the floor-and-escape range (looked up
                                           through the bucket table) plus
                                           Gaussian slots whose aimed cell did not
                                           hold the target                        */
} kvc_decode_info;

typedef struct kvc_params {
    int32_t kv_dtype;        /* KVC_BF16 or KVC_E4M3                               */
    int32_t mu_dtype;        /* KVC_BF16 or KVC_F32                                */
    uint32_t w_narrow_bp;    /* weight of N(mu, sigma^2), basis points: 9500        */
    uint32_t w_wide_bp;      /* weight of N(mu, (3 sigma)^2), basis points: 300     */
                             /* the escape part p_hat gets 10000 - both; (10000, 0)
                                is a single Gaussian and needs no prefix table     */
    uint32_t chunk_tokens;   /* tokens per chunk; 0 = the library's default:
                                of the lengths ceil(tokens / k) between 1024
                                and 256 (or tokens, if fewer), the one with
                                the least rounds x (length + 9), a round being
                                8,192 chunks (one wave each) at once (with
                                sigma blocks: of the divisors of the block
                                length in that range, else the largest
                                divisor below it); chunk_tokens * channels
                                < 2^29                                           */
    uint32_t sigma_block_tokens; /* position-aware sigma ([blog] "limitations and
                                future directions"): 0 = one sigma per (plane,
                                channel), d_sigma [planes][channels]; B > 0 =
                                one sigma per (plane, block of B tokens,
                                channel), d_sigma [planes][ceil(tokens / B)]
                                [channels], token t using block t / B.  B must
                                be a multiple of chunk_tokens unless B >=
                                tokens (KVC_ERR_INVALID).  Recorded in the
                                stream header.                                 */
    uint32_t narrow_dof;     /* the narrow part's shape ([wiki] "future directions",
                                [blog] "limitations and future directions": a
                                better residual model): 0 = the pages'
                                N(mu, sigma^2); nu = 1..16 = Student's t with nu
                                degrees of freedom, location mu, scale sigma,
                                truncated to +-24 sigma and renormalised there.
                                The wide part and p_hat are unchanged.
                                Recorded in the stream header.                 */
    uint32_t channel_split;  /* per-channel mixture weights ([wiki] "future directions",
                                [blog] "limitations and future directions": a
                                better residual model): 0 = the call's weights on
                                every channel; 1 = each (plane, channel) has its
                                own narrow weight w_c in basis points, 0 ..
                                w_narrow_bp + w_wide_bp, its wide weight
                                w_narrow_bp + w_wide_bp - w_c (the escape weight
                                stays the call's).  The weights are side
                                information: the sigma buffer (d_sigma) holds
                                the sigma words followed by planes x channels
                                uint32 weights, [planes][channels], and every
                                call that takes it (encode, decode, reload,
                                estimate) reads both; sigma_bytes / strides
                                count both.  The coder's budgets are T_n(c) =
                                min(floor(T w_c / 10^4), T_n + T_w), T_w(c) =
                                T_n + T_w - T_n(c) with T = 2^31 - N.  A weight
                                above w_narrow_bp + w_wide_bp: KVC_ERR_INVALID.
                                Recorded in the stream header; covered by the
                                side-information checksum.                     */
    int64_t planes;          /* G = layers * 2 * batch * kv_heads                  */
    int64_t tokens;          /* T                                                  */
    int64_t channels;        /* D, a positive multiple of 64                       */
} kvc_params;

/* Stream format version written and accepted: 4 (Gaussian and floor-and-escape
   slots in separate ranges of the coder; the CDF argument q = floor(z * 2^24);
   the header's bytes [92, 96) hold the CRC-32 of its bytes [0, 92)). */
int kvc_version(void);

/* Human-readable name of a status code (static string). */
const char* kvc_status_string(int status);

/*
 * The format's two standard-normal CDF tables on the grid z_k = -24 + k/256,
 * k = 0..12288, computed on the host: h_narrow[k] = round(2^31 Phi(z_k)) and
 * h_wide[k] = round(2^31 Phi(z_k / 3)).  The mixture table the coder uses is
 * floor(T_n h_narrow[k] / 2^31) + floor(T_w h_wide[k] / 2^31).  Needs no GPU.
 * Returns KVC_ERR_INVALID for a NULL pointer.
 */
int kvc_phi_tables(uint32_t* h_narrow /* [12289] */, uint32_t* h_wide /* [12289] */);

/*
 * The narrow part's table for narrow_dof (kvc_params): narrow_dof = 0 gives
 * h_narrow of kvc_phi_tables; nu = 1..16 gives round(2^31 (F(z_k) - F(-24))
 * / (F(24) - F(-24))) for Student's t with nu degrees of freedom.  Needs no
 * GPU.  KVC_ERR_INVALID for a NULL pointer or nu > 16.
 */
int kvc_narrow_table(uint32_t narrow_dof, uint32_t* h_out /* [12289] */);

/*
 * Sizes for kvc_encode: the largest stream the call can produce (every
 * scalar at two 16-bit words, the worst case of the coder) and the workspace
 * it needs.  Host only; returns KVC_ERR_INVALID for bad parameters.
 */
int kvc_encode_sizes(const kvc_params* p, uint64_t* h_max_stream_bytes,
                     uint64_t* h_workspace_bytes);

/*
 * Encoder ([wiki] "pipeline": KV_full and (mu, sigma) go into the arithmetic
 * coder, which emits the bits).  Codes d_kv (bf16 or e4m3 bit patterns,
 * p->planes x p->tokens x p->channels of them) under the mixture around d_mu
 * with d_sigma and the marginal prefix d_prefix (NULL allowed when
 * w_narrow_bp + w_wide_bp == 10000); the buffers must hold what *p
 * describes.  Writes the stream to d_out, its length to *h_out_bytes and,
 * when h_header_out is not NULL, a host copy of its 128-byte header (what
 * kvc_decode takes) to h_header_out.  Every sigma must lie in [2^-96, 2^96],
 * else KVC_ERR_INVALID.  If the stream does not fit out_capacity the call
 * returns KVC_ERR_CAPACITY and sets *h_out_bytes to the size it needed.
 * Synchronises `stream` once.
 * h_out_bytes == NULL makes the call asynchronous: it queues the work and
 * returns KVC_OK (h_header_out and h_info must then be NULL);
 * kvc_encode_result on the same workspace gives the outcome later.
 * h_info: NULL, or receives the GPU time of each stage, measured with HIP
 * events on `stream`.
 */
int kvc_encode(const kvc_params* p, const void* d_kv, const void* d_mu,
               const float* d_sigma, const uint32_t* d_prefix, void* d_out,
               uint64_t out_capacity, uint64_t* h_out_bytes, void* h_header_out,
               void* d_workspace, uint64_t workspace_bytes, void* stream,
               kvc_encode_info* h_info);

/*
 * Outcome of the last encode queued with this workspace: synchronises
 * `stream` once, then returns the status kvc_encode would have returned and
 * fills *h_out_bytes (and, if not NULL, the 128-byte h_header_out) as it
 * would have.
 */
int kvc_encode_result(const void* d_workspace, void* stream, uint64_t* h_out_bytes,
                      void* h_header_out);

/*
 * Parse the 128-byte stream header held in HOST memory into *h_params and
 * the total stream length *h_stream_bytes.  Host only; KVC_ERR_CORRUPT if
 * the header is not a valid KVC-1 header.
 */
int kvc_stream_info(const void* h_header, uint64_t header_bytes, kvc_params* h_params,
                    uint64_t* h_stream_bytes);

/*
 * Decoder ([wiki] "pipeline": the bitstream plus (mu, sigma) give back
 * KV_full exactly).  h_header is a HOST copy of the stream's first 128
 * bytes (kvc_encode's h_header_out, or the head of a host-resident stream);
 * shape and parameters come from it, and the call checks, before anything
 * runs, that the header is a valid KVC-1 header (CRC included:
 * KVC_ERR_CORRUPT), that in_bytes is the length it gives (KVC_ERR_CORRUPT),
 * and that the caller's buffers hold what it describes (KVC_ERR_INVALID):
 * mu_bytes >= scalars x mu element size, sigma_bytes >= 4 x sigma words
 * (with per-channel weights, channel_split in the header: 4 x (sigma words
 * + planes x channels), the weights following sigma in d_sigma),
 * prefix_bytes >= 4 x (N + 1) when the mixture has an escape part,
 * kv_out_bytes >= scalars x KV element size.  On the device the stream's
 * own header must equal h_header (KVC_ERR_CORRUPT, nothing decoded).
 * d_in holds in_bytes of a KVC-1 stream; d_mu, d_sigma, d_prefix must be
 * the encoder's (checked through the stream's checksum: KVC_ERR_MISMATCH,
 * nothing decoded).  Writes KV bit patterns to d_kv_out
 * ([planes][tokens][channels]).  Returns KVC_ERR_CORRUPT if the stream is
 * malformed, truncated or damaged (every lane must start from a state in
 * [2^47, 2^63), end in the initial state and consume exactly its chunk).
 * Workspace: KVC_DECODE_WORKSPACE_BYTES, 256-byte aligned.  Synchronises
 * `stream` once (the status read).  h_info: NULL, or receives the stage
 * times and the number of symbols the aim did not find.
 */
int kvc_decode(const void* h_header, const void* d_in, uint64_t in_bytes,
               const void* d_mu, uint64_t mu_bytes, const float* d_sigma,
               uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
               void* d_kv_out, uint64_t kv_out_bytes, void* d_workspace,
               uint64_t workspace_bytes, void* stream, kvc_decode_info* h_info);

/*
 * kvc_decode without its synchronisation: the host-side checks run and
 * return their status at once; the work is queued on `stream` and its
 * outcome is read later by kvc_decode_result on the same workspace (which
 * must not be reused before that).
 */
int kvc_decode_async(const void* h_header, const void* d_in, uint64_t in_bytes,
                     const void* d_mu, uint64_t mu_bytes, const float* d_sigma,
                     uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                     void* d_kv_out, uint64_t kv_out_bytes, void* d_workspace,
                     uint64_t workspace_bytes, void* stream);

/*
 * kvc_decode for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument and no allocation of any kind.  Its scratch is a
 * fixed array of KVC_NOALLOC_SCRATCH_BYTES in device memory that the
 * library holds on every device it runs on until the process ends; the
 * decoder's scratch does not grow with the stream, so every stream
 * kvc_decode accepts fits (a layout needing more would be refused with
 * KVC_ERR_CAPACITY).  Arguments, checks, output and statuses as
 * kvc_decode; synchronises `stream` once.  Every call on one device
 * shares that device's scratch (cleared by the call where it must start at
 * zero): calls that overlap on one device, from several threads or on
 * several streams, race, and the caller must serialise them.
 */
#define KVC_NOALLOC_SCRATCH_BYTES 917504
int kvc_decode_noalloc(const void* h_header, const void* d_in, uint64_t in_bytes,
                       const void* d_mu, uint64_t mu_bytes, const float* d_sigma,
                       uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                       void* d_kv_out, uint64_t kv_out_bytes, void* stream);

/*
 * Host-offload reload ([wiki] "use scenarios": KV offloaded from DRAM to
 * VRAM; [blog] "application scenarios and deployment parameters": KV moved
 * over PCIe in compressed form, decoding fast enough to keep up with the
 * transfer).  Decodes n KVC-1 streams held in HOST memory (h_streams[l],
 * h_stream_bytes[l] bytes; pinned memory, e.g. from hipHostMalloc, lets the
 * copies run asynchronously) into device memory, one stream per layer: the
 * copy of stream l + 1 to the device runs on copy_stream while stream l is
 * decoded on `stream`, through two halves of d_staging (each 256-byte
 * aligned, staging_bytes / 2 rounded down to 256: every stream must fit one,
 * else KVC_ERR_CAPACITY).  Stream l decodes with the mu at d_mu + l x
 * mu_stride, the sigma at d_sigma + l x sigma_stride bytes and the shared
 * d_prefix, into d_kv_out + l x kv_stride; each stride is also the bytes
 * available there, checked against the stream's header as kvc_decode checks
 * its buffers.  Every layer's header (read in host memory) and buffers
 * pass these checks before anything is copied or launched.  Workspace: n x
 * KVC_DECODE_WORKSPACE_BYTES, 256-byte aligned (one decode workspace per
 * layer).  Synchronises `stream` and `copy_stream` once at the end and
 * returns the first failing layer's status (KVC_OK when all decode), its
 * index in *h_failed (-1 if none; may be NULL).
 */
int kvc_reload(int64_t n, const void* const* h_streams, const uint64_t* h_stream_bytes,
               const void* d_mu, uint64_t mu_stride, const float* d_sigma, uint64_t sigma_stride,
               const uint32_t* d_prefix, uint64_t prefix_bytes, void* d_kv_out, uint64_t kv_stride,
               void* d_staging, uint64_t staging_bytes, void* d_workspace, uint64_t workspace_bytes,
               void* stream, void* copy_stream, int64_t* h_failed);

/*
 * Outcome of the last decode queued with this workspace: synchronises
 * `stream` once and returns the status kvc_decode would have returned;
 * h_info (may be NULL) receives the fallback count (stage times are -1).
 */
int kvc_decode_result(const void* d_workspace, void* stream, kvc_decode_info* h_info);

/*
 * Paged output for kvc_decode_paged: the serving engine's KV cache as page
 * pools.  Pool p = 2 * layer + kv (K then V of each layer) is laid out
 * [num_pages][page_tokens][heads][channels] in the stream's KV dtype; the
 * stream's planes are ordered (layer, kv, batch, head), so planes = layers *
 * 2 * batch * heads; token t of sequence b lives in page
 * block_table[b * max_pages + t / page_tokens], row t % page_tokens.
 */
typedef struct kvc_paged_kv {
    void* const* d_pools;          /* device array of n_pools pool base pointers      */
    const int32_t* d_block_table;  /* device [batch][max_pages] physical page numbers */
    int64_t n_pools;               /* entries of d_pools: layers * 2                  */
    uint64_t pool_bytes;           /* bytes of every pool, >= num_pages x page_tokens
                                      x heads x channels x KV element size           */
    int64_t batch;                 /* sequences                                       */
    int64_t heads;                 /* KV heads per pool row                           */
    int64_t max_pages;             /* row stride of the table, >= ceil(tokens /
                                      page_tokens)                                    */
    int64_t num_pages;             /* pages in every pool, < 2^31                    */
    uint32_t page_tokens;          /* tokens per page                                 */
    uint32_t reserved;             /* 0                                               */
} kvc_paged_kv;

/*
 * Decoder fused into the consumer's layout ([blog] "application scenarios
 * and deployment parameters": a compressed prefix-cache entry is
 * decompressed when it is hit, and decoding has to keep up with the rate
 * at which the cache is consumed).  As kvc_decode, but every decoded row
 * goes straight to its page of the paged KV cache described by *h_paged
 * (host struct; its pointers are device pointers) instead of a contiguous
 * [planes][tokens][channels] array: no second pass over the KV.  Rows of
 * pages the table does not name are left untouched.  KVC_ERR_INVALID if the
 * planes are not n_pools x batch x heads with n_pools even, the table is
 * too narrow, a page holds 2^32 bytes or more, pool_bytes is short of
 * num_pages pages, or (checked on the device before the decode) an entry of
 * the columns the tokens use lies outside [0, num_pages): then nothing is
 * written.  Header and buffer checks as kvc_decode.
 */
int kvc_decode_paged(const void* h_header, const void* d_in, uint64_t in_bytes,
                     const void* d_mu, uint64_t mu_bytes, const float* d_sigma,
                     uint64_t sigma_bytes, const uint32_t* d_prefix, uint64_t prefix_bytes,
                     const kvc_paged_kv* h_paged, void* d_workspace, uint64_t workspace_bytes,
                     void* stream, kvc_decode_info* h_info);

/*
 * Sigma calibration ([wiki] "predictor choice": per-(kv, head, channel)
 * variance calibrated on data, then frozen; [blog] "deployment parameters":
 * 128 sequences of 1024 tokens).  d_kv and d_mu are [reps][planes][tokens]
 * [channels]; writes d_sigma_out[planes][channels] = max(sigma_floor,
 * sqrt(mean over reps and tokens of (kv - mu)^2)), accumulated in float64
 * in a fixed order (deterministic); residuals that are not finite are left
 * out, and a channel with none left gets the floor.  d_workspace (256-byte
 * aligned) holds the float64 partial sums: at least
 * KVC_CALIBRATE_WORKSPACE_BYTES(planes, channels) bytes.  Returns
 * KVC_ERR_INVALID for bad shapes, a non-positive floor or a short
 * workspace.  Does not synchronise.
 */
#define KVC_CALIBRATE_WORKSPACE_BYTES(planes, channels) \
    ((uint64_t)(planes) * (uint64_t)(channels) * 1024u)
int kvc_calibrate_sigma(const void* d_kv, const void* d_mu, int32_t kv_dtype,
                        int32_t mu_dtype, int64_t reps, int64_t planes, int64_t tokens,
                        int64_t channels, float sigma_floor, float* d_sigma_out,
                        void* d_workspace, uint64_t workspace_bytes, void* stream);

/*
 * Position-aware sigma calibration ([blog] "limitations and future
 * directions": a static per-channel sigma ignores how the residual changes
 * with position).  As kvc_calibrate_sigma, per block of block_tokens
 * tokens: d_sigma_out[planes][n_blocks][channels] with n_blocks =
 * ceil(tokens / block_tokens), block j taking the mean over reps and the
 * tokens [j * block_tokens, min((j + 1) * block_tokens, tokens)).
 * block_tokens = 0 or >= tokens gives one block (the per-plane sigma).
 * Workspace: KVC_CALIBRATE_WORKSPACE_BYTES(planes * n_blocks, channels).
 */
int kvc_calibrate_sigma_blocks(const void* d_kv, const void* d_mu, int32_t kv_dtype,
                               int32_t mu_dtype, int64_t reps, int64_t planes, int64_t tokens,
                               int64_t channels, int64_t block_tokens, float sigma_floor,
                               float* d_sigma_out, void* d_workspace, uint64_t workspace_bytes,
                               void* stream);

/*
 * Rate-fitted sigma ([blog] "limitations and future directions": better
 * residual models; [blog] "engineering choice of predictor": sigma measured
 * once on held-out data).  The RMS of kvc_calibrate_sigma_blocks is the base;
 * one outlier in a few hundred inflates it.  For each (plane, block, channel)
 * this call keeps, of the candidates max(sigma_floor, base * (1 - j/32)),
 * j = 0..24 (float32 products), the one under which the held-out data cost
 * the fewest bits in the coder's own integer model: the sum over the data
 * of 2^16 (31 - e) - L[m] for each frequency f = C(s+1) - C(s), with e the
 * top bit of f, m the 8 bits below it and L[m] = round(2^16 log2(1 + m/256));
 * the first j on a tie (an integer sum: deterministic).  The mixture
 * weights, the narrow part (narrow_dof, as in kvc_params) and d_prefix
 * (NULL allowed for a single Gaussian) are the ones the data will be coded
 * with.  sigma_floor in [2^-96, 2^96].  Output and
 * block_tokens as kvc_calibrate_sigma_blocks.  Workspace (256-byte aligned):
 * KVC_CALIBRATE_RATE_WORKSPACE_BYTES(planes * n_blocks, channels).  Does
 * not synchronise.
 */
#define KVC_CALIBRATE_RATE_WORKSPACE_BYTES(rows, channels) \
    ((uint64_t)(rows) * (uint64_t)(channels) * (1024u + 12800u) + 65536u)
int kvc_calibrate_sigma_rate(const void* d_kv, const void* d_mu, int32_t kv_dtype,
                             int32_t mu_dtype, int64_t reps, int64_t planes, int64_t tokens,
                             int64_t channels, int64_t block_tokens, float sigma_floor,
                             uint32_t w_narrow_bp, uint32_t w_wide_bp, uint32_t narrow_dof,
                             const uint32_t* d_prefix, float* d_sigma_out, void* d_workspace,
                             uint64_t workspace_bytes, void* stream);

/*
 * Per-channel mixture weights ([wiki] "future directions" and [blog]
 * "limitations and future directions": a better residual model; the pages'
 * 0.95 / 0.03 split is one choice for every channel, [wiki] "mixture
 * distribution").  For each (plane, channel), of the narrow weights
 * w_j = max(w_narrow_bp + w_wide_bp - 200 j, 0), j = 0..15, writes to
 * d_split_out[planes][channels] (uint32) the one under which the held-out
 * data d_kv / d_mu ([reps][planes][tokens][channels]) cost the fewest bits
 * in the coder's own integer model with that channel's budgets (the sum of
 * kvc_calibrate_sigma_rate; the first j on a tie: deterministic).  d_sigma
 * is the sigma the data will be coded with: [planes][channels], or per
 * block of block_tokens tokens [planes][ceil(tokens / block_tokens)]
 * [channels] (block_tokens = 0 or >= tokens: one block); the weights,
 * narrow_dof and d_prefix (NULL allowed for a single Gaussian) as the
 * stream will use them.  Workspace (256-byte aligned):
 * KVC_CALIBRATE_SPLIT_WORKSPACE_BYTES(planes, channels).  KVC_ERR_INVALID
 * for bad shapes or arguments.  Does not synchronise.
 */
#define KVC_CALIBRATE_SPLIT_WORKSPACE_BYTES(planes, channels) \
    ((uint64_t)(planes) * (uint64_t)(channels) * 8192u)
int kvc_calibrate_split(const void* d_kv, const void* d_mu, int32_t kv_dtype, int32_t mu_dtype,
                        int64_t reps, int64_t planes, int64_t tokens, int64_t channels,
                        int64_t block_tokens, const float* d_sigma, uint32_t w_narrow_bp,
                        uint32_t w_wide_bp, uint32_t narrow_dof, const uint32_t* d_prefix,
                        uint32_t* d_split_out, void* d_workspace, uint64_t workspace_bytes,
                        void* stream);

/*
 * Empirical marginal ([wiki] "mixture distribution": an empirical BF16
 * distribution catches extreme outliers).  d_samples holds n bit patterns
 * (bf16 or e4m3); writes the integer prefix d_prefix_out[b] =
 * floor(T_e * cum[b] / cum[N]) of the +1-smoothed histogram in value order,
 * with T_e the escape budget of the weights.  n < 2^32 - 2^16.  Does not
 * synchronise.
 */
int kvc_build_marginal(const void* d_samples, int32_t dtype, uint64_t n,
                       uint32_t w_narrow_bp, uint32_t w_wide_bp,
                       uint32_t* d_prefix_out, void* stream);

/*
 * Bits per scalar ([wiki] "core idea": the rate is the cross-entropy of the
 * model).  h_bits_out[0] = mean of -log2(f/2^31) under the integer model the
 * coder uses; h_bits_out[1] = mean -log2 q under the continuous mixture over
 * the same cells (float64, per-scalar cost capped at 64 bits).  With
 * p->channel_split = 1, d_sigma carries the per-channel weights after sigma
 * (as for kvc_encode) and each channel's weights are used.  Workspace:
 * KVC_ESTIMATE_WORKSPACE_BYTES.  Synchronises `stream` once.
 */
int kvc_estimate_bits(const kvc_params* p, const void* d_kv, const void* d_mu,
                      const float* d_sigma, const uint32_t* d_prefix, double* h_bits_out,
                      void* d_workspace, uint64_t workspace_bytes, void* stream);

/*
 * The shared CDF itself ([blog] "deployment parameters": encoder and decoder
 * must agree on it bit for bit), with the narrow part narrow_dof (as in
 * kvc_params).  For each of `pairs` (mu, sigma) pairs,
 * writes C(b) for b = 0..N to d_out[pair][N + 1].  d_mu holds `pairs`
 * values of mu_dtype, d_sigma `pairs` floats.  Synchronises `stream` once
 * (to report an invalid sigma).
 */
int kvc_cdf_table(int32_t kv_dtype, int32_t mu_dtype, uint32_t w_narrow_bp,
                  uint32_t w_wide_bp, uint32_t narrow_dof, const void* d_mu, const float* d_sigma,
                  int64_t pairs, const uint32_t* d_prefix, uint32_t* d_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
