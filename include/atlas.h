/*
 * atlas.h - C ABI of the paged, folded attention library (libatlas.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes exact causal scaled-dot-product attention
 *     out = softmax(scale * q K^T + causal mask) V,   lse = log sum exp(scale * q K^T)
 * (RustAttention README, "Mathematical Framework Covered") over a paged K/V
 * cache, folding the keys page by page with an online softmax (CFR-Atlas
 * README, overview: "exact folded online-softmax attention"; ARGUS,
 * "Latency & Throughput Impact": page-by-page online softmax without a
 * concatenated K/V tensor).  Long contexts are split over pages across
 * workgroups and the partial results merged by log-sum-exp (cortiq README,
 * "split-K flash-decoding"; attnres AGENTS.md, "online softmax merge").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers unless a field says "host".
 *    Every layout is dense row-major with the shape given; the caller owns
 *    all memory.  The library never allocates device memory; temporary
 *    storage comes from the caller's `workspace`.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Buffers must stay valid until the stream's work completes.
 *  - Every argument check runs on the host before anything is launched, so a
 *    call that returns an error has written nothing (CFR-Atlas README, test
 *    list: rejection of invalid configs and ranges, transactional behaviour).
 *    Launch failures return ATLAS_EDEVICE; faults surface at the caller's
 *    next synchronisation.
 *  - Device-side guards: a page-table entry that names a block outside the
 *    pool, or a context length outside [0, max_pages_per_seq * page_tokens]
 *    or above max_context_len, never causes an out-of-bounds read; the rows
 *    it affects are written as NaN (out and lse), so such inputs fail loudly
 *    rather than silently (attnres AGENTS.md, "Non-Negotiable Invariants").
 *  - The library is stateless and thread-safe.  Results are bitwise
 *    deterministic run to run; split boundaries are fixed in tokens, so the
 *    page size and the physical placement of pages do not change the result
 *    bits.  (Tiered calls visit the pages of a split grouped by tier; there
 *    the placement still leaves the bits alone, the page size -- which sets
 *    the tier granularity -- may change the last bits.)
 */
#ifndef ATLAS_H
#define ATLAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATLAS_ABI_VERSION 4u

typedef int32_t atlas_status;
#define ATLAS_OK 0           /* success (work enqueued) */
#define ATLAS_EINVAL 1       /* invalid argument: null pointer, bad size, ... */
#define ATLAS_EUNSUPPORTED 2 /* valid but not implemented: head_dim, dtype, ... */
#define ATLAS_EWORKSPACE 3   /* workspace missing or smaller than required */
#define ATLAS_EDEVICE 4      /* the HIP runtime reported an error */
#define ATLAS_ECAPACITY 5    /* residency runtime: a pool has no room for what the
                                policy needs (nothing was changed) */

/* Element types of q and of resident K/V pages. */
#define ATLAS_F32 0
#define ATLAS_BF16 1
#define ATLAS_F16 2

/* Tiered page-table entries (atlas_paged_attention_tiered): the top two bits
 * hold the tier, the low 30 bits the slot in that tier's pool. */
#define ATLAS_TIER_SHIFT 30
#define ATLAS_TIER_HOT 0  /* f16 / bf16 page in the hot pool (args k_pool/v_pool) */
#define ATLAS_TIER_INT8 1 /* int8 codes, one f32 scale per (page, kv head) */
#define ATLAS_TIER_INT4 2 /* int4 codes, two per byte, same scale layout */
#define ATLAS_TIER_FP8 3  /* FP8 E4M3 codes (OCP "e4m3fn"), same scale layout */
/* Tier 3 is the extension tier: bits 29-28 of its entries give the kind and
 * bits 27-0 the slot (so FP8 slots stay below 2^28).  Kind 3 names no pool. */
#define ATLAS_EXT_KIND_SHIFT 28
#define ATLAS_EXT_FP8 0   /* (3 << 30) | (0 << 28) | slot: FP8 pool */
#define ATLAS_EXT_INT2 1  /* (3 << 30) | (1 << 28) | slot: INT2 codes, four per byte */
/* (3 << 30) | (2 << 28) | slot: 1-bit archival pool (argus-cache, heatmap
 * legend: "8-way sign-packed with FP16 outlier preservation"; its limitations
 * section keeps such pages out of attention).  Attention calls treat these
 * entries like entries that name no page (NaN rows; atlas_validate_tables
 * counts them); atlas_promote_pages reconstructs them into hot blocks first. */
#define ATLAS_EXT_1BIT 2
#define ATLAS_1BIT_MAX_OUTLIERS 64

/*
 * One attention call (decode or chunked prefill).  CFR-Atlas README,
 * "Config::builder(page_tokens, head_dim)" and "AttentionRequest::new(layer,
 * head, query, context_tokens)" name the same quantities for one head.
 *
 * Query rows.  With query_start == NULL every sequence has exactly one query
 * row (decode) and total_q == num_seqs.  Otherwise sequence s owns rows
 * query_start[s] .. query_start[s+1]-1 (chunked prefill), which are the last
 * n_q = query_start[s+1]-query_start[s] positions of its context: row t of
 * the chunk sees keys 0 .. context_lens[s] - n_q + t.  A decode row sees all
 * context_lens[s] keys, its own included.
 *
 * Heads.  Query head h reads kv head h / (num_heads / num_kv_heads): MHA when
 * the counts are equal, MQA when num_kv_heads == 1, GQA otherwise (CFR-Atlas
 * README, module list: "MHA/MQA/GQA head mapping").
 *
 * Paging.  Logical token j of sequence s is row j % page_tokens of block
 * page_table[s * max_pages_per_seq + j / page_tokens] (CFR-Atlas README,
 * PageKey and token_range of a regenerated page).
 *
 * Positional policy (CFR-Atlas README, module list and test list: RoPE and
 * ALiBi).  The position of a query row is its own key, i = (keys it sees)
 * - 1.
 *  - ALiBi (Press et al., 2022): with alibi_slopes != NULL the score of key j
 *    for query head h becomes scale * q.k_j - alibi_slopes[h] * (i - j).
 *  - RoPE (Su et al., RoFormer, 2021): with rope_theta > 0 dims (2m, 2m + 1)
 *    of q are rotated by the angle i * rope_theta^(-2m / head_dim) before
 *    the dot products.  K pages hold keys already rotated by their own
 *    position, as a model caches them (atlas_write_kv rotates new keys);
 *    regenerated keys are produced unrotated, rotated in the kernel by their
 *    token position and rounded to bf16 (the value a bf16 cache holds, which
 *    the regenerator must reproduce).  V is never rotated.  The angle is reduced in f64
 *    turns and taken through the hardware sine and cosine (absolute error
 *    about 1e-6); rotated q enters the 16-bit matrix-core paths as a
 *    hi + lo pair, so its rounding stays near f32.
 */
typedef struct atlas_attn_args {
    uint32_t struct_size;       /* = sizeof(atlas_attn_args); ABI guard */
    int32_t q_dtype;            /* ATLAS_F32 / ATLAS_BF16 / ATLAS_F16 */
    int32_t kv_dtype;           /* element type of k_pool / v_pool */
    int32_t num_seqs;           /* >= 1 */
    int32_t num_heads;          /* query heads, multiple of num_kv_heads */
    int32_t num_kv_heads;       /* >= 1 */
    int32_t head_dim;           /* 64 or 128 */
    int32_t page_tokens;        /* tokens per page, multiple of 16 */
    int32_t max_pages_per_seq;  /* row length of page_table */
    int32_t num_blocks;         /* blocks in k_pool / v_pool */
    int32_t max_context_len;    /* host: >= every context_lens[s] */
    int32_t max_query_len;      /* host: >= every chunk length (1 for decode) */
    int32_t total_q;            /* query rows (== num_seqs for decode) */
    int32_t split_tokens;       /* keys per split-K work item of decode, or per
                                   window of a regenerating prefill (multiple of 64);
                                   0 = the library chooses from the shape */
    float scale;                /* softmax scale, finite (e.g. 1/sqrt(head_dim)) */
    const void *q;              /* [total_q][num_heads][head_dim], q_dtype */
    const void *k_pool;         /* [num_blocks][num_kv_heads][page_tokens][head_dim] */
    const void *v_pool;         /* same shape and type as k_pool */
    const int32_t *page_table;  /* [num_seqs][max_pages_per_seq] block ids */
    const int32_t *context_lens;/* [num_seqs] keys per sequence, >= 0 */
    const int32_t *query_start; /* [num_seqs + 1] prefix sums, or NULL (decode) */
    float *out;                 /* [total_q][num_heads][head_dim] f32 */
    float *lse;                 /* [total_q][num_heads] f32, natural log;
                                   -inf (and out = 0) for a row with no keys */
    void *workspace;            /* device scratch, >= atlas_workspace_size() */
    size_t workspace_bytes;
    void *stream;               /* hipStream_t, NULL = default stream */
    void *profile_events[2];    /* optional hipEvent_t pair (or NULLs): recorded on
                                   `stream` just before and just after the main
                                   attention kernel, so a caller can time that
                                   kernel alone (the split merge and a
                                   regeneration pre-pass fall outside the pair;
                                   a windowed matrix-core prefill has the pair
                                   around all its windows, each a preparation
                                   and a fold kernel) */
    const float *alibi_slopes;  /* [num_heads] f32 ALiBi slopes, finite, or NULL */
    float rope_theta;           /* rotary base (e.g. 10000), finite and > 1, or 0 */
    int32_t reserved;           /* 0 */
} atlas_attn_args;

/*
 * Cold-tier pools of atlas_paged_attention_tiered (ARGUS, "Visual
 * Architecture": FP16 hot pool, FP8, INT8, INT4 "2-way Bit-Packed"; pages are
 * reconstructed in registers just before the dot products, ARGUS "Why It
 * Works: Storage vs. Computation").  Value = code * scale, symmetric, one f32
 * scale per (page, kv head), separately for K and V.  int4 byte i of a row
 * holds element 2i in its low nibble and element 2i+1 in its high nibble,
 * two's complement.  FP8 codes are OCP E4M3 ("e4m3fn": bias 7, largest
 * finite 448, 0x7F / 0xFF NaN) and value = e4m3(code) * scale.  INT2 ("4-way
 * Bit-Packed"): byte i of a row holds elements 4i .. 4i+3, element 4i+j in
 * bits 2j, 2j+1, two's complement; codes -1, 0, 1 (scale = max|x| / 1).  A
 * pool with zero slots may pass NULL pointers.
 */
typedef struct atlas_tier_pools {
    uint32_t struct_size;       /* = sizeof(atlas_tier_pools) */
    int32_t num_int8;           /* slots in the int8 pool */
    int32_t num_int4;           /* slots in the int4 pool */
    int32_t reserved;
    const int8_t *int8_k;       /* [num_int8][num_kv_heads][page_tokens][head_dim] */
    const int8_t *int8_v;
    const float *int8_k_scale;  /* [num_int8][num_kv_heads] */
    const float *int8_v_scale;
    const uint8_t *int4_k;      /* [num_int4][num_kv_heads][page_tokens][head_dim/2] */
    const uint8_t *int4_v;
    const float *int4_k_scale;  /* [num_int4][num_kv_heads] */
    const float *int4_v_scale;
    int32_t num_fp8;            /* slots in the FP8 pool */
    int32_t reserved2;          /* 0 */
    const uint8_t *fp8_k;       /* [num_fp8][num_kv_heads][page_tokens][head_dim] */
    const uint8_t *fp8_v;
    const float *fp8_k_scale;   /* [num_fp8][num_kv_heads] */
    const float *fp8_v_scale;
    int32_t num_int2;           /* slots in the INT2 pool */
    int32_t reserved3;          /* 0 */
    const uint8_t *int2_k;      /* [num_int2][num_kv_heads][page_tokens][head_dim/4] */
    const uint8_t *int2_v;
    const float *int2_k_scale;  /* [num_int2][num_kv_heads] */
    const float *int2_v_scale;
    /* 1-bit archival pool.  A (page, kv head) block of n = page_tokens *
     * head_dim elements (row-major) is stored as
     *   signs: bit j of byte i set iff element 8 i + j is negative (x < 0);
     *   scale: f32, the mean |x| of the elements that are not outliers (0 if
     *          there are none);
     *   outliers: the `outliers_1bit` elements of largest |x| (ordered by the
     *          bit pattern of f32 |x|, ties to the lower index), sorted by
     *          index, one uint32 each: index in bits 0-15, FP16 value bits
     *          (round to nearest even) in bits 16-31.
     * Element e decodes to the FP16 value of an outlier entry with index e (a
     * later entry wins; indices >= n are ignored), else -scale if its sign
     * bit is set, else +scale.  Needs n <= 65536. */
    int32_t num_1bit;           /* slots in the 1-bit pool */
    int32_t outliers_1bit;      /* outliers per block, 0 .. ATLAS_1BIT_MAX_OUTLIERS */
    const uint8_t *bit_k;       /* [num_1bit][num_kv_heads][page_tokens * head_dim / 8] */
    const uint8_t *bit_v;
    const float *bit_k_scale;   /* [num_1bit][num_kv_heads] */
    const float *bit_v_scale;
    const uint32_t *bit_k_out;  /* [num_1bit][num_kv_heads][outliers_1bit] */
    const uint32_t *bit_v_out;
} atlas_tier_pools;

/*
 * Regenerated pages (CFR-Atlas README: cold pages are "regenerated
 * deterministically into scratch buffers" and the fold stays exact when the
 * regenerator reproduces the stored rows).  Logical pages
 * 0 .. regen_pages[s]-1 of sequence s are not read from the pool (their
 * page-table entries are ignored); their K/V values are
 *     c  = layer<<48 | kv_head<<40 | token<<9 | dim<<1 | kv   (kv: 0 = K, 1 = V)
 *     z  = mix64(seed + (c + 1) * 0x9E3779B97F4A7C15)   (SplitMix64 output c+1)
 *     x  = (z >> 40) * 2^-23 - 1                         (uniform on [-1, 1))
 *     value = bf16(x), round to nearest even.
 * Bounds: layer < 2^16, kv_head < 2^8, token < 2^31, dim < 2^8.  Requires
 * kv_dtype == ATLAS_BF16.  Resident pages must hold the same values for the
 * result to equal full-KV attention (atlas_regenerate_pages writes them).
 */
typedef struct atlas_regen_spec {
    uint32_t struct_size;       /* = sizeof(atlas_regen_spec) */
    uint32_t layer;
    uint64_t seed;
    const int32_t *regen_pages; /* [num_seqs] regenerated leading pages */
    int32_t max_regen_pages;    /* host: >= every regen_pages[s] */
    int32_t reserved;
} atlas_regen_spec;

/* ABI version of the loaded library (ATLAS_ABI_VERSION it was built with). */
uint32_t atlas_abi_version(void);

/* Static description of a status code. */
const char *atlas_status_string(atlas_status status);

/* Human-readable reason of the last error returned on this host thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char *atlas_last_error(void);

/*
 * Workspace bytes needed by atlas_paged_attention (regen == NULL) or
 * atlas_paged_attention_regen (regen != NULL) for these arguments, and of
 * atlas_paged_attention_tiered (regen NULL; its pools do not change the
 * size, and the hot-pool fields are not checked here, so an all-cold call
 * with num_blocks 0 can be sized).  Reads host fields only.  The workspace holds the split-K partials of decode (one f32
 * vector of head_dim plus one lse per (row, head, split)).  Matrix-core
 * chunked prefill takes the keys in windows of W tokens (W = split_tokens,
 * or 16384 when split_tokens is 0, at most 4194304, cut to the longest
 * context rounded up to 64) and gathers each window -- regenerated keys from the regenerator,
 * resident keys through the page table -- into one ring that every window
 * reuses (CFR-Atlas README, overview: scratch buffers that are reused), so
 * its workspace is
 *     2 * num_seqs * num_kv_heads * W * head_dim * 2 bytes
 * (K in the kv dtype and V in f16, V stored per 64-key tile dims-major;
 * 64 MiB for one sequence, 8 kv heads,
 * head_dim 128 and W = 16384), at most that for any context length.  Each
 * regenerated value is still computed once per call.  Its contents need no
 * initialisation and are not meaningful between calls; two calls in flight
 * at the same time must not share a workspace.
 */
atlas_status atlas_workspace_size(const atlas_attn_args *args,
                                  const atlas_regen_spec *regen,
                                  size_t *bytes);

/*
 * Paged causal attention: decode (query_start == NULL) or chunked prefill.
 * kv_dtype F32, BF16 or F16; q_dtype F32 with F32 K/V, otherwise BF16 or F16.
 * head_dim 64 or 128; num_heads / num_kv_heads in {1, 2, 4, 8}.  Decode
 * rows are split over pages (split-K) and merged by log-sum-exp; with 16-bit
 * K/V (q of the same type), head_dim 128 and 2, 4 or 8 query heads per kv
 * head both products run on matrix cores (PV with P as f16 for F16 pages and
 * as a bf16 hi + lo pair for BF16 pages, so decode has no range limit on V),
 * otherwise on the vector ALUs.  Chunked prefill over BF16/F16 K/V (q of the
 * same type) with head_dim 128 runs QK^T and PV on matrix cores; other
 * prefill shapes use the vector-ALU kernel.  Prefill PV takes the
 * probabilities and V in f16, so there V must lie within the f16 range
 * (|v| <= 65504).
 */
atlas_status atlas_paged_attention(const atlas_attn_args *args);

/*
 * Decode over tiered pages: page_table entries are (tier << 30) | slot.  Hot
 * pages come from args->k_pool / v_pool (kv_dtype F16 or BF16, num_blocks
 * slots); int8, int4, FP8 and INT2 pages from `pools`.  Decode only (query_start must
 * be NULL).  Codes are decoded in registers and the per-page scales are applied
 * to the dot products and to the probabilities, never written back.  With
 * F16 hot pages, head_dim 128 and 2, 4 or 8 query heads per kv head both
 * products run on matrix cores in f16 (when a split spans at most 510
 * pages): the codes convert exactly (FP8 through the gfx950 hardware
 * conversion), q is rounded to f16 (exact for bf16 q
 * with 2^-14 <= |q| <= 65504; smaller magnitudes carry an absolute error of
 * at most 2^-25, larger ones are out of range).
 */
atlas_status atlas_paged_attention_tiered(const atlas_attn_args *args,
                                          const atlas_tier_pools *pools);

/*
 * Attention with regenerated leading pages (see atlas_regen_spec).  Decode
 * rows regenerate each value inside the attention kernel, where it is used
 * once.  Chunked prefill walks the keys window by window (see
 * atlas_workspace_size): the window's regenerated keys are written once into
 * the workspace ring, the matrix-core kernel folds the window over resident
 * and regenerated pages alike and merges it into out / lse by log-sum-exp.
 * The windows are fixed in tokens, so the result bits do not depend on which
 * pages are regenerated or on the page size.
 */
atlas_status atlas_paged_attention_regen(const atlas_attn_args *args,
                                         const atlas_regen_spec *regen);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as atlas_paged_attention, with its workspace taken from a
 * scratch array built into the library instead of args->workspace (which is
 * ignored).  The array holds ATLAS_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU;
 * each GPU the library runs on keeps its own copy until the process ends.
 * A call whose plan needs more (atlas_workspace_size with regen NULL) fails
 * with ATLAS_EWORKSPACE before any launch.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a device
 * looks up that device's array address.  Every call on one GPU shares the
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  The array's contents need no
 * initialisation and carry nothing from one call to the next.
 */
#define ATLAS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
atlas_status atlas_paged_attention_noalloc(const atlas_attn_args *args);

/*
 * Log-sum-exp merge of split-K partials (attnres AGENTS.md, "online softmax
 * merge"):  lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * o_s.
 *   part_out [splits][rows][head_dim] f32: normalised partial outputs
 *   part_lse [splits][rows] f32, natural log; -inf marks an empty split
 *   out [rows][head_dim] f32, lse [rows] f32
 * A row whose splits are all empty gets out = 0 and lse = -inf.  Splits are
 * combined in index order (deterministic).  head_dim <= 256, splits >= 1.
 */
atlas_status atlas_fold_partials(const float *part_out, const float *part_lse,
                                 int32_t splits, int32_t rows, int32_t head_dim,
                                 float *out, float *lse, void *stream);

/*
 * Inspection entry points.  Each copies or decodes stored values without
 * attention arithmetic so that the page walk and the encodings can be checked
 * bit for bit against an independent implementation.
 */

/* Gather tokens 0 .. num_tokens-1 of sequence `seq` through the page table
 * into contiguous [num_tokens][num_kv_heads][head_dim] arrays of kv_dtype
 * (plain pools; tiered tables are rejected).  num_tokens <= max_pages_per_seq
 * * page_tokens. */
atlas_status atlas_gather_pages(const atlas_attn_args *args, int32_t seq,
                                int32_t num_tokens, void *k_out, void *v_out);

/* Write the regenerated K/V values of logical pages logical_pages[i] into
 * pool blocks dst_blocks[i] (i < n), pools of shape [*][num_kv_heads]
 * [page_tokens][head_dim] and type kv_dtype (BF16 or F32; without a rotary
 * embedding the values are bf16-exact either way).  Both index arrays are device int32.  With
 * rope_theta > 0 the K rows are stored rotated by their token position (see
 * the positional policy of atlas_attn_args), rounded to kv_dtype, so that
 * resident pages hold what the regenerating kernels compute.
 * nonfinite (device int32 [n], optional; CFR-Atlas README, hardening
 * baseline: finite-value validation before hot-cache admission): after the
 * call, nonfinite[i] is the number of non-finite K and V values stored in
 * block dst_blocks[i], or -1 if that block id is outside [0, num_blocks)
 * (nothing written); atlas_residency_refuse_admissions takes the flagged
 * pages back.  Needs page_tokens * head_dim * element bytes to be a
 * multiple of 16. */
atlas_status atlas_regenerate_pages(uint64_t seed, uint32_t layer,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    int32_t page_tokens, int32_t kv_dtype,
                                    float rope_theta,
                                    const int32_t *logical_pages,
                                    const int32_t *dst_blocks, int32_t n,
                                    int32_t num_blocks, void *k_pool,
                                    void *v_pool, void *stream,
                                    int32_t *nonfinite);

/* Decode tier-tagged pages entries[i] (i < n, device int32, (tier << 30) |
 * slot) to f32 K/V [n][num_kv_heads][page_tokens][head_dim]: hot pages are
 * widened exactly, int8 / int4 pages give f32(code * scale). */
atlas_status atlas_dequant_pages(const atlas_attn_args *args,
                                 const atlas_tier_pools *pools,
                                 const int32_t *entries, int32_t n,
                                 float *k_out, float *v_out);

/*
 * Debug check of the tables behind a call (the CFR-Atlas README asks that
 * invalid configurations and page ranges be rejected; attention kernels only
 * turn a bad entry into NaN rows, this call counts them).  Same arguments as
 * the attention call it guards: pools != NULL checks a tiered call, regen !=
 * NULL a regenerated one (not both).  Reads only the visible keys of every
 * sequence.  report_dev: caller-owned device buffer of 4 uint32 counters,
 * overwritten:
 *   [0] page-table entries of visible, non-regenerated pages that name no
 *       page (slot beyond its pool);
 *   [1] sequences whose context length, query range or regenerated-page
 *       count is out of bounds;
 *   [2] non-finite K or V elements among visible tokens of resident pages,
 *       and FP8 NaN codes of visible FP8 pages (check_values != 0 only;
 *       reads every such element);
 *   [3] non-finite K or V scales of visible cold pages (check_values only).
 * Asynchronous on args->stream; if report_host != NULL the counters are also
 * copied there and the call waits for the stream.  Allocates nothing.
 */
atlas_status atlas_validate_tables(const atlas_attn_args *args,
                                   const atlas_tier_pools *pools,
                                   const atlas_regen_spec *regen,
                                   int32_t check_values, uint32_t *report_dev,
                                   uint32_t *report_host);

/*
 * KV write path (the write side of the cache the attention calls read).
 *
 * atlas_write_kv: every query row of `args` (a decode token, or a token of a
 * prefill chunk) owns the key at its own position ctx - n_q + t; its K and V
 * rows k_new / v_new[row][kv_head][head_dim] (kv_dtype, device, 16-byte
 * aligned like the pools) are written to row pos % page_tokens of block
 * page_table[s][pos / page_tokens] of args->k_pool / v_pool, so that the
 * attention call on the same arguments sees them.  The pools are written
 * through args' pointers.  With args->rope_theta > 0 the K row is stored
 * rotated by its position (rounded to kv_dtype); V is stored as given.  Rows
 * whose block id or context length is invalid are skipped
 * (atlas_validate_tables counts them).  Same argument checks as
 * atlas_paged_attention; asynchronous on args->stream.
 */
atlas_status atlas_write_kv(const atlas_attn_args *args, const void *k_new,
                            const void *v_new);

/*
 * atlas_demote_pages: encodes pages into the cold tiers (argus-cache,
 * "Visual Architecture": the compression cascade FP16 -> FP8 -> INT8 ->
 * INT4 -> INT2 -> 1-bit).  For i < n, the source src_slots[i] is a tiered
 * entry (tier << 30) | slot: tier 0 is a hot block of args->k_pool / v_pool
 * (kv_dtype F16 or BF16, every row finite; a plain block id is such an
 * entry), an int8, int4, FP8 or INT2 entry a cold slot of `pools` whose values
 * enter as f32(code * scale).  It is encoded into dst_entries[i], an int8,
 * int4, FP8, INT2 or 1-bit entry of `pools`: for each kv head, K and V
 * separately,
 *     scale = max|x| / qmax    (f32, correctly rounded; qmax 127 / 7 / 448 / 1)
 *     code  = clamp(rint(x / scale), -qmax, qmax)   (round half to even)
 *     FP8:  code = the E4M3 code nearest to x / scale (ties to the even
 *           code; x / scale is correctly rounded f32)
 * and an all-zero block gets scale 0 and codes 0; a 1-bit destination takes
 * the encoding described at atlas_tier_pools (its scale sums |x| in f64, so
 * it can differ from the exactly rounded mean by one f32 ulp).  Codes and
 * scales are written through the pools' pointers; the caller then points its
 * page-table entries at dst_entries.  A destination outside its pool, or a
 * 1-bit source (use atlas_promote_pages), rejects the page (nothing written);
 * a source outside its pool writes NaN scales (and, into a 1-bit slot, NaN
 * outlier values at index 0), so every value read from the page is NaN.
 * Each rejected page adds 1 to *rejected (device int32, optional).
 * The source and destination sets must not overlap between calls in flight.
 * Asynchronous on args->stream.
 */
atlas_status atlas_demote_pages(const atlas_attn_args *args,
                                const atlas_tier_pools *pools,
                                const int32_t *src_slots,
                                const int32_t *dst_entries, int32_t n,
                                int32_t *rejected);

/*
 * atlas_promote_pages: the transient reconstruction of argus-cache's
 * overview (cold or archived pages restored to FP16 when a query needs
 * them).  For i < n, the page of the tiered entry src_entries[i] (any class:
 * hot, int8, int4, FP8, INT2 or 1-bit; device int32) is written into hot block
 * dst_blocks[i] of args->k_pool / v_pool (device int32): every element's value
 * (f32(code * scale), the 1-bit decoding, or the hot value itself) rounded to
 * kv_dtype (F32, F16 or BF16; round to nearest even), K and V, every kv head.
 * A destination block outside [0, num_blocks) rejects the page (nothing
 * written); a source outside its pool, or of kind 3, fills the destination
 * block with NaN.  Each such page adds 1 to *rejected (device int32,
 * optional).  nonfinite (device int32 [n], optional): after the call,
 * nonfinite[i] counts the non-finite K and V values now in block
 * dst_blocks[i] (-1 for a rejected destination), so a caller can see which
 * rebuilt pages would turn rows NaN.  Sources and destinations must not
 * overlap within a call or with calls in flight.  Asynchronous on
 * args->stream; allocates nothing.
 */
atlas_status atlas_promote_pages(const atlas_attn_args *args,
                                 const atlas_tier_pools *pools,
                                 const int32_t *src_entries,
                                 const int32_t *dst_blocks, int32_t n,
                                 int32_t *rejected, int32_t *nonfinite);

/*
 * Measurement helper (not part of the attention method): reads `bytes`
 * (multiple of 16, src 16-byte aligned) of device memory once with 16-byte
 * loads spread over `blocks` workgroups of 256 threads, and writes one xor of
 * the words read per workgroup to out[0 .. blocks-1] (device, caller-owned).
 * Timing it gives the streaming read bandwidth the attention kernels are
 * compared against.  Asynchronous on `stream`.
 */
atlas_status atlas_read_probe(const void *src, size_t bytes, uint32_t *out,
                              int32_t blocks, void *stream);

/*
 * Measurement helper (not part of the attention method): the issue rates the
 * matrix-core prefill is built from.  Launches 1024 workgroups, one per CU at
 * a time (each holds 96 KiB of LDS), of 256 * waves_per_simd threads
 * (waves_per_simd 1 or 2); every wave repeats `iters` (1 .. 2^20) times one
 * fixed mix of 32x32x16 bf16 matrix products on four independent
 * accumulators, f32 exponentials and fused multiply-adds, and LDS reads:
 *   mix 0: 16 exponentials          mix 4: 8 16-byte + 16 8-byte transposing reads
 *   mix 1: 16 multiply-adds         mix 5: 16 products + the reads of mix 4
 *   mix 2: 16 products              mix 6: 16 products + 16 16-byte reads
 *   mix 3: 16 products, 16 exponentials and 16 multiply-adds
 *   mix 7: 32 products + 16 16-byte reads
 * (mixes 5 and 6 read 1 KiB of LDS per product, mix 7 0.5 KiB).  Writes the
 * shader-clock ticks and the 100 MHz constant-clock ticks of workgroup 0's
 * loop to clocks[0..1] (device, caller-owned); sink (device, 1024 floats,
 * caller-owned) keeps the work from being dropped and is normally left
 * unwritten.  Timing the launch gives the cycles each mix takes per SIMD.
 * EINVAL for NULL pointers or arguments outside the ranges above.
 * Asynchronous on `stream`.
 */
atlas_status atlas_issue_probe(int32_t mix, int32_t waves_per_simd, int32_t iters,
                               uint64_t *clocks, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATLAS_H */
