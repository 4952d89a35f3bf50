// Internal launch parameters shared by the host dispatcher (api.hip) and the
// kernels.  Plain structs of pointers and sizes, passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atlas {

enum KvType : int { KV_F32 = 0, KV_BF16 = 1, KV_F16 = 2 };
enum Mode : int { MODE_PLAIN = 0, MODE_TIERED = 1, MODE_REGEN = 2 };

// Where a query row sits: its sequence and how many leading keys it sees.
// Shared by the decode kernel and the fold kernel so both agree on the
// number of splits of every row.
struct RowMap {
    const int32_t *context_lens;  // [num_seqs]
    const int32_t *query_start;   // [num_seqs + 1] or nullptr (one row per sequence)
    int32_t num_seqs;
    int32_t max_context_len;      // host bound
    int32_t max_keys;             // max_pages_per_seq * page_tokens
};

// Positional policy of a call: ALiBi slopes and the rotary embedding.
struct PosParams {
    const float *alibi;       // [num_heads] slopes, or nullptr
    double rope_log2_theta;   // log2 of the rotary base
    int32_t rope;             // 1: rotate q (and regenerated / new K)
};

struct DecodeParams {
    RowMap rows;
    PosParams pos;
    const void *q;            // [total_q][H][D]
    int32_t q_dtype;
    const void *k_pool;       // [num_blocks][Hkv][P][D] (hot pool in tiered mode)
    const void *v_pool;
    const int32_t *page_table;
    int32_t num_heads, num_kv_heads, page_tokens, max_pages, num_blocks, total_q;
    int32_t split_tokens, max_splits;
    uint32_t p_magic, p_shift;  // x / page_tokens == (umulhi(x, p_magic) + x) >> p_shift, x < 2^31
    float scale_log2;         // softmax scale * log2(e)
    float *part_o;            // [total_q * H][max_splits][D]
    float *part_lse;          // [total_q * H][max_splits], natural log
    float *out;               // [total_q][H][D]  (written directly if direct != 0)
    float *lse;               // [total_q][H]
    int32_t direct;
    // tiered pools
    const int8_t *i8_k, *i8_v;
    const float *i8_ks, *i8_vs;
    const uint8_t *i4_k, *i4_v;
    const float *i4_ks, *i4_vs;
    int32_t n_i8, n_i4;
    const uint8_t *f8_k, *f8_v;   // FP8 E4M3 codes
    const float *f8_ks, *f8_vs;
    int32_t n_f8;
    const uint8_t *i2_k, *i2_v;   // INT2 codes, four per byte
    const float *i2_ks, *i2_vs;
    int32_t n_i2;
    const uint8_t *b1_k, *b1_v;   // 1-bit archive: sign bits, eight per byte
    const float *b1_ks, *b1_vs;
    const uint32_t *b1_ko, *b1_vo;  // outliers: index | f16 bits << 16
    int32_t n_b1, b1_nout;
    // regenerated pages
    uint64_t seed;
    uint32_t layer;
    const int32_t *regen_pages;  // [num_seqs]
    int32_t max_regen;           // host bound on regen_pages[s]
};

struct FoldParams {
    const float *part_o;
    const float *part_lse;
    float *out;
    float *lse;
    int64_t o_row_stride, o_split_stride;   // in floats
    int64_t l_row_stride, l_split_stride;
    int32_t rows;          // rows to merge (total_q * H internally)
    int32_t head_dim;
    int32_t fixed_splits;  // > 0: every row has this many splits
    // otherwise the split count of a row comes from its visible keys
    RowMap map;
    int32_t num_heads;
    int32_t split_tokens;
};

struct PrefillParams {
    RowMap rows;
    PosParams pos;
    const void *q;            // [total_q][H][D] bf16 / f16
    const void *k_pool;
    const void *v_pool;
    const int32_t *page_table;
    // the keys of the current window, gathered: ring_k (kv type) / ring_v
    // (f16) [num_seqs][Hkv][ring_tokens][D], row = key - key_begin
    const void *ring_k;
    const void *ring_v;
    int32_t ring_tokens;
    const int32_t *regen_pages;   // validated only (the window preparation reads them)
    int32_t max_regen;
    int32_t num_heads, num_kv_heads, total_q;
    int32_t max_query_len;
    int32_t q_blocks;         // query tiles per sequence (grid)
    int32_t key_begin;        // keys of this launch: [key_begin, key_end), key_begin a
    int32_t key_end;          // multiple of 64, window length <= ring_tokens with a ring
    int32_t carry;            // 1: merge into the out / lse an earlier window wrote
    float scale_log2;
    float *out;
    float *lse;
};

struct RegenFillParams {
    PosParams pos;                 // rope: K written rotated by its token position
    uint64_t seed;
    uint32_t layer;
    int32_t num_kv_heads, head_dim, page_tokens;
    const int32_t *logical_pages;  // [n]
    const int32_t *dst_blocks;     // [n]
    int32_t n;
    int32_t num_blocks;
    int32_t kv_f32;                // 1: write f32 values, 0: bf16
    void *k_dst;
    void *v_dst;
};

// One key window of a chunked prefill gathered into the ring the prefill
// kernel reads: ring[seq][Hkv][window_tokens][128], K in the kv type, V in
// f16; regenerated keys from the page regenerator, other keys through the
// page table.
struct WindowParams {
    PosParams pos;                 // rope: regenerated K rotated by its token position
    uint64_t seed;
    uint32_t layer;
    int32_t num_seqs, num_kv_heads, page_tokens, max_pages, num_blocks;
    const void *k_pool, *v_pool;   // [num_blocks][Hkv][P][128]
    const int32_t *page_table;
    int32_t kv_f16;                // 1: f16 pools, 0: bf16 pools
    const int32_t *regen_pages;    // [num_seqs] or null
    int32_t max_regen;
    const int32_t *context_lens;   // [num_seqs]
    int32_t max_context_len, max_keys;
    int32_t key_begin;             // first key of the window (multiple of 64)
    int32_t window_tokens;         // ring rows per (seq, kv head), multiple of 64
    void *ring_k;
    void *ring_v;
};

// Debug check of the tables and pools behind a call.
struct ValidateParams {
    DecodeParams p;           // tables, lengths, pools, regen counts (regen_pages may be null)
    int32_t mode;             // MODE_PLAIN / MODE_TIERED / MODE_REGEN
    int32_t kv_type, head_dim;
    int32_t check_values;
    int32_t max_query_len;
    uint32_t *report;         // [4] counters, zeroed by the launcher's first kernel
};

// New tokens' K/V rows written into their pages (one row per query row).
struct WriteKvParams {
    RowMap rows;
    PosParams pos;              // rope: K rows stored rotated by their position
    const void *k_new, *v_new;  // [total_q][Hkv][D]
    void *k_pool, *v_pool;      // [num_blocks][Hkv][P][D]
    const int32_t *page_table;
    int32_t num_kv_heads, head_dim, page_tokens, max_pages, num_blocks, total_q;
    int32_t elem_bytes;
    int32_t kv_type;
};

// Hot pages encoded into int8 / int4 cold-tier slots.
struct DemoteParams {
    const void *k_pool, *v_pool;   // hot pool, bf16 or f16
    int32_t kv_type;
    int32_t num_kv_heads, head_dim, page_tokens, num_blocks;
    const int32_t *src_slots;      // [n] sources: (tier << 30) | slot, tier 0 = hot block
    const int32_t *dst_entries;    // [n] (tier << 30) | slot, tier 1 or 2
    int32_t n;
    int8_t *i8_k, *i8_v;
    float *i8_ks, *i8_vs;
    uint8_t *i4_k, *i4_v;
    float *i4_ks, *i4_vs;
    int32_t n_i8, n_i4;
    uint8_t *f8_k, *f8_v;
    float *f8_ks, *f8_vs;
    int32_t n_f8;
    uint8_t *i2_k, *i2_v;
    float *i2_ks, *i2_vs;
    int32_t n_i2;
    uint8_t *b1_k, *b1_v;
    float *b1_ks, *b1_vs;
    uint32_t *b1_ko, *b1_vo;
    int32_t n_b1, b1_nout;
    int32_t *rejected;             // device counter or null
};

// Cold (or hot) pages reconstructed into hot blocks.  `p` describes every
// source pool (its hot pool pointers are the destination too).
struct PromoteParams {
    DecodeParams p;
    void *k_dst, *v_dst;           // the hot pool, written
    int32_t kv_type, head_dim;
    const int32_t *src_entries;    // [n] tiered entries
    const int32_t *dst_blocks;     // [n] hot block ids
    int32_t n;
    int32_t *rejected;             // device counter or null
};

// Classes of a tiered page-table entry: tiers 0-2 as they are, tier 3 split
// by its kind bits (29-28) into FP8, INT2 and the 1-bit archive; kind 3
// names no pool.  Attention reads classes below CLS_B1 only.
enum EntryClass : int {
    CLS_HOT = 0, CLS_I8 = 1, CLS_I4 = 2, CLS_F8 = 3, CLS_I2 = 4, CLS_B1 = 5, CLS_BAD = 6
};
// Branch-free, so callers can issue several entry loads before decoding any.
__host__ __device__ inline int entry_class(uint32_t e, uint32_t &slot) {
    const uint32_t tier = e >> 30;
    const uint32_t kind = (e >> 28) & 3u;
    const bool ext = tier == 3u;
    slot = e & (ext ? ((1u << 28) - 1u) : ((1u << 30) - 1u));
    return ext ? (kind < 3u ? CLS_F8 + (int)kind : CLS_BAD) : (int)tier;
}

// Page-table entries a decode workgroup stages in LDS for its split.
constexpr int kDecodeStagedPages = 512;

// Launchers (defined next to their kernels).  Each returns the HIP error of
// the launch.
hipError_t launch_decode(const DecodeParams &p, int kv_type, int head_dim, int group,
                         int mode, hipStream_t stream);
hipError_t launch_fold(const FoldParams &f, hipStream_t stream);
// Matrix-core decode (QK^T on MFMA) for 16-bit and tiered pages.
bool decode_mfma_supported(int kv_type, int head_dim, int group, int mode, int page_tokens,
                           int split_tokens);
hipError_t launch_decode_mfma(const DecodeParams &p, int kv_type, int group, int mode,
                              hipStream_t stream);
// Query rows per workgroup of the matrix-core prefill kernel.
constexpr int kPrefillRows = 256;
// Keys per window of a matrix-core chunked prefill (the default when the
// caller leaves split_tokens at 0).
constexpr int kPrefillWindow = 16384;
// largest window: the ring rows of one (sequence, kv head) stay within the
// 32-bit byte range of the buffer loads that stage them
constexpr int kPrefillMaxWindow = 1 << 22;
hipError_t launch_prefill(const PrefillParams &p, int kv_type, int group, hipStream_t stream);
hipError_t launch_regen_fill(const RegenFillParams &r, hipStream_t stream);
// Per job i: the non-finite K and V values now stored in block dst_blocks[i]
// of the pools ([*][num_kv_heads][page_tokens][head_dim], elem_bytes 2 or 4;
// f16_bits: 2-byte elements are f16, else bf16), or -1 when the block id is
// outside [0, num_blocks).  Writes out[0 .. n-1].
hipError_t launch_count_nonfinite(const void *k_pool, const void *v_pool,
                                  const int32_t *dst_blocks, int32_t n, int32_t num_blocks,
                                  int32_t num_kv_heads, int32_t page_tokens, int32_t head_dim,
                                  int32_t elem_bytes, int32_t f16_bits, int32_t *out,
                                  hipStream_t stream);
hipError_t launch_window_prepare(const WindowParams &r, hipStream_t stream);
hipError_t launch_gather(const void *k_pool, const void *v_pool, const int32_t *table_row,
                         int32_t num_kv_heads, int32_t head_dim, int32_t page_tokens,
                         int32_t num_blocks, int32_t elem_bytes, int32_t num_tokens,
                         void *k_out, void *v_out, hipStream_t stream);
hipError_t launch_validate(const ValidateParams &v, hipStream_t stream);
hipError_t launch_write_kv(const WriteKvParams &w, hipStream_t stream);
hipError_t launch_demote(const DemoteParams &d, hipStream_t stream);
hipError_t launch_promote(const PromoteParams &q, hipStream_t stream);
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *out, int blocks,
                             hipStream_t stream);
// workgroups of the issue probe: four rounds of one workgroup per CU
constexpr int kIssueProbeBlocks = 1024;
hipError_t launch_issue_probe(int mix, int waves_per_simd, int iters, uint64_t *clocks,
                              float *sink, hipStream_t stream);
hipError_t launch_dequant(const DecodeParams &p, int kv_type, int head_dim,
                          const int32_t *entries, int32_t n, float *k_out, float *v_out,
                          hipStream_t stream);

}  // namespace atlas
