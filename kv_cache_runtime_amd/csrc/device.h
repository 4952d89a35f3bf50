// Device helpers for gfx950 kernels: storage-type widening, 16-lane DPP
// reductions, the page regenerator's value function and the row map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace atlas {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Widening of stored 16-bit values packed two to a 32-bit word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Element i of a row slice held as 32-bit words, for each storage type.
template <int KV>
__device__ __forceinline__ float widen_word(const uint32_t *w, int i) {
    if constexpr (KV == KV_F32) {
        return __uint_as_float(w[i]);
    } else if constexpr (KV == KV_BF16) {
        return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    } else {
        return (i & 1) ? f16_hi(w[i >> 1]) : f16_lo(w[i >> 1]);
    }
}

__device__ __forceinline__ float load_elem(const void *base, int64_t idx, int dtype) {
    if (dtype == KV_F32) return reinterpret_cast<const float *>(base)[idx];
    uint16_t b = reinterpret_cast<const uint16_t *>(base)[idx];
    if (dtype == KV_BF16) return __uint_as_float(((uint32_t)b) << 16);
    return (float)__builtin_bit_cast(_Float16, b);
}

// ---------------------------------------------------------------------------
// Rotary position embedding (RoFormer, Su et al. 2021; the CFR-Atlas README
// lists RoPE as a positional policy).  The pair of dims (2m, 2m + 1) at
// position i turns by the angle i * theta^(-2m / D).
// ---------------------------------------------------------------------------

// Turns (angle / 2 pi) per position of pair m, in f64.
__device__ __forceinline__ double rope_turns(int m, int D, double log2_theta) {
    return exp2(-(double)(2 * m) / (double)D * log2_theta) * 0.15915494309189535;
}

// Rotates (x0, x1) by pos * turns full turns.  The angle is reduced to
// [-1/2, 1/2] turn in f64, then the hardware sine and cosine (which take
// turns) give about 1e-6 absolute accuracy for any position below 2^31.
__device__ __forceinline__ void rope_rotate(float &x0, float &x1, int pos, double turns) {
    double t = (double)pos * turns;
    t -= rint(t);
    const float tf = (float)t;
    const float sn = __builtin_amdgcn_sinf(tf);
    const float cs = __builtin_amdgcn_cosf(tf);
    const float y0 = x0 * cs - x1 * sn;
    const float y1 = x0 * sn + x1 * cs;
    x0 = y0;
    x1 = y1;
}

// f32 rounded to the nearest bf16 value (ties to even), returned as f32.
__device__ __forceinline__ float bf16_round(float x) {
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// Sign-extended bit field: the `bits`-wide field that ends at bit 31 after a
// left shift by `sh` (shift done unsigned, then an arithmetic right shift).
__device__ __forceinline__ int32_t sext_field(uint32_t w, int sh, int bits) {
    return ((int32_t)(w << sh)) >> (32 - bits);
}

// ---------------------------------------------------------------------------
// Streaming loads of K/V pages.  Every page byte an attention call reads is
// read once (the query heads of a kv head share the registers), so the loads
// carry the non-temporal hint (global_load_* ... nt).  On MI355X a plain
// streaming read of 2 GiB measured 5.85 TB/s with ordinary 16-byte loads and
// 6.66 TB/s with non-temporal ones.
// ---------------------------------------------------------------------------
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void *src) {
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(src));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void *src) {
    const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2 *>(src));
    return make_uint2(v.x, v.y);
}

// Vector loads of NB bytes (NB in {1, 2, 4, 8, 16, 32}) of a K/V page into
// 32-bit words, non-temporal.
template <int NB>
__device__ __forceinline__ void load_words(uint32_t *dst, const void *src) {
    if constexpr (NB == 32) {
        const char *s = reinterpret_cast<const char *>(src);
        const uint4 a = ld_stream16(s), b = ld_stream16(s + 16);
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
        dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
    } else if constexpr (NB == 16) {
        const uint4 a = ld_stream16(src);
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    } else if constexpr (NB == 8) {
        const uint2 a = ld_stream8(src);
        dst[0] = a.x; dst[1] = a.y;
    } else if constexpr (NB == 4) {
        dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(src));
    } else if constexpr (NB == 2) {
        dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(src));
    } else {
        static_assert(NB == 1, "unsupported load width");
        dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint8_t *>(src));
    }
}

// ---------------------------------------------------------------------------
// Cross-lane sums within a row of 16 lanes (DPP row_ror).  Rotations by 8, 4,
// 2 and 1 leave the full row sum in every lane, and every lane adds the same
// pairs in the same tree, so all 16 lanes hold bit-identical sums.
// ---------------------------------------------------------------------------
// Lane permutation within 16-lane rows (row_ror only: every lane reads a
// lane of its own row, so bound_ctrl never applies; setting it lets the
// compiler fold the move into the instruction that consumes it).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    static_assert(CTRL >= 0x121 && CTRL <= 0x12F, "row_ror controls only");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0x128>(x);  // row_ror:8
    x += dpp_f<0x124>(x);  // row_ror:4
    x += dpp_f<0x122>(x);  // row_ror:2
    x += dpp_f<0x121>(x);  // row_ror:1
    return x;
}

// ---------------------------------------------------------------------------
// Page regenerator (counter-based SplitMix64, Steele-Lea-Flood 2014).
// Counter c = layer<<48 | kv_head<<40 | token<<9 | dim<<1 | kv addresses
// output c+1 of the stream seeded with `seed`; the value is bf16(2u - 1) with
// u = top 24 bits / 2^24.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t regen_counter(uint32_t layer, int kv_head, int token,
                                                  int dim, int kv) {
    return ((uint64_t)layer << 48) | ((uint64_t)(uint32_t)kv_head << 40) |
           ((uint64_t)(uint32_t)token << 9) | ((uint64_t)(uint32_t)dim << 1) | (uint64_t)kv;
}

__device__ __forceinline__ uint32_t regen_bf16_bits(uint64_t seed, uint64_t ctr) {
    uint64_t z = seed + (ctr + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    const int32_t u = (int32_t)(uint32_t)(z >> 40) - (1 << 23);
    const float x = (float)u * (1.0f / 8388608.0f);   // exact: |u| < 2^24
    uint32_t b = __float_as_uint(x);
    b += 0x7FFFu + ((b >> 16) & 1u);                   // round to nearest even
    return b >> 16;
}

__device__ __forceinline__ float regen_value(uint64_t seed, uint64_t ctr) {
    return __uint_as_float(regen_bf16_bits(seed, ctr) << 16);
}

// ---------------------------------------------------------------------------
// Row map: sequence of a query row and the number of keys it sees.  Returns
// false when the sequence's context length is outside what the page table
// and the host bound allow (the caller then writes NaN for the row).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool map_row(const RowMap &m, int row, int &seq, int &visible) {
    int n_q = 1, t = 0;
    if (m.query_start == nullptr) {
        seq = row;
    } else {
        int lo = 0, hi = m.num_seqs - 1;   // last s with query_start[s] <= row
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (m.query_start[mid] <= row) lo = mid; else hi = mid - 1;
        }
        seq = lo;
        const int q0 = m.query_start[seq];
        n_q = m.query_start[seq + 1] - q0;
        t = row - q0;
    }
    const int ctx = m.context_lens[seq];
    // A chunk's rows are the last n_q tokens of the context, so a chunk longer
    // than its context is malformed; a decode row may see zero keys.
    const bool ok = ctx >= 0 && ctx <= m.max_context_len && ctx <= m.max_keys &&
                    n_q >= 1 && t < n_q && (m.query_start == nullptr || n_q <= ctx);
    visible = ok ? ctx - n_q + t + 1 : 0;
    if (visible < 0) visible = 0;
    return ok;
}

// Stages n page-table entries of a tiered split in LDS grouped by entry
// class (hot, int8, int4, FP8, INT2, then entries that name no pool),
// keeping the logical order inside a class.  s_slot receives each staged
// page's slot in its pool, s_lp its offset from lp_first, and count[c]
// (every thread) the number of entries of class c.  The ranks come from wave
// ballots, so the order is fixed (no atomics).  Whole workgroup of 256
// threads, n <= 512; ends with a barrier.  Folding keys with an online
// softmax does not depend on their order, so a split may visit its pages in
// this order: the waves then mostly meet pages of one class and take one
// load path.
constexpr int kClasses = 6;  // the attended classes, then one bin for every other entry
__device__ __forceinline__ void stage_pages_by_tier(const int32_t *trow, int n, int32_t *s_slot,
                                                    int16_t *s_lp, int (&count)[kClasses]) {
    __shared__ int s_cnt[2][4][kClasses];  // chunk, wave, class
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t slot[2];
    int t[2], rank[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int i = ch * 256 + tid;
        t[ch] = i < n ? min(entry_class((uint32_t)trow[i], slot[ch]), kClasses - 1) : kClasses;
        rank[ch] = 0;
#pragma unroll
        for (int tt = 0; tt < kClasses; ++tt) {
            const uint64_t m = __ballot(t[ch] == tt);
            if (lane == 0) s_cnt[ch][wave][tt] = __popcll(m);
            if (t[ch] == tt)
                rank[ch] = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kClasses; ++tt) {
        int sum = 0;
        for (int c2 = 0; c2 < 2; ++c2)
            for (int w2 = 0; w2 < 4; ++w2) sum += s_cnt[c2][w2][tt];
        count[tt] = sum;
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int i = ch * 256 + tid;
        if (i >= n) continue;
        const int tt = t[ch];
        int pos = rank[ch];
        for (int c2 = 0; c2 < 2; ++c2)
            for (int w2 = 0; w2 < 4; ++w2) {
                for (int u = 0; u < tt; ++u) pos += s_cnt[c2][w2][u];
                if (c2 < ch || (c2 == ch && w2 < wave)) pos += s_cnt[c2][w2][tt];
            }
        s_slot[pos] = (int32_t)slot[ch];
        s_lp[pos] = (int16_t)i;
    }
    __syncthreads();
}

__device__ __forceinline__ int splits_of(int visible, int split_tokens) {
    const int n = (visible + split_tokens - 1) / split_tokens;
    return n < 1 ? 1 : n;
}

}  // namespace atlas
