// The KV write path: new tokens' K/V written into their pages, and hot pages
// demoted into the int8 / int4 cold tiers.
//
// Writing: every query row of a call (a decode token, or a token of a prefill
// chunk) owns the key at its own position, ctx - n_q + t; its K/V rows go to
// row pos % P of block page_table[s][pos / P] of every kv head (CFR-Atlas
// README, PageKey and token ranges; the pages are written in place, never
// concatenated).  Under a rotary embedding the K row is stored rotated by
// its position, as the attention kernels expect cached keys.
//
// Demotion (argus-cache, "Visual Architecture": FP16 -> FP8 -> INT8 -> INT4
// tiers): one block per (page, kv head, K|V) gets a symmetric f32 scale
// max|x| / qmax and codes rint(x / scale) clamped to [-qmax, qmax] (FP8: the
// nearest E4M3 code to x / scale, qmax 448); both divisions are correctly
// rounded f32 so the code decisions are reproducible.  The source is a hot
// block or a cold slot (the cascade's next step): cold values enter as
// f32(code * scale).  int4 codes are
// two's-complement nibbles, element 2i in the low nibble of byte i.
#include "device.h"

namespace atlas {

namespace {

// A 16-byte chunk of a K row starting at dim d0 (even), rotated by the row's
// position (rotary embedding; pairs (2m, 2m + 1) lie inside the chunk) and
// rounded back to its storage type (nearest, ties to even).
__device__ uint4 rotate_chunk(const uint4 k, const int kv_type, const int pos, const int d0,
                              const int D, const double log2_theta) {
    uint32_t w[4] = {k.x, k.y, k.z, k.w};
    if (kv_type == KV_F32) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            float x0 = __uint_as_float(w[2 * m]), x1 = __uint_as_float(w[2 * m + 1]);
            rope_rotate(x0, x1, pos, rope_turns(d0 / 2 + m, D, log2_theta));
            w[2 * m] = __float_as_uint(x0);
            w[2 * m + 1] = __float_as_uint(x1);
        }
    } else {
        const bool bf = kv_type == KV_BF16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float x0 = bf ? bf16_lo(w[m]) : f16_lo(w[m]);
            float x1 = bf ? bf16_hi(w[m]) : f16_hi(w[m]);
            rope_rotate(x0, x1, pos, rope_turns(d0 / 2 + m, D, log2_theta));
            if (bf) {
                w[m] = (__float_as_uint(bf16_round(x0)) >> 16) |
                       (__float_as_uint(bf16_round(x1)) & 0xFFFF0000u);
            } else {
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                const h2 h = {(_Float16)x0, (_Float16)x1};
                w[m] = __builtin_bit_cast(uint32_t, h);
            }
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One thread per 16-byte chunk of a (row, kv head) K or V row.
__global__ __launch_bounds__(256) void write_kv_kernel(const WriteKvParams w) {
    const int64_t chunks_per_row = (int64_t)w.head_dim * w.elem_bytes / 16;
    const int64_t total = (int64_t)w.total_q * w.num_kv_heads * chunks_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t ch = i % chunks_per_row;
        const int64_t rg = i / chunks_per_row;
        const int g = (int)(rg % w.num_kv_heads);
        const int row = (int)(rg / w.num_kv_heads);
        int seq, nvis;
        if (!map_row(w.rows, row, seq, nvis) || nvis < 1) continue;  // nothing to own
        const int pos = nvis - 1;                                      // the row's own key
        const int lp = pos / w.page_tokens;
        const int32_t blk = w.page_table[(int64_t)seq * w.max_pages + lp];
        if (blk < 0 || blk >= w.num_blocks) continue;  // counted by atlas_validate_tables
        const int64_t dst = (((int64_t)blk * w.num_kv_heads + g) * w.page_tokens +
                             (pos - lp * w.page_tokens)) * chunks_per_row + ch;
        const int64_t src = ((int64_t)row * w.num_kv_heads + g) * chunks_per_row + ch;
        uint4 k = reinterpret_cast<const uint4 *>(w.k_new)[src];
        if (w.pos.rope) k = rotate_chunk(k, w.kv_type, pos, (int)ch * (16 / w.elem_bytes),
                                         w.head_dim, w.pos.rope_log2_theta);
        reinterpret_cast<uint4 *>(w.k_pool)[dst] = k;
        reinterpret_cast<uint4 *>(w.v_pool)[dst] = reinterpret_cast<const uint4 *>(w.v_new)[src];
    }
}

// The source block of a demotion: hot 16-bit rows, or the codes and scale of
// a cold slot.  A chunk is 8 consecutive elements: 16 bytes hot, 8 bytes
// int8 / FP8, 4 bytes int4 (loaded into the low words of a uint4).
struct DemoteSrc {
    bool bf16;           // hot pool type
    const uint8_t *base; // the block's first byte
    float scale;         // cold tiers
};

// ONCE: the chunk is read only this time (non-temporal load); chunks a kernel
// reads again stay ordinary loads, so the second read finds them cached.
template <int ST, bool ONCE = false>  // source class: 0 hot, 1 int8, 2 int4, 3 FP8, 4 INT2
__device__ inline uint4 load_chunk(const DemoteSrc &s, int64_t ch) {
    if constexpr (ST == 0)
        return ONCE ? ld_stream16(reinterpret_cast<const uint4 *>(s.base) + ch)
                    : reinterpret_cast<const uint4 *>(s.base)[ch];
    if constexpr (ST == 2) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(s.base) + ch;
        return make_uint4(ONCE ? __builtin_nontemporal_load(p) : *p, 0u, 0u, 0u);
    }
    if constexpr (ST == 4) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(s.base) + ch;
        return make_uint4(ONCE ? __builtin_nontemporal_load(p) : *p, 0u, 0u, 0u);
    }
    const uint2 v = ONCE ? ld_stream8(reinterpret_cast<const uint2 *>(s.base) + ch)
                         : reinterpret_cast<const uint2 *>(s.base)[ch];
    return make_uint4(v.x, v.y, 0u, 0u);
}

// The 8 values of a chunk in f32: hot values exactly, cold values as
// f32(code * scale) (one rounding of the exact product).
template <int ST>
__device__ inline void widen8(const DemoteSrc &s, const uint4 w, float (&x)[8]) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    if constexpr (ST == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint16_t b = (uint16_t)(ww[j >> 1] >> (16 * (j & 1)));
            x[j] = s.bf16 ? __uint_as_float((uint32_t)b << 16)
                          : (float)__builtin_bit_cast(_Float16, b);
        }
    } else if constexpr (ST == 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = (float)sext_field(ww[j >> 2], 24 - 8 * (j & 3), 8) * s.scale;
    } else if constexpr (ST == 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)sext_field(ww[0], 28 - 4 * j, 4) * s.scale;
    } else if constexpr (ST == 4) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)sext_field(ww[0], 30 - 2 * j, 2) * s.scale;
    } else {
        typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(ww[q], false);
            const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(ww[q], true);
            x[4 * q] = a[0] * s.scale;
            x[4 * q + 1] = a[1] * s.scale;
            x[4 * q + 2] = b[0] * s.scale;
            x[4 * q + 3] = b[1] * s.scale;
        }
    }
}

// max |x| of the 8 elements, +inf if any of them is NaN or infinite (a
// plain fmaxf would drop a NaN).  Hot (16-bit) values are compared as their
// bit patterns without the sign: in both formats the patterns of
// non-negative values order like the values, and every infinity or NaN
// pattern lies above every finite one, so one packed integer max per two
// elements does the work.  Integer codes are finite; a block whose scale is
// not finite is caught by the caller (scale_not_finite).
template <int ST>
__device__ inline float absmax8(const DemoteSrc &s, const uint4 w) {
    if constexpr (ST == 0) {
        typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
        auto mag = [](uint32_t x) { return __builtin_bit_cast(u16x2_t, x & 0x7FFF7FFFu); };
        const u16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(mag(w.x), mag(w.y)),
                                                     __builtin_elementwise_max(mag(w.z), mag(w.w)));
        const uint32_t mb = max((uint32_t)m2[0], (uint32_t)m2[1]);
        if (s.bf16) return mb >= 0x7F80u ? __builtin_inff() : __uint_as_float(mb << 16);
        return mb >= 0x7C00u ? __builtin_inff()
                             : (float)__builtin_bit_cast(_Float16, (uint16_t)mb);
    } else {
        float x[8];
        widen8<ST>(s, w, x);
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float a = fabsf(x[j]);
            // FP8 codes include NaN codes; integer codes times a finite
            // scale give no NaN
            m = fmaxf(m, ST == 3 && a != a ? __builtin_inff() : a);
        }
        return m;
    }
}

// a cold source block whose scale is NaN or infinite decodes to non-finite
// values (0 * inf is NaN), so it demotes like a block holding them
template <int ST>
__device__ inline bool scale_not_finite(const DemoteSrc &s) {
    return ST != 0 && !(fabsf(s.scale) < __builtin_inff());
}

// The FP8 E4M3 code nearest to y (ties to the even code), sign from y's sign
// bit, magnitudes of 448 and above saturating to 448 (0x7E; the next step
// would be the NaN code).
__device__ inline uint32_t e4m3_nearest(const float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);  // subnormal grid 2^-9
    uint32_t u = __float_as_uint(a);
    u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;  // 3 mantissa bits, ties to even
    return sign | ((((u >> 23) - 120u) << 3) | ((u >> 20) & 7u));  // exponent bias 127 -> 7
}

// Codes of the 8 elements of chunk ch, stored at their place in the int8 or
// FP8 (8 bytes per chunk), int4 (one 32-bit word) or INT2 (16 bits) block.
template <int ST, int DT>  // source and destination classes
__device__ inline void encode8(const DemoteSrc &src, const uint4 w, const float scale,
                               int8_t *i8, uint8_t *i4, uint8_t *i2, const int64_t ch) {
    constexpr int qmax = DT == 1 ? 127 : DT == 2 ? 7 : DT == 3 ? 448 : 1;
    float x[8];
    widen8<ST>(src, w, x);
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if constexpr (DT == 3) {
            c[j] = scale > 0.0f ? (int)e4m3_nearest(__fdiv_rn(x[j], scale)) : 0;
        } else {
            const float q = scale > 0.0f ? rintf(__fdiv_rn(x[j], scale)) : 0.0f;
            c[j] = (int)fminf(fmaxf(q, (float)-qmax), (float)qmax);
        }
    }
    if constexpr (DT == 1 || DT == 3) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= (uint32_t)(c[j] & 0xFF) << (8 * j);
            hi |= (uint32_t)(c[4 + j] & 0xFF) << (8 * j);
        }
        reinterpret_cast<uint2 *>(i8)[ch] = make_uint2(lo, hi);
    } else if constexpr (DT == 2) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) word |= (uint32_t)(c[j] & 0xF) << (4 * j);
        reinterpret_cast<uint32_t *>(i4)[ch] = word;
    } else {
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) bits |= (uint32_t)(c[j] & 0x3) << (2 * j);
        reinterpret_cast<uint16_t *>(i2)[ch] = (uint16_t)bits;
    }
}

// Max |x| pass, then the encoding pass, of one block by one wave.
template <int R, int ST, int DT>
__device__ inline void encode_block(const DemoteSrc &src, const int64_t nch, int8_t *i8,
                                    uint8_t *i4, uint8_t *i2, float *scale_out, const int lane) {
    constexpr int qmax = DT == 1 ? 127 : DT == 2 ? 7 : DT == 3 ? 448 : 1;
    uint4 keep[R];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t ch = lane + 64 * j;
        keep[j] = ch < nch ? load_chunk<ST, true>(src, ch) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < R; ++j) amax = fmaxf(amax, absmax8<ST>(src, keep[j]));
    for (int64_t ch = lane + 64 * R; ch < nch; ch += 64)
        amax = fmaxf(amax, absmax8<ST>(src, load_chunk<ST>(src, ch)));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (scale_not_finite<ST>(src)) amax = __builtin_inff();
    // a block holding a non-finite value gets a NaN scale (and codes 0, since
    // no code is formed from a NaN scale), so every value read back from it
    // is NaN instead of a finite stand-in
    const float scale = amax == __builtin_inff() ? __builtin_nanf("")
                                                  : __fdiv_rn(amax, (float)qmax);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t ch = lane + 64 * j;
        if (ch < nch) encode8<ST, DT>(src, keep[j], scale, i8, i4, i2, ch);
    }
    for (int64_t ch = lane + 64 * R; ch < nch; ch += 64)
        encode8<ST, DT>(src, load_chunk<ST>(src, ch), scale, i8, i4, i2, ch);
    if (lane == 0) *scale_out = scale;
}

template <int R, int ST>
__device__ inline void dispatch_dst(int dt, const DemoteSrc &src, int64_t nch, int8_t *i8,
                                    uint8_t *i4, uint8_t *i2, float *sdst, int lane) {
    if (dt == CLS_I8) encode_block<R, ST, CLS_I8>(src, nch, i8, i4, i2, sdst, lane);
    else if (dt == CLS_I4) encode_block<R, ST, CLS_I4>(src, nch, i8, i4, i2, sdst, lane);
    else if (dt == CLS_F8) encode_block<R, ST, CLS_F8>(src, nch, i8, i4, i2, sdst, lane);
    else encode_block<R, ST, CLS_I2>(src, nch, i8, i4, i2, sdst, lane);
}

template <int R>
__device__ inline void dispatch_block(int st, int dt, const DemoteSrc &src, int64_t nch,
                                      int8_t *i8, uint8_t *i4, uint8_t *i2, float *sdst,
                                      int lane) {
    switch (st) {
        case CLS_HOT: dispatch_dst<R, CLS_HOT>(dt, src, nch, i8, i4, i2, sdst, lane); break;
        case CLS_I8: dispatch_dst<R, CLS_I8>(dt, src, nch, i8, i4, i2, sdst, lane); break;
        case CLS_I4: dispatch_dst<R, CLS_I4>(dt, src, nch, i8, i4, i2, sdst, lane); break;
        case CLS_F8: dispatch_dst<R, CLS_F8>(dt, src, nch, i8, i4, i2, sdst, lane); break;
        default: dispatch_dst<R, CLS_I2>(dt, src, nch, i8, i4, i2, sdst, lane); break;
    }
}

// One wave per (page i, kv head g, K or V) block, four blocks per
// workgroup.  Lane l owns the chunks l + 64 j.  A block of up to 64 * R
// chunks (P * D <= 2048 at R = 4) is read once and kept in registers
// between the max |x| pass and the encoding pass; a larger block is read a
// second time for the encoding.  No barrier: the waves are independent.
template <int R>
__global__ __launch_bounds__(256) void demote_kernel(const DemoteParams d) {
    const int lane = threadIdx.x & 63;
    // the wave's block index, held in scalar registers
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= (int64_t)d.n * d.num_kv_heads * 2) return;
    const int kv = (int)(unit & 1);
    const int g = (int)((unit >> 1) % d.num_kv_heads);
    const int i = (int)((unit >> 1) / d.num_kv_heads);
    // both entries are loaded before either is decoded
    const uint32_t se = (uint32_t)d.src_slots[i];
    const uint32_t de = (uint32_t)d.dst_entries[i];
    uint32_t sslot, slot;
    const int stier = entry_class(se, sslot);
    const int tier = entry_class(de, slot);
    if (tier == CLS_B1 && d.n_b1 > 0) return;  // archive_kernel's page
    auto in_pool = [&](int cls, uint32_t s) {
        return (cls == CLS_HOT && s < (uint32_t)d.num_blocks) ||
               (cls == CLS_I8 && s < (uint32_t)d.n_i8) || (cls == CLS_I4 && s < (uint32_t)d.n_i4) ||
               (cls == CLS_F8 && s < (uint32_t)d.n_f8) || (cls == CLS_I2 && s < (uint32_t)d.n_i2);
    };
    const bool dst_ok = tier != CLS_HOT && in_pool(tier, slot);
    const bool src_ok = in_pool(stier, sslot);
    float *sc = tier == CLS_I8   ? (kv ? d.i8_vs : d.i8_ks)
                : tier == CLS_I4 ? (kv ? d.i4_vs : d.i4_ks)
                : tier == CLS_F8 ? (kv ? d.f8_vs : d.f8_ks)
                                 : (kv ? d.i2_vs : d.i2_ks);
    if (!dst_ok || !src_ok) {
        if (lane == 0 && g == 0 && kv == 0 && d.rejected) atomicAdd(d.rejected, 1);
        // a bad source: the page turns its rows into NaN (a 1-bit source is
        // refused without writing)
        if (dst_ok && stier != CLS_B1 && lane == 0)
            sc[(int64_t)slot * d.num_kv_heads + g] = __builtin_nanf("");
        return;
    }
    const int64_t n = (int64_t)d.page_tokens * d.head_dim;  // multiple of 8
    const int64_t sblk = ((int64_t)sslot * d.num_kv_heads + g);
    DemoteSrc src;
    src.bf16 = d.kv_type == KV_BF16;
    src.scale = 1.0f;
    if (stier == 0) {
        src.base = reinterpret_cast<const uint8_t *>(kv ? d.v_pool : d.k_pool) + sblk * n * 2;
    } else if (stier == 1) {
        src.base = reinterpret_cast<const uint8_t *>(kv ? d.i8_v : d.i8_k) + sblk * n;
        src.scale = (kv ? d.i8_vs : d.i8_ks)[sblk];
    } else if (stier == 2) {
        src.base = (kv ? d.i4_v : d.i4_k) + sblk * (n / 2);
        src.scale = (kv ? d.i4_vs : d.i4_ks)[sblk];
    } else if (stier == CLS_I2) {
        src.base = (kv ? d.i2_v : d.i2_k) + sblk * (n / 4);
        src.scale = (kv ? d.i2_vs : d.i2_ks)[sblk];
    } else {
        src.base = (kv ? d.f8_v : d.f8_k) + sblk * n;
        src.scale = (kv ? d.f8_vs : d.f8_ks)[sblk];
    }

    const int64_t dst_base = ((int64_t)slot * d.num_kv_heads + g) * n;  // in elements
    int8_t *i8 = tier == 1   ? (kv ? d.i8_v : d.i8_k) + dst_base
                 : tier == 3 ? reinterpret_cast<int8_t *>(kv ? d.f8_v : d.f8_k) + dst_base
                             : nullptr;
    uint8_t *i4 = tier == 2 ? (kv ? d.i4_v : d.i4_k) + dst_base / 2 : nullptr;
    uint8_t *i2 = tier == CLS_I2 ? (kv ? d.i2_v : d.i2_k) + dst_base / 4 : nullptr;
    float *sdst = sc + (int64_t)slot * d.num_kv_heads + g;
    // one straight-line body per (source, destination) tier pair (the
    // choice is wave-uniform)
    dispatch_block<R>(stier, tier, src, n / 8, i8, i4, i2, sdst, lane);
}

// ---- 1-bit archive (sign bits, mean-|x| scale, FP16 outliers) -------------

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ inline uint32_t mag_key(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// Set bits of a wave mask in the lanes below this one / in all lanes.
__device__ inline int below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Threshold search over one key per lane (0 < k <= 64), bit by bit from the
// top; bits that no lane's key has set are skipped, as they cannot move t.
// Returns t with at least k lanes holding v >= t.  When a prefix t >= floor
// selects exactly k lanes the search stops there and `exact` is set: then
// exactly k lanes hold v >= t.  Otherwise t is the k-th largest v.  (Counts
// below `floor` may be incomplete, so no exit is taken there.)
__device__ inline uint32_t kth_largest_lane(uint32_t v, int k, uint32_t floor, bool &exact) {
    uint32_t o = v;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) o |= (uint32_t)__shfl_xor((int)o, sh);
    const uint32_t any = __builtin_amdgcn_readfirstlane(o);
    uint32_t t = 0;
    exact = false;
    for (int b = 30; b >= 0 && !exact; --b) {
        if (((any >> b) & 1u) == 0u) continue;  // uniform
        const uint32_t cand = t | (1u << b);
        const int c = (int)__popcll(__ballot(v >= cand));
        if (c >= k) t = cand;
        exact = c == k && cand >= floor;
    }
    return t;
}

// Encodes one block into the 1-bit format (one wave).  The outlier
// threshold T is the k-th largest magnitude key.  When the block's keys are
// held in registers, a lower bound t0 comes first: a threshold that at least
// k of the 64 lane maxima reach (then at least k keys do).  If at most 64
// keys reach t0, they are compacted into this wave's 64 words of LDS
// (`cand`), one per lane, and T is searched bit by bit over those alone.
// Otherwise T is found bit by bit from the top over the whole block; each
// pass counts the keys >= a candidate with one ballot per element (no
// cross-lane data movement).  Both searches stop early once a prefix selects
// exactly k keys, and both give the same outliers: the k largest keys, ties
// taken in index order.  Elements above T are outliers, and of those equal
// to T the lowest-indexed ones fill the remaining places (ranks in index
// order from lane-prefix bit counts).  The keys of the first R rounds of
// chunks stay in registers and their raw chunks in this wave's LDS (`stage`,
// R * 64 chunks, each lane reading back only what it wrote); later rounds are
// read again from memory per pass.
template <int R, int ST>
__device__ void archive_block(const DemoteSrc &src, const int64_t nch, uint8_t *signs,
                              float *scale_out, uint32_t *outs, const int kout, const int lane,
                              uint32_t *cand, uint4 *stage) {
    const int64_t n = nch * 8;
    const int k = (int)min((int64_t)kout, n);
    const int rounds = (int)((nch + 63) / 64);
    uint32_t key[R][8];  // 0 past the block: never >= a candidate (>= 1)
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t ch = lane + 64 * j;
        float x[8];
        if (ch < nch) {
            const uint4 w = load_chunk<ST>(src, ch);
            stage[64 * j + lane] = w;
            widen8<ST>(src, w, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) key[j][e] = ch < nch ? mag_key(x[e]) : 0u;
    }
    // keys >= c over the block (c >= 1; wave-uniform)
    auto count_at_least = [&](uint32_t c) {
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) cnt += __popcll(__ballot(key[j][e] >= c));
        for (int r = R; r < rounds; ++r) {
            const int64_t ch = lane + 64 * (int64_t)r;
            float x[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            if (ch < nch) widen8<ST>(src, load_chunk<ST>(src, ch), x);
#pragma unroll
            for (int e = 0; e < 8; ++e) cnt += __popcll(__ballot(ch < nch && mag_key(x[e]) >= c));
        }
        return cnt;
    };

    uint32_t T = 0;  // count(key >= T) >= k throughout
    int need = 0;
    bool selected = false;
    if (k > 0 && rounds <= R) {
        uint32_t lmax = 0;
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) lmax = max(lmax, key[j][e]);
        bool ex;
        // at least k lane maxima reach t0, so at least k keys do
        const uint32_t t0 = kth_largest_lane(lmax, k, 0u, ex);
        int c = 0;
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) c += key[j][e] >= t0 ? 1 : 0;
        int incl = c;  // inclusive prefix sum of c over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d);
            if (lane >= d) incl += t;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        // t0 >= 1 keeps the zero keys past the block out of the candidates
        if (t0 >= 1u && total <= 64) {
            int at = incl - c;
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (key[j][e] >= t0) cand[at++] = key[j][e];
            __builtin_amdgcn_wave_barrier();
            const uint32_t mine = lane < total ? cand[lane] : 0u;
            // only keys >= t0 were gathered: counts below t0 are short
            T = kth_largest_lane(mine, k, t0, ex);
            if (ex) --T;  // then key > T selects exactly the k outliers
            need = k - (int)__popcll(__ballot(mine > T));
            selected = true;
        }
    }
    if (k > 0 && !selected) {
        // A bit that no key has set never moves T: no key lies in [T + 2^b,
        // T + 2^(b+1)), so its count equals that of the higher candidate,
        // which fell short of k.  Its pass is skipped (16-bit sources leave
        // the low 13 to 16 bits of every key clear).
        uint32_t any = 0x7FFFFFFFu;
        if (rounds <= R) {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) o |= key[j][e];
#pragma unroll
            for (int sh = 32; sh >= 1; sh >>= 1) o |= (uint32_t)__shfl_xor((int)o, sh);
            any = __builtin_amdgcn_readfirstlane(o);
        }
        bool exact = false;
        for (int b = 30; b >= 0 && !exact; --b) {
            if (((any >> b) & 1u) == 0u) continue;  // uniform
            const uint32_t cand = T | (1u << b);
            const int c = count_at_least(cand);
            if (c >= k) T = cand;
            exact = c == k;
        }
        if (exact) --T;  // then key > T selects exactly the k outliers
        need = k - (T == 0x7FFFFFFFu ? 0 : count_at_least(T + 1));
    }

    // final pass over the chunks again: the first R rounds from LDS, later
    // ones from memory (the threshold passes keep only keys)
    int eq_base = 0, out_base = 0;
    double sum = 0.0;
    for (int r = 0; r < rounds; ++r) {
        const int64_t ch = lane + 64 * (int64_t)r;
        const bool valid = ch < nch;
        float x[8];
        if (valid) {
            widen8<ST>(src, r < R ? stage[64 * r + lane] : load_chunk<ST>(src, ch), x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
        // ties at T matter only while places are left for them (need > 0), and
        // their ranks only in rounds that hold one
        bool tie[8], any_tie = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            tie[e] = need > 0 && valid && mag_key(x[e]) == T;
            any_tie |= tie[e];
        }
        int rank = eq_base;
        if (__ballot(any_tie) != 0) {  // uniform
            int eq_tot = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint64_t m = __ballot(tie[e]);
                rank += below(m);
                eq_tot += __popcll(m);
            }
            eq_base += eq_tot;
        }
        bool is_out[8];
        int pos = out_base, out_tot = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            is_out[e] = k > 0 && valid && (mag_key(x[e]) > T || (tie[e] && rank < need));
            rank += tie[e] ? 1 : 0;
            const uint64_t m = __ballot(is_out[e]);
            pos += below(m);
            out_tot += __popcll(m);
        }
        out_base += out_tot;
        uint32_t byte = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (is_out[e]) {
                const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)x[e]);
                outs[pos++] = (uint32_t)(ch * 8 + e) | ((uint32_t)h << 16);
            } else if (valid) {
                sum += (double)fabsf(x[e]);
            }
            byte |= (x[e] < 0.0f ? 1u : 0u) << e;
        }
        if (valid) signs[ch] = (uint8_t)byte;
    }
    sum = wave_sum(sum);
    const int64_t m = n - k;
    if (lane == 0) *scale_out = m > 0 ? (float)(sum / (double)m) : 0.0f;
}

// One wave per (page i, kv head g, K or V) block whose destination is a
// 1-bit entry; every other page is demote_kernel's.
template <int R>
__global__ __launch_bounds__(256) void archive_kernel(const DemoteParams d) {
    __shared__ uint32_t s_cand[4][64];  // each wave's outlier candidates
    __shared__ uint4 s_stage[4][R * 64];  // each wave's register-round chunks
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= (int64_t)d.n * d.num_kv_heads * 2) return;
    const int kv = (int)(unit & 1);
    const int g = (int)((unit >> 1) % d.num_kv_heads);
    const int i = (int)((unit >> 1) / d.num_kv_heads);
    const uint32_t se = (uint32_t)d.src_slots[i];
    const uint32_t de = (uint32_t)d.dst_entries[i];
    uint32_t sslot, slot;
    const int stier = entry_class(se, sslot);
    const int tier = entry_class(de, slot);
    if (tier != CLS_B1) return;
    const bool dst_ok = slot < (uint32_t)d.n_b1;
    const bool src_ok = (stier == CLS_HOT && sslot < (uint32_t)d.num_blocks) ||
                        (stier == CLS_I8 && sslot < (uint32_t)d.n_i8) ||
                        (stier == CLS_I4 && sslot < (uint32_t)d.n_i4) ||
                        (stier == CLS_F8 && sslot < (uint32_t)d.n_f8) ||
                        (stier == CLS_I2 && sslot < (uint32_t)d.n_i2);
    const int64_t dblk = (int64_t)slot * d.num_kv_heads + g;
    float *sdst = (kv ? d.b1_vs : d.b1_ks) + dblk;
    if (!dst_ok || !src_ok) {
        if (lane == 0 && g == 0 && kv == 0 && d.rejected) atomicAdd(d.rejected, 1);
        if (dst_ok && stier != CLS_B1) {
            // poison the slot: NaN scale, and every outlier a NaN at index 0,
            // so no stale outlier decodes to a finite value
            if (lane == 0) *sdst = __builtin_nanf("");
            if (lane < d.b1_nout) ((kv ? d.b1_vo : d.b1_ko) + dblk * d.b1_nout)[lane] = 0x7E00u << 16;
        }
        return;
    }
    const int64_t n = (int64_t)d.page_tokens * d.head_dim;
    const int64_t sblk = (int64_t)sslot * d.num_kv_heads + g;
    DemoteSrc src;
    src.bf16 = d.kv_type == KV_BF16;
    src.scale = 1.0f;
    if (stier == CLS_HOT) {
        src.base = reinterpret_cast<const uint8_t *>(kv ? d.v_pool : d.k_pool) + sblk * n * 2;
    } else if (stier == CLS_I8) {
        src.base = reinterpret_cast<const uint8_t *>(kv ? d.i8_v : d.i8_k) + sblk * n;
        src.scale = (kv ? d.i8_vs : d.i8_ks)[sblk];
    } else if (stier == CLS_I4) {
        src.base = (kv ? d.i4_v : d.i4_k) + sblk * (n / 2);
        src.scale = (kv ? d.i4_vs : d.i4_ks)[sblk];
    } else if (stier == CLS_I2) {
        src.base = (kv ? d.i2_v : d.i2_k) + sblk * (n / 4);
        src.scale = (kv ? d.i2_vs : d.i2_ks)[sblk];
    } else {
        src.base = (kv ? d.f8_v : d.f8_k) + sblk * n;
        src.scale = (kv ? d.f8_vs : d.f8_ks)[sblk];
    }
    uint8_t *signs = (kv ? d.b1_v : d.b1_k) + dblk * (n / 8);
    uint32_t *outs = (kv ? d.b1_vo : d.b1_ko) + dblk * d.b1_nout;
    switch (stier) {
        case CLS_HOT: archive_block<R, CLS_HOT>(src, n / 8, signs, sdst, outs, d.b1_nout, lane, s_cand[threadIdx.x >> 6], s_stage[threadIdx.x >> 6]); break;
        case CLS_I8: archive_block<R, CLS_I8>(src, n / 8, signs, sdst, outs, d.b1_nout, lane, s_cand[threadIdx.x >> 6], s_stage[threadIdx.x >> 6]); break;
        case CLS_I4: archive_block<R, CLS_I4>(src, n / 8, signs, sdst, outs, d.b1_nout, lane, s_cand[threadIdx.x >> 6], s_stage[threadIdx.x >> 6]); break;
        case CLS_F8: archive_block<R, CLS_F8>(src, n / 8, signs, sdst, outs, d.b1_nout, lane, s_cand[threadIdx.x >> 6], s_stage[threadIdx.x >> 6]); break;
        default: archive_block<R, CLS_I2>(src, n / 8, signs, sdst, outs, d.b1_nout, lane, s_cand[threadIdx.x >> 6], s_stage[threadIdx.x >> 6]); break;
    }
}

// ---- reconstruction of pages into hot blocks --------------------------------

// Stores the 8 values of chunk ch of a hot block as kv_type (round to
// nearest even).
__device__ inline void store_hot8(void *dst, int64_t ch, int kv_type, const float (&x)[8]) {
    if (kv_type == KV_F32) {
        float4 *o = reinterpret_cast<float4 *>(dst) + 2 * ch;
        o[0] = make_float4(x[0], x[1], x[2], x[3]);
        o[1] = make_float4(x[4], x[5], x[6], x[7]);
        return;
    }
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint16_t a, b;
        if (kv_type == KV_BF16) {
            a = __builtin_bit_cast(uint16_t, (__bf16)x[2 * j]);
            b = __builtin_bit_cast(uint16_t, (__bf16)x[2 * j + 1]);
        } else {
            a = __builtin_bit_cast(uint16_t, (_Float16)x[2 * j]);
            b = __builtin_bit_cast(uint16_t, (_Float16)x[2 * j + 1]);
        }
        w[j] = (uint32_t)a | ((uint32_t)b << 16);
    }
    // streaming store: a promoted block is written once, whole
    const nt_u32x4 v = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4 *>(dst) + ch);
}

template <int ST>
__device__ void promote_codes(const DemoteSrc &src, int64_t nch, void *dst, int kv_type, int lane) {
    for (int64_t ch = lane; ch < nch; ch += 64) {
        float x[8];
        widen8<ST>(src, load_chunk<ST, true>(src, ch), x);
        store_hot8(dst, ch, kv_type, x);
    }
}

// One wave per (page i, kv head g, K or V) block.
__global__ __launch_bounds__(256) void promote_kernel(const PromoteParams q) {
    const DecodeParams &p = q.p;
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= (int64_t)q.n * p.num_kv_heads * 2) return;
    const int kv = (int)(unit & 1);
    const int g = (int)((unit >> 1) % p.num_kv_heads);
    const int i = (int)((unit >> 1) / p.num_kv_heads);
    const uint32_t se = (uint32_t)q.src_entries[i];
    const int32_t db = q.dst_blocks[i];
    uint32_t slot;
    const int cls = entry_class(se, slot);
    const bool dst_ok = db >= 0 && db < p.num_blocks;
    const bool src_ok = (cls == CLS_HOT && slot < (uint32_t)p.num_blocks) ||
                        (cls == CLS_I8 && slot < (uint32_t)p.n_i8) ||
                        (cls == CLS_I4 && slot < (uint32_t)p.n_i4) ||
                        (cls == CLS_F8 && slot < (uint32_t)p.n_f8) ||
                        (cls == CLS_I2 && slot < (uint32_t)p.n_i2) ||
                        (cls == CLS_B1 && slot < (uint32_t)p.n_b1);
    if (!dst_ok || !src_ok) {
        if (lane == 0 && g == 0 && kv == 0 && q.rejected) atomicAdd(q.rejected, 1);
        if (!dst_ok) return;
    }
    const int64_t n = (int64_t)p.page_tokens * q.head_dim;  // multiple of 8
    const int64_t nch = n / 8;
    const int eb = q.kv_type == KV_F32 ? 4 : 2;
    void *dst = reinterpret_cast<uint8_t *>(kv ? q.v_dst : q.k_dst) +
                ((int64_t)db * p.num_kv_heads + g) * n * eb;
    if (!src_ok) {  // a NaN block, so that rows reading it fail loudly
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_nanf("");
        for (int64_t ch = lane; ch < nch; ch += 64) store_hot8(dst, ch, q.kv_type, x);
        return;
    }
    const int64_t sblk = (int64_t)slot * p.num_kv_heads + g;
    if (cls == CLS_HOT) {  // a copy
        const uint4 *s4 = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint8_t *>(kv ? p.v_pool : p.k_pool) + sblk * n * eb);
        uint4 *d4 = reinterpret_cast<uint4 *>(dst);
        for (int64_t c = lane; c < n * eb / 16; c += 64) {
            const uint4 x = ld_stream16(s4 + c);
            const nt_u32x4 v = {x.x, x.y, x.z, x.w};
            __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4 *>(d4) + c);
        }
        return;
    }
    if (cls == CLS_B1) {
        const uint8_t *signs = (kv ? p.b1_v : p.b1_k) + sblk * nch;
        const float sc = (kv ? p.b1_vs : p.b1_ks)[sblk];
        const uint32_t *outs = (kv ? p.b1_vo : p.b1_ko) + sblk * p.b1_nout;
        // lane l holds outlier entry l; entries are applied in list order.
        // Four rounds of chunks are decoded into registers, then one scan of
        // the entries patches them (each entry's round and element are
        // wave-uniform).
        const uint32_t mine = lane < p.b1_nout ? outs[lane] : 0xFFFFu;
        for (int64_t r0 = 0; 64 * r0 < nch; r0 += 4) {
            float x[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t ch = lane + 64 * (r0 + u);
                const uint32_t byte = ch < nch ? signs[ch] : 0u;
#pragma unroll
                for (int j = 0; j < 8; ++j) x[u][j] = ((byte >> j) & 1u) ? -sc : sc;
            }
            for (int o = 0; o < p.b1_nout; ++o) {
                const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)mine, o);
                const int64_t c = (int64_t)((e & 0xFFFFu) >> 3);
                const int64_t u = c / 64 - r0;
                if (u < 0 || u >= 4) continue;  // uniform: another group of rounds
                const float v = (float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16));
                // this lane's element that the entry names (8: none)
                const int t = (c % 64) == lane ? (int)(e & 7u) : 8;
#pragma unroll
                for (int uu = 0; uu < 4; ++uu) {
                    if (uu != u) continue;  // uniform
#pragma unroll
                    for (int j = 0; j < 8; ++j) x[uu][j] = t == j ? v : x[uu][j];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t ch = lane + 64 * (r0 + u);
                if (ch < nch) store_hot8(dst, ch, q.kv_type, x[u]);
            }
        }
        return;
    }
    DemoteSrc src;
    src.bf16 = false;
    if (cls == CLS_I8) {
        src.base = reinterpret_cast<const uint8_t *>(kv ? p.i8_v : p.i8_k) + sblk * n;
        src.scale = (kv ? p.i8_vs : p.i8_ks)[sblk];
        promote_codes<CLS_I8>(src, nch, dst, q.kv_type, lane);
    } else if (cls == CLS_I4) {
        src.base = (kv ? p.i4_v : p.i4_k) + sblk * (n / 2);
        src.scale = (kv ? p.i4_vs : p.i4_ks)[sblk];
        promote_codes<CLS_I4>(src, nch, dst, q.kv_type, lane);
    } else if (cls == CLS_F8) {
        src.base = (kv ? p.f8_v : p.f8_k) + sblk * n;
        src.scale = (kv ? p.f8_vs : p.f8_ks)[sblk];
        promote_codes<CLS_F8>(src, nch, dst, q.kv_type, lane);
    } else {
        src.base = (kv ? p.i2_v : p.i2_k) + sblk * (n / 4);
        src.scale = (kv ? p.i2_vs : p.i2_ks)[sblk];
        promote_codes<CLS_I2>(src, nch, dst, q.kv_type, lane);
    }
}

}  // namespace

hipError_t launch_write_kv(const WriteKvParams &w, hipStream_t stream) {
    const int64_t total = (int64_t)w.total_q * w.num_kv_heads * w.head_dim * w.elem_bytes / 16;
    if (total <= 0) return hipSuccess;
    const int64_t blocks = min((total + 255) / 256, (int64_t)65536);
    hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w);
    return hipGetLastError();
}

hipError_t launch_demote(const DemoteParams &d, hipStream_t stream) {
    const int64_t waves = (int64_t)d.n * d.num_kv_heads * 2;  // one per block
    if (waves <= 0) return hipSuccess;
    hipLaunchKernelGGL(demote_kernel<4>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream,
                       d);
    if (d.n_b1 > 0) {  // pages bound for the 1-bit archive
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(archive_kernel<4>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                           stream, d);
    }
    return hipGetLastError();
}

hipError_t launch_promote(const PromoteParams &q, hipStream_t stream) {
    const int64_t waves = (int64_t)q.n * q.p.num_kv_heads * 2;  // one per block
    if (waves <= 0) return hipSuccess;
    hipLaunchKernelGGL(promote_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, q);
    return hipGetLastError();
}

}  // namespace atlas
