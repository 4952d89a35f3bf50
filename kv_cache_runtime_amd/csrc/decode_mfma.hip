// Paged decode attention on the matrix cores (gfx950), for 16-bit and tiered
// (f16 hot + int8 / int4 / FP8 cold) pages, head_dim 128 and 2, 4 or 8 query heads
// per kv head.  Same method and split-K structure as decode.hip: keys folded
// tile by tile with an online softmax (CFR-Atlas README, overview; ARGUS
// "Latency & Throughput Impact"), splits merged by log-sum-exp.
//
// gfx950 mapping.  A workgroup is 4 wave64s and owns one (row, kv head,
// split); each wave walks 64-token tiles, four 16-token groups each (a group
// lies in one page: pages are multiples of 16 tokens, tiles start at
// multiples of 64 positions).
//  * Scores: v_mfma_f32_16x16x32 with the query heads as A (rows, zero-padded
//    to 16) and 16 tokens as B (lane l supplies 8 dims of token l % 16), so
//    every K load is 16 tokens x 64 contiguous bytes; the result has token
//    l % 16 in lane l and heads 4 (l / 16) .. + 3 in its four registers.
//  * Softmax: one reference max per head, moved only when a tile's max
//    exceeds it by 2^8, reduced within 16-lane rows by DPP.  With four query
//    heads per kv head the heads sit in the first row only, so the four
//    16-token groups are first packed into the four rows (lane swaps) and
//    the softmax runs on one register per head.
//  * P.V: O^T[dim][head] += V^T[dim][token] P^T[token][head], also on
//    v_mfma_f32_16x16x32.  V rows are written to LDS as they are stored
//    (token-major, int codes widened to f16 on the way) and read back as the
//    token-contiguous operand by the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16); P goes through LDS the same way.  bf16 pages keep
//    P as a bf16 pair (hi + lo, ~16 significant bits); f16 pages use f16 P.
//  * The next tile's K and V are requested while the current tile computes
//    (software pipeline), so HBM latency overlaps the softmax and P.V.
//
// Tiered pages: the split's page-table entries are staged in LDS grouped by
// tier, and each tier's run of pages is padded to whole tiles, so every tile
// holds one tier and runs straight-line code for it.  K int8 / int4 / FP8
// codes become f16 in registers (exact), the K scale multiplies the finished score
// and the V scale the probability.  The matrix-core operand type is bf16 for
// bf16 pages (query used as stored) and f16 otherwise (the query converted to
// f16: exact for |q| in [2^-14, 65504], smaller magnitudes round with
// absolute error at most 2^-25).
#include "device.h"

namespace atlas {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kTileTok = 64;  // tokens per wave tile (one per lane for QK)
constexpr int kStagedPages = kDecodeStagedPages;  // page-table entries staged per split

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <int QT>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (QT == KV_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// Byte permutes that take the constant byte 0x64 from a register: placing a
// code byte u under it gives the f16 0x64uu = 1024 + u.
constexpr uint32_t kMagic64 = 0x64646464u;

// The f16 offsets that the code widenings below subtract.  With BIASED set
// a widening leaves the offset in (code + offset, still exact in f16); the
// score kernel then starts its dot products from -offset * sum(q) instead.
constexpr uint32_t kBiasI8 = 0x6480u;  // 1152
constexpr uint32_t kBiasI4 = 0x6408u;  // 1032
constexpr uint32_t kBiasI2 = 0x6402u;  // 1026

// int8 codes (4 per word) -> f16 pairs, exact: bias to unsigned (u = c + 128),
// form 0x64uu (= 1024 + u) with one byte permute per pair, subtract 1152.
template <bool BIASED = false>
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t u = w ^ 0x80808080u;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t a = __builtin_amdgcn_perm(kMagic64, u, 0x05010400u);  // bytes 0, 1
    const uint32_t b = __builtin_amdgcn_perm(kMagic64, u, 0x05030402u);  // bytes 2, 3
    if constexpr (BIASED) {
        lo = a;
        hi = b;
    } else {
        const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
        lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - bias);
        hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - bias);
    }
}

// int4 codes (8 per word, element e in nibble e, two's complement) -> f16
// pairs (e, e + 1), exact: bias to unsigned nibbles, gather the even and the
// odd elements into bytes, interleave them, place each byte under 0x64 and
// subtract 1032.
template <bool BIASED = false>
__device__ __forceinline__ void i4x8_to_f16x8(uint32_t w, uint32_t (&out)[4]) {
    const uint32_t u = w ^ 0x88888888u;
    const uint32_t ev = u & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6
    const uint32_t od = (u >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
    const uint32_t e03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);  // elements 0..3
    const uint32_t e47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);  // elements 4..7
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t p0 = __builtin_amdgcn_perm(kMagic64, e03, 0x05010400u);
    const uint32_t p1 = __builtin_amdgcn_perm(kMagic64, e03, 0x05030402u);
    const uint32_t p2 = __builtin_amdgcn_perm(kMagic64, e47, 0x05010400u);
    const uint32_t p3 = __builtin_amdgcn_perm(kMagic64, e47, 0x05030402u);
    if constexpr (BIASED) {
        out[0] = p0;
        out[1] = p1;
        out[2] = p2;
        out[3] = p3;
    } else {
        out[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p0) - bias);
        out[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p1) - bias);
        out[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p2) - bias);
        out[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p3) - bias);
    }
}

// FP8 E4M3 codes (4 per word) -> f16 pairs, exact, by the gfx950 hardware
// conversion (two codes per instruction).
__device__ __forceinline__ void f8x4_to_f16x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// INT2 codes (16 per word, element j in bits 2j, 2j + 1, two's complement)
// -> f16 pairs (2m, 2m + 1), exact: bias each field to unsigned (f + 2),
// place it under the f16 1024 and subtract 1026.
template <bool BIASED = false>
__device__ __forceinline__ void i2x16_to_f16x16(uint32_t w, uint32_t (&out)[8]) {
    const uint32_t u = w ^ 0xAAAAAAAAu;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 bias = {(_Float16)1026.0f, (_Float16)1026.0f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t b = 0x64006400u | ((u >> (4 * m)) & 3u) | (((u >> (4 * m + 2)) & 3u) << 16);
        out[m] = BIASED ? b : __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - bias);
    }
}

// Tile kinds.  kByte covers the one-byte code tiers (int8, FP8 when alt) and
// kSub the sub-byte ones (int4, INT2 when alt): same layout within a kind;
// alt is a compile-time constant of each run, so every class gets its own
// straight-line body.
constexpr int kHot = 0, kByte = 1, kSub = 2;
// 16-byte chunks per lane of one 16-token group, for K and for V (INT2 uses
// the low half of its one chunk)
template <int TIER>
constexpr int chunks() { return TIER == kHot ? 4 : TIER == kByte ? 2 : 1; }
// f16 offset that the K and V widenings leave in a class's operands (0: none)
template <int TIER, bool ALT>
constexpr uint32_t k_offset() {
    return TIER == kHot ? 0u : TIER == kByte ? (ALT ? 0u : kBiasI8) : (ALT ? kBiasI2 : kBiasI4);
}

// Raw K of row row0 + c of a group for this lane (row r of the 16-lane
// rows).  `base` is the first row of the group's (slot, kv head) block in its
// pool, negative for an entry outside its pool (then nothing is read and the
// call returns false).  Resident pages give the four operands directly
// (operand ks = dims 32 ks + 8 r .. + 8); tiered pages give dims 32 r .. 32 r
// + 31 as one run (hot: 64 bytes, int8: 32, int4: 16), widened by widen_k.
// The row is a wave-uniform base plus this lane's offset c.
template <int KV, int MODE, int TIER>
__device__ __forceinline__ bool load_k_group(const DecodeParams &p, int64_t base, int row0, int c,
                                             int r, uint4 (&kr)[chunks<TIER>()], bool alt) {
    if (base < 0) return false;
    const int64_t r0 = base + row0;
    if constexpr (TIER == kHot) {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(p.k_pool) + r0 * kD;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int d0 = MODE == MODE_TIERED ? 32 * r + 8 * ks : 32 * ks + 8 * r;
            // the tiered layout spreads a lane's 64-byte run over four loads,
            // each touching a quarter of every 64-byte stretch of the row: those
            // stay ordinary loads, so the later ones find the lines cached
            kr[ks] = MODE == MODE_TIERED ? *reinterpret_cast<const uint4 *>(src + (c * kD + d0))
                                         : ld_stream16(src + (c * kD + d0));
        }
    } else if constexpr (TIER == kByte) {
        const uint8_t *pool = alt ? p.f8_k : reinterpret_cast<const uint8_t *>(p.i8_k);
        // two loads per 32-byte run, each touching half of it: ordinary loads
        const uint4 *src = reinterpret_cast<const uint4 *>(pool + r0 * kD + (c * kD + 32 * r));
        kr[0] = src[0];
        kr[1] = src[1];
    } else if (alt) {  // INT2: dims 32 r .. 32 r + 31 are 8 bytes
        const uint2 v = ld_stream8(p.i2_k + r0 * (kD / 4) + (c * (kD / 4) + 8 * r));
        kr[0] = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        kr[0] = ld_stream16(p.i4_k + r0 * (kD / 2) + (c * (kD / 2) + 16 * r));
    }
    return true;
}

// Raw K -> the four 16-bit operands (codes widened to f16, exact; int8,
// int4 and INT2 codes keep their offset k_offset).
template <int TIER>
__device__ __forceinline__ void widen_k(const uint4 (&kr)[chunks<TIER>()], uint4 (&kb)[4],
                                       bool alt) {
    if constexpr (TIER == kHot) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[ks] = kr[ks];
    } else if constexpr (TIER == kByte) {
        const uint32_t w[8] = {kr[0].x, kr[0].y, kr[0].z, kr[0].w, kr[1].x, kr[1].y, kr[1].z, kr[1].w};
        if (alt) {  // FP8, run-uniform
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint32_t a, b, c, d;
                f8x4_to_f16x4(w[2 * ks], a, b);
                f8x4_to_f16x4(w[2 * ks + 1], c, d);
                kb[ks] = make_uint4(a, b, c, d);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint32_t a, b, c, d;
                i8x4_to_f16x4<true>(w[2 * ks], a, b);
                i8x4_to_f16x4<true>(w[2 * ks + 1], c, d);
                kb[ks] = make_uint4(a, b, c, d);
            }
        }
    } else if (alt) {  // INT2, run-uniform: 16 codes per word, two operands
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t o[8];
            i2x16_to_f16x16<true>(h ? kr[0].y : kr[0].x, o);
            kb[2 * h] = make_uint4(o[0], o[1], o[2], o[3]);
            kb[2 * h + 1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    } else {
        const uint32_t w[4] = {kr[0].x, kr[0].y, kr[0].z, kr[0].w};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint32_t o[4];
            i4x8_to_f16x8<true>(w[ks], o);
            kb[ks] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// Raw V of one 16-token group (rows row0 .. row0 + 15 of a page, one
// contiguous slab): lane l takes 16-byte chunks l, l + 64, ...  `base` as for
// load_k_group (false, nothing read, when negative).
template <int KV, int TIER>
__device__ __forceinline__ bool load_v_group(const DecodeParams &p, int64_t base, int row0,
                                             int lane, uint4 (&vr)[chunks<TIER>()], bool alt) {
    if (base < 0) return false;
    const int64_t r0 = base + row0;
    if constexpr (TIER == kHot) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.v_pool) + r0 * kD);
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = ld_stream16(src + 64 * i + lane);
    } else if constexpr (TIER == kByte) {
        const uint8_t *pool = alt ? p.f8_v : reinterpret_cast<const uint8_t *>(p.i8_v);
        const uint4 *src = reinterpret_cast<const uint4 *>(pool + r0 * kD);
        vr[0] = ld_stream16(src + lane);
        vr[1] = ld_stream16(src + 64 + lane);
    } else if (alt) {  // INT2: 8 bytes per lane
        const uint2 v = ld_stream8(reinterpret_cast<const uint2 *>(p.i2_v + r0 * (kD / 4)) + lane);
        vr[0] = make_uint4(v.x, v.y, 0u, 0u);
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(p.i4_v + r0 * (kD / 2));
        vr[0] = ld_stream16(src + lane);
    }
    return true;
}

constexpr int kVPitch = kD + 16;  // LDS row pitch of the V tile (16-bit elements, 72 words)

// Component-wise select (a select of whole uint4 values can turn into a
// select of addresses and a trip through scratch memory).
__device__ __forceinline__ uint4 keep_if(bool ok, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return make_uint4(ok ? a : 0u, ok ? b : 0u, ok ? c : 0u, ok ? d : 0u);
}

// Writes the group's V rows, as 16-bit operands, into rows base .. base + 15
// of the wave's LDS V tile; rows whose token is not visible (tok_ok false)
// are written as zeros, so NaN garbage in page tails never meets a zero
// probability.  Integer codes keep their f16 offset (k_offset), which the
// P.V step takes out again.
template <int TIER, typename TokOk>
__device__ __forceinline__ void store_v_group(uint16_t *vt, int base,
                                              const uint4 (&vr)[chunks<TIER>()], int lane,
                                              TokOk tok_ok, bool alt) {
    if constexpr (TIER == kHot) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // chunk 64 i + lane: token 4 i + lane / 16
            const int tok = 4 * i + (lane >> 4);
            *reinterpret_cast<uint4 *>(vt + (base + tok) * kVPitch + 8 * (lane & 15)) =
                keep_if(tok_ok(tok), vr[i].x, vr[i].y, vr[i].z, vr[i].w);
        }
    } else if constexpr (TIER == kByte) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {  // chunk 64 i + lane: token 8 i + lane / 8
            const int tok = 8 * i + (lane >> 3);
            const bool ok = tok_ok(tok);
            const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
            uint32_t h[8];
            if (alt) {  // FP8, run-uniform
#pragma unroll
                for (int j = 0; j < 4; ++j) f8x4_to_f16x4(w[j], h[2 * j], h[2 * j + 1]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) i8x4_to_f16x4<true>(w[j], h[2 * j], h[2 * j + 1]);
            }
            uint16_t *dst = vt + (base + tok) * kVPitch + 16 * (lane & 7);
            *reinterpret_cast<uint4 *>(dst) = keep_if(ok, h[0], h[1], h[2], h[3]);
            *reinterpret_cast<uint4 *>(dst + 8) = keep_if(ok, h[4], h[5], h[6], h[7]);
        }
    } else {
        const int tok = lane >> 2;  // chunk lane: token lane / 4, dims 32 (lane % 4) ..
        const bool ok = tok_ok(tok);
        uint16_t *dst = vt + (base + tok) * kVPitch + 32 * (lane & 3);
        if (alt) {  // INT2, run-uniform
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t o[8];
                i2x16_to_f16x16<true>(h ? vr[0].y : vr[0].x, o);
                *reinterpret_cast<uint4 *>(dst + 16 * h) = keep_if(ok, o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4 *>(dst + 16 * h + 8) = keep_if(ok, o[4], o[5], o[6], o[7]);
            }
        } else {
            const uint32_t w[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t o[4];
                i4x8_to_f16x8<true>(w[j], o);
                *reinterpret_cast<uint4 *>(dst + 8 * j) = keep_if(ok, o[0], o[1], o[2], o[3]);
            }
        }
    }
}

typedef short s16x4_lds_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// s supplies the address of 4 consecutive 16-bit elements; lane i receives
// element i % 4 of the chunks of lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12.
// With lane s of the group pointing at row k0 + s / 4, column n0 + 4 (s % 4)
// of a row-major tile, lane i receives column n0 + i of rows k0 .. k0 + 3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *ptr) {
    const s16x4_lds_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_lds_t *)(ptr));
    return __builtin_bit_cast(uint2, v);
}

template <int V>
struct TierC {  // compile-time int argument of the tile-run lambda
    static constexpr int value = V;
};

template <int QT, int KV, int G, int MODE>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(const DecodeParams p) {
    constexpr int NR = (G + 3) / 4;  // 16-lane rows holding score heads (4 heads per row)
    constexpr float kSlack = 8.0f;   // lazy rescale threshold (log2 units)
    constexpr float kPScale = 7.0f;  // probabilities kept relative to m_ref - 7
    constexpr int NP = QT == KV_BF16 ? 2 : 1;  // P operand parts (bf16: hi + lo)
    const float kNegInf = -__builtin_inff();

    // per wave: V tile of 32 tokens (one half of a 64-token tile at a time),
    // reused for the wave's final accumulators; P of 64 tokens x 16 heads
    __shared__ __attribute__((aligned(16))) uint16_t s_v[kWaves][32 * kVPitch];
    __shared__ __attribute__((aligned(16))) uint16_t s_p[kWaves][NP][kTileTok * 16];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane >> 4, c = lane & 15;  // 16-lane row, position in row

    // split index slowest: consecutive workgroups (which the dispatcher
    // spreads over the XCDs) take the same split of different (row, kv head)
    // pairs, so the mostly empty high splits of short contexts neither pile
    // onto a subset of XCDs nor interleave with the busy ones
    const int pairs = p.total_q * p.num_kv_heads;
    const int split = blockIdx.x / pairs;
    const int rg = blockIdx.x - split * pairs;
    const int g = rg % p.num_kv_heads;
    const int row = rg / p.num_kv_heads;

    int seq, nvis;
    const bool row_ok = map_row(p.rows, row, seq, nvis);
    const int T = p.split_tokens;
    const int t0 = split * T;
    if (split > 0 && t0 >= nvis) return;  // past this row's keys (uniform)
    const int t1 = min(t0 + T, nvis);

    // page-table entries of this split, staged once (a dependent global load
    // per tile would add a memory round trip before every K/V load); tiered
    // splits stage them grouped by tier (the host keeps every tiered split
    // within kStagedPages pages)
    __shared__ int32_t s_pages[kStagedPages];
    __shared__ int16_t s_lp[MODE == MODE_TIERED ? kStagedPages : 1];
    // ALiBi slopes (log2 units) of score rows 0..15, zero past G; read per
    // tile from LDS (published by the staging barrier below)
    __shared__ __attribute__((aligned(16))) float s_ab[16];
    if (tid < 16)
        s_ab[tid] = (p.pos.alibi != nullptr && tid < G) ? p.pos.alibi[g * G + tid] * kLog2e : 0.0f;
    const int32_t *trow = p.page_table + (int64_t)seq * p.max_pages;
    const int P = p.page_tokens;
    const int lp_first = t0 / P;
    const int lp_count = t1 > t0 ? (t1 - 1) / P - lp_first + 1 : 0;
    const bool staged = lp_count <= kStagedPages;
    int tier_count[kClasses] = {0, 0, 0, 0, 0, 0};
    // tiered splits: per staged page, the first row of its (slot, kv head)
    // block in its pool (-1 outside the pool) and its K and V scales, computed
    // once here instead of per tile and group
    __shared__ int64_t s_base[MODE == MODE_TIERED ? kStagedPages : 1];
    __shared__ float s_ksc[MODE == MODE_TIERED ? kStagedPages : 1];
    __shared__ float s_vsc[MODE == MODE_TIERED ? kStagedPages : 1];
    if constexpr (MODE == MODE_TIERED) {
        const int n_st = min(lp_count, kStagedPages);
        stage_pages_by_tier(trow + lp_first, n_st, s_pages, s_lp, tier_count);
        // staged positions are sorted by class: hot, int8, int4, FP8, INT2, other
        const int b1 = tier_count[0], b2 = b1 + tier_count[1], b3 = b2 + tier_count[2];
        const int b4 = b3 + tier_count[3], b5 = b4 + tier_count[4];
        for (int i = tid; i < n_st; i += 256) {
            const uint32_t sl = (uint32_t)s_pages[i];
            uint32_t cap = 0;
            const float *ksp = nullptr, *vsp = nullptr;
            if (i < b1) {
                cap = (uint32_t)p.num_blocks;
            } else if (i < b2) {
                cap = (uint32_t)p.n_i8, ksp = p.i8_ks, vsp = p.i8_vs;
            } else if (i < b3) {
                cap = (uint32_t)p.n_i4, ksp = p.i4_ks, vsp = p.i4_vs;
            } else if (i < b4) {
                cap = (uint32_t)p.n_f8, ksp = p.f8_ks, vsp = p.f8_vs;
            } else if (i < b5) {
                cap = (uint32_t)p.n_i2, ksp = p.i2_ks, vsp = p.i2_vs;
            }
            const bool ok = sl < cap;  // cap 0 past the attended classes
            const int64_t blk = (int64_t)sl * p.num_kv_heads + g;
            s_base[i] = ok ? blk * P : (int64_t)-1;
            s_ksc[i] = ok && ksp ? ksp[blk] : 1.0f;
            s_vsc[i] = ok && vsp ? vsp[blk] : 1.0f;
        }
        __syncthreads();
    } else {
        if (staged)
            for (int i = tid; i < lp_count; i += 256) s_pages[i] = trow[lp_first + i];
        __syncthreads();
    }

    // positional policy: the row sits at its own key, qpos
    const int qpos = nvis - 1;
    const bool rope = p.pos.rope != 0;
    const bool alibi = p.pos.alibi != nullptr;

    // A operand of the scores: query head c (zero for c >= G).  A rotated q
    // is no longer exact in 16 bits: rows G .. 2G - 1 (padding otherwise)
    // then carry the rounding remainder of heads 0 .. G - 1, and each head's
    // two score rows are added after the product.
    const bool lo_row = rope && c >= G && c < 2 * G;
    uint4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (c < G || lo_row) {
            // operand ks, lane row r holds dims 32 ks + 8 r (16-bit pages) or
            // 32 r + 8 ks (tiered pages, so each lane's K bytes are one run);
            // a dot product does not depend on how its terms are dealt out
            const int d0 = MODE == MODE_TIERED ? 32 * r + 8 * ks : 32 * ks + 8 * r;
            const int hq = c < G ? c : c - G;
            const int64_t q0 = ((int64_t)row * p.num_heads + g * G + hq) * kD + d0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x0 = load_elem(p.q, q0 + 2 * i, p.q_dtype);
                float x1 = load_elem(p.q, q0 + 2 * i + 1, p.q_dtype);
                if (rope) {
                    rope_rotate(x0, x1, qpos, rope_turns(d0 / 2 + i, kD, p.pos.rope_log2_theta));
                    if constexpr (QT == KV_BF16) {
                        const float h0 = bf16_round(x0), h1 = bf16_round(x1);
                        x0 = lo_row ? bf16_round(x0 - h0) : h0;
                        x1 = lo_row ? bf16_round(x1 - h1) : h1;
                    } else {
                        const float h0 = (float)(_Float16)x0, h1 = (float)(_Float16)x1;
                        x0 = lo_row ? x0 - h0 : x0;
                        x1 = lo_row ? x1 - h1 : x1;
                    }
                }
                if constexpr (QT == KV_BF16) {  // bf16-exact here
                    w[i] = (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xFFFF0000u);
                } else {
                    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                    const h2 h = {(_Float16)x0, (_Float16)x1};
                    w[i] = __builtin_bit_cast(uint32_t, h);
                }
            }
        }
        qf[ks] = make_uint4(w[0], w[1], w[2], w[3]);
    }

    // m_ref / l of heads 4 r + i (score layout); acc[mb][i] = O^T[dim
    // 16 mb + 4 r + i][head c] (P.V result layout; columns c >= G unused)
    float m_ref[4], l[4];
    f32x4_t acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_ref[i] = kNegInf;
        l[i] = 0.0f;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    bool bad = !row_ok;

    uint16_t *vt = s_v[wave];
    uint16_t *pt = s_p[wave][0];
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto in_range = [&](int tok) { return tok >= t0 && tok < t1; };

    if constexpr (G == 4) {  // the P columns of heads 4-15 are never written
#pragma unroll
        for (int part = 0; part < NP; ++part)
#pragma unroll
            for (int j = 0; j < kTileTok * 16 / (64 * 8); ++j)
                *reinterpret_cast<uint4 *>(pt + part * kTileTok * 16 + 8 * (lane + 64 * j)) =
                    make_uint4(0u, 0u, 0u, 0u);
    }

    // Walks the tiles of one run of pages with one tier: the whole split in
    // token order (natural), or the sp .. sp + np - 1 staged entries of a
    // tier.  Each wave takes every fourth tile of the run.
    auto run = [&](auto tier_c, auto alt_c, auto natural_c, int sp, int np) {
        constexpr int TIER = decltype(tier_c)::value;
        constexpr bool alt = decltype(alt_c)::value != 0;  // FP8 / INT2 of a code width
        constexpr bool natural = decltype(natural_c)::value != 0;
        constexpr int NC = chunks<TIER>();
        const int n_pos = natural ? t1 - t0 : np * P;
        const int n_tiles = n_pos > 0 ? (n_pos + kTileTok - 1) / kTileTok : 0;
        if (n_tiles == 0) return;

        // Integer-code K and V operands carry the f16 offset b (code + b is
        // exact).  Each score starts from -b * sum(q) of its row instead of zero:
        // one product of q with a constant-b operand, in the score layout
        // (the remainder rows of a rotated q included).  The P.V step removes
        // b * sum(P) with a second product per 32 tokens.  This saves the
        // subtraction of b from every widened code.
        f32x4_t s0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        constexpr uint32_t kOff = k_offset<TIER, alt>();
        if constexpr (kOff != 0u) {
            static_assert(QT == KV_F16, "the offsets are f16 values");
            const uint32_t bb = kOff | (kOff << 16);
            const uint4 ob = make_uint4(bb, bb, bb, bb);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) s0 = mfma16<QT>(qf[ks], ob, s0);
#pragma unroll
            for (int i = 0; i < 4; ++i) s0[i] = -s0[i];
        }
        // the P.V operand that removes the V offset: -b in every element
        constexpr uint32_t kNeg = kOff | 0x8000u;
        const uint4 vneg = make_uint4(kNeg | (kNeg << 16), kNeg | (kNeg << 16),
                                      kNeg | (kNeg << 16), kNeg | (kNeg << 16));

        // the 16-position groups of a tile: first token, slot and liveness,
        // all wave-uniform (a group lies in one page)
        struct Groups {
            int tok[4];       // first token
            int row[4];       // its row in the page
            int64_t base[4];  // first row of the (slot, kv head) block, -1 outside the pool
            float ks[4], vs[4];  // K and V scales (1 for resident pages)
            bool live[4];
        };
        auto page_div = [&](int x) {  // x / P, x < 2^31
            return (int)((__umulhi((uint32_t)x, p.p_magic) + (uint32_t)x) >> p.p_shift);
        };
        auto groups_of = [&](int tile, Groups &G_) {
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                const int q = tile * kTileTok + 16 * tg;
                bool live;
                int tok, row0;
                if constexpr (natural) {
                    tok = t0 + q;
                    live = tile < n_tiles && tok < t1;
                    const int lp = page_div(tok);
                    row0 = tok - lp * P;
                    const uint32_t ent = __builtin_amdgcn_readfirstlane(
                        live ? (uint32_t)(staged ? s_pages[lp - lp_first] : trow[lp]) : 0u);
                    G_.base[tg] = ent < (uint32_t)p.num_blocks
                                      ? ((int64_t)ent * p.num_kv_heads + g) * P : (int64_t)-1;
                    G_.ks[tg] = 1.0f;
                    G_.vs[tg] = 1.0f;
                } else {
                    const int pi = page_div(q);
                    live = tile < n_tiles && pi < np;
                    // unconditional reads (index kept inside the staged table), so the
                    // four groups' LDS reads are in flight together
                    const int si = min(sp + (live ? pi : 0), kStagedPages - 1);
                    const int lpv = s_lp[si];
                    const int64_t bv = s_base[si];
                    const float ksv = s_ksc[si], vsv = s_vsc[si];
                    const int lp = lp_first + (live ? lpv : 0);
                    row0 = q - pi * P;
                    tok = lp * P + row0;
                    const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)bv);
                    const uint32_t bhi =
                        __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)bv >> 32));
                    G_.base[tg] = (int64_t)(((uint64_t)bhi << 32) | blo);
                    G_.ks[tg] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ksv)));
                    G_.vs[tg] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vsv)));
                }
                G_.tok[tg] = __builtin_amdgcn_readfirstlane(tok);
                G_.row[tg] = __builtin_amdgcn_readfirstlane(row0);
                G_.live[tg] = live;
            }
        };
        uint4 kr[4][NC], vr[4][NC];
        float kscale[4], vscale[4];
        bool kok[4], vok[4];
        // A cold page's V scale multiplies the probabilities before they
        // become f16 operands.  The reference max of a tile is taken as its
        // score max plus lv = max(0, ceil(log2(largest V scale of the tile))):
        // the lazy rescale then bounds p by 2^(15 - lv), so p * scale <= 2^15
        // stays finite.  Integer steps on the (wave-uniform) scale bits.
        auto v_headroom = [&]() -> float {
            if constexpr (TIER == kHot) {
                return 0.0f;
            } else {
                float vm = 0.0f;
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) vm = vok[tg] ? fmaxf(vm, fabsf(vscale[tg])) : vm;
                const uint32_t b = __float_as_uint(vm);
                const int e = (int)(b >> 23) - 127 + ((b & 0x7FFFFFu) != 0u ? 1 : 0);
                return (float)max(e, 0);
            }
        };

        // Four query heads per kv head: the score tiles hold them in the first
        // 16 lanes only.  The softmax of a 64-token tile then runs on one packed
        // register per head instead of four: lane (r, c) holds token 16 r + c
        // (group r), moved there by two 16-lane swaps and a 32-lane swap.  The
        // head max and the rescale factors are wave-uniform; P is written for
        // heads 0-3 (the other columns of the P tile stay zero).
        auto softmax_packed = [&](const f32x4_t (&sc)[4], const float (&kf)[4],
                                  const bool (&kvalid)[4], const int (&tok)[4]) {
            float ps[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const auto s01 = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(sc[0][i]), __float_as_uint(sc[1][i]), false, false);
                const auto s23 = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(sc[2][i]), __float_as_uint(sc[3][i]), false, false);
                const auto sw = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
                ps[i] = __uint_as_float(sw[0]);
            }
            // this lane's group r: K scale, visibility, V scale, first token.
            // Two-level selects on the bits of r, from values held one by one (a
            // select chain over an array would become an indexed stack load).
            const bool r1 = (r & 1) != 0, r2 = (r & 2) != 0;
            auto pick = [&](auto a0, auto a1, auto a2, auto a3) {
                return r2 ? (r1 ? a3 : a2) : (r1 ? a1 : a0);
            };
            const float kf0 = kf[0], kf1 = kf[1], kf2 = kf[2], kf3 = kf[3];
            const float kfl = pick(kf0, kf1, kf2, kf3);
            const bool v0 = kvalid[0], v1 = kvalid[1], v2 = kvalid[2], v3 = kvalid[3];
            const bool vis = pick(v0, v1, v2, v3);
            float vsl = 1.0f;
            if constexpr (TIER != kHot) {
                const float vs0 = vscale[0], vs1 = vscale[1], vs2 = vscale[2], vs3 = vscale[3];
                vsl = pick(vs0, vs1, vs2, vs3);
            }
            const int tk0 = tok[0], tk1 = tok[1], tk2 = tok[2], tk3 = tok[3];
            const int tokl = pick(tk0, tk1, tk2, tk3);
    #pragma unroll
            for (int i = 0; i < 4; ++i) ps[i] = vis ? ps[i] * kfl : kNegInf;
            if (alibi) {  // wave-uniform
                const float4 ab = *reinterpret_cast<const float4 *>(&s_ab[0]);
                const float dist = (float)(tokl + c - qpos);
                ps[0] = fmaf(ab.x, dist, ps[0]);
                ps[1] = fmaf(ab.y, dist, ps[1]);
                ps[2] = fmaf(ab.z, dist, ps[2]);
                ps[3] = fmaf(ab.w, dist, ps[3]);
            }
            bool move_any = false;
            float alpha[4];
            const float lv = v_headroom();
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                float mx = ps[i];
                mx = __builtin_elementwise_maximum(mx, dpp_f<0x128>(mx));
                mx = __builtin_elementwise_maximum(mx, dpp_f<0x124>(mx));
                mx = __builtin_elementwise_maximum(mx, dpp_f<0x122>(mx));
                mx = __builtin_elementwise_maximum(mx, dpp_f<0x121>(mx));
                const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                __float_as_uint(mx), false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(h[0]), __uint_as_float(h[1]));
                const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx),
                                                                __float_as_uint(mx), false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(q[0]), __uint_as_float(q[1]));
                mx += lv;
                const bool move = mx > m_ref[i] + kSlack;  // also true on the first tile
                const float m_new = move ? mx : m_ref[i];
                alpha[i] = move ? __builtin_amdgcn_exp2f(m_ref[i] - m_new) : 1.0f;
                move_any = move_any || move;
                m_ref[i] = m_new;
            }
            if (__any(move_any)) {  // wave-uniform
    #pragma unroll
                for (int i = 0; i < 4; ++i) l[i] *= alpha[i];
                const float ac = c == 0 ? alpha[0] : c == 1 ? alpha[1] : c == 2 ? alpha[2]
                                 : c == 3 ? alpha[3] : 1.0f;
    #pragma unroll
                for (int mb = 0; mb < 8; ++mb) acc[mb] *= ac;
            }
            float pr[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float m_off = (m_ref[i] == kNegInf) ? 0.0f : m_ref[i] - kPScale;
                pr[i] = __builtin_amdgcn_exp2f(ps[i] - m_off);
                if constexpr (TIER != kHot) {
                    l[i] += pr[i];
                    pr[i] *= vsl;
                }
            }
            uint2 hi, lo;
            if constexpr (QT == KV_BF16) {
                uint32_t hb[4], lb[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t u = __float_as_uint(pr[i]);
                    const uint32_t h16 = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                    const float hf = __uint_as_float(h16 << 16);
                    const uint32_t v = __float_as_uint(pr[i] - hf);
                    const uint32_t l16 = (v + 0x7FFFu + ((v >> 16) & 1u)) >> 16;
                    hb[i] = h16;
                    lb[i] = l16;
                    l[i] += hf + __uint_as_float(l16 << 16);
                }
                hi = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                lo = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
            } else {
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                const h2 a = {(_Float16)pr[0], (_Float16)pr[1]};
                const h2 b = {(_Float16)pr[2], (_Float16)pr[3]};
                if constexpr (TIER == kHot) {
                    l[0] += (float)a[0];
                    l[1] += (float)a[1];
                    l[2] += (float)b[0];
                    l[3] += (float)b[1];
                }
                hi = make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
                lo = make_uint2(0u, 0u);
            }
            *reinterpret_cast<uint2 *>(pt + (16 * r + c) * 16) = hi;
            if constexpr (NP == 2) *reinterpret_cast<uint2 *>(pt + kTileTok * 16 + (16 * r + c) * 16) = lo;
        };
        auto load_k = [&](const Groups &G_, int tg) {
            kok[tg] = G_.live[tg];
            kscale[tg] = G_.ks[tg];
            if (kok[tg] && !load_k_group<KV, MODE, TIER>(p, G_.base[tg], G_.row[tg], c, r,
                                                         kr[tg], alt)) {
                bad = true;
                kok[tg] = false;
            }
            if (!kok[tg]) {  // uniform: a dead group scores zeros (masked below)
#pragma unroll
                for (int i = 0; i < NC; ++i) kr[tg][i] = make_uint4(0u, 0u, 0u, 0u);
            }
        };
        auto load_v = [&](const Groups &G_, int tg) {
            vok[tg] = G_.live[tg];
            vscale[tg] = G_.vs[tg];
            if (vok[tg] && !load_v_group<KV, TIER>(p, G_.base[tg], G_.row[tg], lane, vr[tg],
                                                   alt)) {
                bad = true;
                vok[tg] = false;
            }
        };

        // software pipeline: the next tile's K is requested right after this
        // tile's scores, its V groups as soon as this tile's are in LDS
        Groups cur;
        groups_of(wave_u, cur);
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            load_k(cur, tg);
            load_v(cur, tg);
        }

        for (int tile = wave_u; tile < n_tiles; tile += kWaves) {
            Groups nxt;
            groups_of(tile + kWaves, nxt);

            // ---- scores: sc[tg][i] = head 4 r + i, token tok[tg] + c
            // (log2 domain)
            f32x4_t sc[4];
            bool kvalid[4];
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                kvalid[tg] = kok[tg] && in_range(cur.tok[tg] + c);
                uint4 kb[4];
                widen_k<TIER>(kr[tg], kb, alt);
                sc[tg] = s0;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) sc[tg] = mfma16<QT>(qf[ks], kb[ks], sc[tg]);
            }
            if (rope) {  // add the remainder rows G .. 2G - 1 to heads 0 .. G - 1
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) {
                    if constexpr (G == 2) {
                        sc[tg][0] += sc[tg][2];
                        sc[tg][1] += sc[tg][3];
                    } else if constexpr (G == 4) {  // rows 4..7 sit 16 lanes up
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sc[tg][i] += __int_as_float(
                                __builtin_amdgcn_ds_swizzle(__float_as_int(sc[tg][i]), 0x401F));
                    } else {  // rows 8..15 sit 32 lanes up
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t u = __float_as_uint(sc[tg][i]);
                            const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
                            sc[tg][i] += __uint_as_float(sw[1]);  // lane l < 32: lane l + 32
                        }
                    }
                }
            }
            float kf[4];  // hot pages carry no scale
#pragma unroll
            for (int tg = 0; tg < 4; ++tg)
                kf[tg] = TIER == kHot ? p.scale_log2 : kscale[tg] * p.scale_log2;
            // next tile's K (its registers are free once the scores are issued)
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) load_k(nxt, tg);
            if constexpr (G == 4) {
                softmax_packed(sc, kf, kvalid, cur.tok);
            } else {
    #pragma unroll
                for (int tg = 0; tg < 4; ++tg) {
    #pragma unroll
                    for (int i = 0; i < 4; ++i) sc[tg][i] = kvalid[tg] ? sc[tg][i] * kf[tg] : kNegInf;
                }
                if (alibi) {  // wave-uniform
                    const float4 ab = *reinterpret_cast<const float4 *>(&s_ab[4 * r]);
    #pragma unroll
                    for (int tg = 0; tg < 4; ++tg) {
                        const float dist = (float)(cur.tok[tg] + c - qpos);
                        sc[tg][0] = fmaf(ab.x, dist, sc[tg][0]);
                        sc[tg][1] = fmaf(ab.y, dist, sc[tg][1]);
                        sc[tg][2] = fmaf(ab.z, dist, sc[tg][2]);
                        sc[tg][3] = fmaf(ab.w, dist, sc[tg][3]);
                    }
                }

                // ---- online softmax, one reference max per head (uniform in a row)
                bool move_any = false;
                float alpha[4];
                const float lv = v_headroom();
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // IEEE maximum (v_maximum3_f32): no operand canonicalisation,
                    // and a NaN score (from NaN keys) propagates into the row
                    float mx = __builtin_elementwise_maximum(
                        __builtin_elementwise_maximum(sc[0][i], sc[1][i]),
                        __builtin_elementwise_maximum(sc[2][i], sc[3][i]));
                    mx = __builtin_elementwise_maximum(mx, dpp_f<0x128>(mx));
                    mx = __builtin_elementwise_maximum(mx, dpp_f<0x124>(mx));
                    mx = __builtin_elementwise_maximum(mx, dpp_f<0x122>(mx));
                    mx = __builtin_elementwise_maximum(mx, dpp_f<0x121>(mx));
                    mx += lv;
                    const bool move = mx > m_ref[i] + kSlack;  // also true on the first tile
                    const float m_new = move ? mx : m_ref[i];
                    alpha[i] = move ? __builtin_amdgcn_exp2f(m_ref[i] - m_new) : 1.0f;
                    move_any = move_any || move;
                    m_ref[i] = m_new;
                }
                if (__any(move_any)) {  // wave-uniform
    #pragma unroll
                    for (int i = 0; i < 4; ++i) l[i] *= alpha[i];
                    // alpha of head c, from the score layout (row c / 4, register c % 4)
                    float ac = 1.0f;
    #pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float ah = __int_as_float(
                            __builtin_amdgcn_readlane(__float_as_int(alpha[h & 3]), 16 * (h >> 2)));
                        ac = c == h ? ah : ac;
                    }
    #pragma unroll
                    for (int mb = 0; mb < 8; ++mb) acc[mb] *= ac;
                }
                // probabilities of token tok[tg] + c, heads 4 r .. 4 r + 3 -> P
                // tile (token-major, 16 heads), scaled by the group's V scale.
                // Resident pages add the rounded weights the matrix cores use to
                // l, so the normalisation matches them exactly (a constant V row
                // comes back unchanged); cold pages add the unscaled weights.
    #pragma unroll
                for (int tg = 0; tg < 4; ++tg) {
                    float pr[4];
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float m_off = (m_ref[i] == kNegInf) ? 0.0f : m_ref[i] - kPScale;
                        pr[i] = __builtin_amdgcn_exp2f(sc[tg][i] - m_off);
                        if constexpr (TIER != kHot) {
                            l[i] += pr[i];
                            pr[i] *= vscale[tg];
                        }
                    }
                    uint2 hi, lo;
                    if constexpr (QT == KV_BF16) {
                        uint32_t hb[4], lb[4];
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // round to nearest even; the remainder is exact in
                            // f32, and so is hi + lo
                            const uint32_t u = __float_as_uint(pr[i]);
                            const uint32_t h16 = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                            const float hf = __uint_as_float(h16 << 16);
                            const uint32_t v = __float_as_uint(pr[i] - hf);
                            const uint32_t l16 = (v + 0x7FFFu + ((v >> 16) & 1u)) >> 16;
                            hb[i] = h16;
                            lb[i] = l16;
                            l[i] += hf + __uint_as_float(l16 << 16);
                        }
                        hi = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                        lo = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
                    } else {
                        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                        const h2 a = {(_Float16)pr[0], (_Float16)pr[1]};
                        const h2 b = {(_Float16)pr[2], (_Float16)pr[3]};
                        if constexpr (TIER == kHot) {
                            l[0] += (float)a[0];
                            l[1] += (float)a[1];
                            l[2] += (float)b[0];
                            l[3] += (float)b[1];
                        }
                        hi = make_uint2(__builtin_bit_cast(uint32_t, a),
                                        __builtin_bit_cast(uint32_t, b));
                        lo = make_uint2(0u, 0u);
                    }
                    *reinterpret_cast<uint2 *>(pt + (16 * tg + c) * 16 + 4 * r) = hi;
                    if constexpr (NP == 2)
                        *reinterpret_cast<uint2 *>(pt + kTileTok * 16 + (16 * tg + c) * 16 + 4 * r) = lo;
                }
            }

            // ---- P.V on the matrix cores, one 32-token half at a time
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int tg = 2 * half + j;
                    const bool live = vok[tg];
                    const int tb = cur.tok[tg];
                    if (live && tb >= t0 && tb + 16 <= t1)  // whole group visible (uniform)
                        store_v_group<TIER>(vt, 16 * j, vr[tg], lane, [](int) { return true; }, alt);
                    else
                        store_v_group<TIER>(vt, 16 * j, vr[tg], lane,
                                            [&](int tok) { return live && in_range(tb + tok); }, alt);
                    load_v(nxt, tg);  // this group's registers are free again
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // Contraction index k = 8 r + e of lane row r stands for
                // token 4 r + e (e < 4) or 16 + 4 r + e - 4 (e >= 4) of the
                // half, for A and B alike, so that the 32 lanes serviced
                // together by one transposing read touch 8 consecutive tile
                // rows (no bank conflicts with the 72-word row pitch).
                // B = P^T: lane supplies those tokens of head c
                const int s4 = c >> 2, s1 = c & 3;  // this lane's address in its group
                uint4 bp[NP];
#pragma unroll
                for (int part = 0; part < NP; ++part) {
                    const uint16_t *base = pt + part * kTileTok * 16;
                    const uint2 x0 = lds_read_tr16(base + (32 * half + 4 * r + s4) * 16 + 4 * s1);
                    const uint2 x1 =
                        lds_read_tr16(base + (32 * half + 16 + 4 * r + s4) * 16 + 4 * s1);
                    bp[part] = make_uint4(x0.x, x0.y, x1.x, x1.y);
                }
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) {
                    // A = V^T: lane supplies dim 16 mb + c of the same tokens
                    const uint2 y0 = lds_read_tr16(vt + (4 * r + s4) * kVPitch + 16 * mb + 4 * s1);
                    const uint2 y1 =
                        lds_read_tr16(vt + (16 + 4 * r + s4) * kVPitch + 16 * mb + 4 * s1);
                    const uint4 av = make_uint4(y0.x, y0.y, y1.x, y1.y);
#pragma unroll
                    for (int part = 0; part < NP; ++part)
                        acc[mb] = mfma16<QT>(av, bp[part], acc[mb]);
                    // integer V codes carry the offset b: take b * sum(P) of
                    // these 32 tokens out at once (a constant -b operand), so
                    // the offset never accumulates across tiles
                    if constexpr (kOff != 0u) acc[mb] = mfma16<QT>(vneg, bp[0], acc[mb]);
                }
            }
            __builtin_amdgcn_wave_barrier();  // P and V tiles are rewritten by the next tile
            cur = nxt;
        }
    };

    if constexpr (MODE == MODE_TIERED) {
        // one straight-line run body per class: hot, int8, int4, FP8, INT2
        // (a run-time choice between two classes inside one body costs more
        // than the larger code)
        const int c01 = tier_count[0] + tier_count[1];
        const int c012 = c01 + tier_count[2];
        run(TierC<kHot>{}, TierC<0>{}, TierC<0>{}, 0, tier_count[0]);
        run(TierC<kByte>{}, TierC<0>{}, TierC<0>{}, tier_count[0], tier_count[1]);
        run(TierC<kSub>{}, TierC<0>{}, TierC<0>{}, c01, tier_count[2]);
        run(TierC<kByte>{}, TierC<1>{}, TierC<0>{}, c012, tier_count[3]);
        run(TierC<kSub>{}, TierC<1>{}, TierC<0>{}, c012 + tier_count[3], tier_count[4]);
        if (tier_count[5] > 0 || !staged) bad = true;
    } else {
        run(TierC<kHot>{}, TierC<0>{}, TierC<1>{}, 0, 0);
    }

    // ---- merge the waves: l is summed over the 16 lanes of the row holding
    // the head; the wave's accumulators go to its own (now unused) V tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        l[i] = row16_sum(l[i]);
        if constexpr (G == 4) {  // packed softmax: the head's sum spans all four rows
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[i]),
                                                            __float_as_uint(l[i]), false, false);
            l[i] = __uint_as_float(h[0]) + __uint_as_float(h[1]);
            const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(l[i]),
                                                            __float_as_uint(l[i]), false, false);
            l[i] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
        }
    }
    __builtin_amdgcn_wave_barrier();
    float *s_acc = reinterpret_cast<float *>(vt);  // [G][kD] of this wave
    if (c < G) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_acc[c * kD + 16 * mb + 4 * r + i] = acc[mb][i];
    }
    if (c == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * r + i;
            if (r < NR && h < G) {
                s_m[wave][h] = (m_ref[i] == kNegInf) ? kNegInf : m_ref[i] - kPScale;
                s_l[wave][h] = l[i];
            }
        }
    }
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;

    const int nsplit = splits_of(nvis, T);
    const bool final_here = p.direct || nsplit == 1;
    if (wave == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = s_m[0][h];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
            const float M_use = (M == kNegInf) ? 0.0f : M;
            float fw[kWaves];
            float L = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                fw[w] = __builtin_amdgcn_exp2f(s_m[w][h] - M_use);
                L += fw[w] * s_l[w][h];
            }
            const int64_t orow = (int64_t)row * p.num_heads + g * G + h;
            const float qnan = __builtin_nanf("");
            for (int col = lane; col < kD; col += 64) {
                float o = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w)
                    o = fmaf(fw[w], reinterpret_cast<const float *>(s_v[w])[h * kD + col], o);
                o = L > 0.0f ? o / L : 0.0f;
                if (any_bad) o = qnan;
                if (final_here) p.out[orow * kD + col] = o;
                else p.part_o[(orow * p.max_splits + split) * kD + col] = o;
            }
            if (lane == 0) {
                float lse = L > 0.0f ? (M + log2f(L)) * kLn2 : kNegInf;
                if (any_bad) lse = qnan;
                if (final_here) p.lse[orow] = lse;
                else p.part_lse[orow * p.max_splits + split] = lse;
            }
        }
    }
}

template <int QT, int KV, int MODE>
hipError_t by_group(const DecodeParams &p, int group, hipStream_t s) {
    const int64_t blocks = (int64_t)p.total_q * p.num_kv_heads * p.max_splits;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(256);
    switch (group) {
        case 2: hipLaunchKernelGGL((decode_mfma_kernel<QT, KV, 2, MODE>), grid, block, 0, s, p); break;
        case 4: hipLaunchKernelGGL((decode_mfma_kernel<QT, KV, 4, MODE>), grid, block, 0, s, p); break;
        case 8: hipLaunchKernelGGL((decode_mfma_kernel<QT, KV, 8, MODE>), grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(int kv_type, int head_dim, int group, int mode, int page_tokens,
                           int split_tokens) {
    if (head_dim != kD || (group != 2 && group != 4 && group != 8)) return false;
    if (mode == MODE_PLAIN) return kv_type == KV_BF16 || kv_type == KV_F16;
    // a tiered split must fit the LDS staging of its page-table entries
    // (a split starting inside a page touches one page more)
    if (mode == MODE_TIERED)
        return kv_type == KV_F16 && split_tokens / page_tokens + 2 <= kDecodeStagedPages;
    return false;
}

hipError_t launch_decode_mfma(const DecodeParams &p, int kv_type, int group, int mode,
                              hipStream_t stream) {
    if (mode == MODE_PLAIN && kv_type == KV_BF16)
        return by_group<KV_BF16, KV_BF16, MODE_PLAIN>(p, group, stream);
    if (mode == MODE_PLAIN && kv_type == KV_F16)
        return by_group<KV_F16, KV_F16, MODE_PLAIN>(p, group, stream);
    if (mode == MODE_TIERED && kv_type == KV_F16)
        return by_group<KV_F16, KV_F16, MODE_TIERED>(p, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace atlas
