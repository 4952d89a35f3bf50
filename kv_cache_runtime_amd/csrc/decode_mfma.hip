// Paged decode attention with QK^T on the matrix cores (gfx950), for 16-bit
// and tiered (f16 hot + int8 / int4 cold) pages, head_dim 128 and 2 or 4 query
// heads per kv head.  Same method and split-K structure as decode.hip: keys
// folded tile by tile with an online softmax (CFR-Atlas README, overview;
// ARGUS "Latency & Throughput Impact"), splits merged by log-sum-exp.
//
// gfx950 mapping.  A workgroup is 4 wave64s and owns one (row, kv head,
// split); each wave walks 64-token tiles.  Scores come from
// v_mfma_f32_16x16x32 with the query heads as A (rows, zero-padded to 16)
// and the K rows of 16 tokens as B: lane l supplies 8 dims of token l % 16,
// so every K load is 16 tokens x 64 contiguous bytes, and the result of 16
// tokens x (up to) 16 heads lands with token l % 16 in lane l and heads
// 4 (l / 16) .. + 3 in its four registers.  Four token groups per tile keep
// four independent accumulators in flight.  The softmax keeps one reference
// max per head (moved only when a tile's max exceeds it by 2^8) and reduces
// within 16-lane rows only; probabilities go through LDS, and P.V runs on the
// vector ALUs in the row-slot layout of decode.hip: 16-lane row-slots, each
// lane owning 8 of the 128 dims of 16 consecutive tokens.
//
// Tiered pages: K int8 / int4 codes become f16 in registers (exact), the K
// scale multiplies the finished score and the V scale the probability.  The
// matrix-core operand type is bf16 for bf16 pages (query used as stored) and
// f16 otherwise (the query converted to f16: exact for |q| in [2^-14, 65504],
// smaller magnitudes round with absolute error at most 2^-25).
#include "device.h"

namespace atlas {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kTileTok = 64;  // tokens per wave tile (one per lane for QK)
constexpr int kSlotTok = 16;  // tokens per row-slot for P.V
constexpr int kStagedPages = 512;  // page-table entries staged in LDS per split

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

// int8 codes (4 per word) -> f16 pairs, exact: bias to unsigned, place each
// byte under the f16 exponent of 1024 (0x64xx == 1024 + byte), subtract 1152.
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t u = w ^ 0x80808080u;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t a = __builtin_amdgcn_perm(0u, u, 0x0C010C00u) | 0x64006400u;  // bytes 0, 1
    const uint32_t b = __builtin_amdgcn_perm(0u, u, 0x0C030C02u) | 0x64006400u;  // bytes 2, 3
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - bias);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - bias);
}

// int4 codes (8 per word, element e in nibble e) -> f16 pairs (e, e + 1), exact.
__device__ __forceinline__ void i4x8_to_f16x8(uint32_t w, uint32_t (&out)[4]) {
    const uint32_t u = w ^ 0x88888888u;  // two's complement nibble -> biased by 8
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t byte = (u >> (8 * i)) & 0xFFu;
        const uint32_t pair = (byte & 0x0Fu) | ((byte & 0xF0u) << 12) | 0x64006400u;
        out[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, pair) - bias);
    }
}

// Loads dims d0 .. d0 + 7 of K row `row` of a page as one 16-bit operand
// (uint4) and returns the page's K scale.  Returns false for an invalid
// page-table entry.
template <int KV, int MODE>
__device__ __forceinline__ bool load_k_chunk(const DecodeParams &p, uint32_t entry, int g, int row,
                                             int d0, uint4 &kv, float &kscale) {
    kscale = 1.0f;
    uint32_t tier = 0, slot = entry;
    if constexpr (MODE == MODE_TIERED) {
        tier = entry >> 30;
        slot = entry & ((1u << 30) - 1u);
    }
    const int P = p.page_tokens;
    if (tier == 0) {
        if (slot >= (uint32_t)p.num_blocks) return false;
        kv = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.k_pool) +
                                              (((int64_t)slot * p.num_kv_heads + g) * P + row) * kD +
                                              d0);
        return true;
    }
    if constexpr (MODE == MODE_TIERED) {
        if (tier == 1) {
            if (slot >= (uint32_t)p.n_i8) return false;
            const int64_t r0 = ((int64_t)slot * p.num_kv_heads + g) * P + row;
            const uint2 w = *reinterpret_cast<const uint2 *>(p.i8_k + r0 * kD + d0);
            kscale = p.i8_ks[(int64_t)slot * p.num_kv_heads + g];
            i8x4_to_f16x4(w.x, kv.x, kv.y);
            i8x4_to_f16x4(w.y, kv.z, kv.w);
            return true;
        }
        if (tier == 2) {
            if (slot >= (uint32_t)p.n_i4) return false;
            const int64_t r0 = ((int64_t)slot * p.num_kv_heads + g) * P + row;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(p.i4_k + r0 * (kD / 2) + d0 / 2);
            kscale = p.i4_ks[(int64_t)slot * p.num_kv_heads + g];
            uint32_t o[4];
            i4x8_to_f16x8(w, o);
            kv = make_uint4(o[0], o[1], o[2], o[3]);
            return true;
        }
    }
    return false;
}

// Tiered pages: loads dims 32 r .. 32 r + 31 of K row `row` of a page as the
// four 16-bit operands kv[ks] = dims 32 r + 8 ks .. + 8 (hot: 64 bytes, int8:
// 32, int4: 16, each one contiguous run) and returns the page's K scale.
// Returns false for an invalid page-table entry.
template <int KV>
__device__ __forceinline__ bool load_k_row_tiered(const DecodeParams &p, uint32_t entry, int g,
                                                  int row, int r, uint4 (&kv)[4], float &kscale) {
    kscale = 1.0f;
    const uint32_t tier = entry >> 30, slot = entry & ((1u << 30) - 1u);
    const int P = p.page_tokens;
    const int64_t r0 = ((int64_t)slot * p.num_kv_heads + g) * P + row;
    if (tier == 0) {
        if (slot >= (uint32_t)p.num_blocks) return false;
        const uint4 *src = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.k_pool) + r0 * kD + 32 * r);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kv[ks] = src[ks];
        return true;
    }
    if (tier == 1) {
        if (slot >= (uint32_t)p.n_i8) return false;
        const uint4 *src = reinterpret_cast<const uint4 *>(p.i8_k + r0 * kD + 32 * r);
        kscale = p.i8_ks[(int64_t)slot * p.num_kv_heads + g];
        const uint4 a = src[0], b = src[1];
        i8x4_to_f16x4(a.x, kv[0].x, kv[0].y);
        i8x4_to_f16x4(a.y, kv[0].z, kv[0].w);
        i8x4_to_f16x4(a.z, kv[1].x, kv[1].y);
        i8x4_to_f16x4(a.w, kv[1].z, kv[1].w);
        i8x4_to_f16x4(b.x, kv[2].x, kv[2].y);
        i8x4_to_f16x4(b.y, kv[2].z, kv[2].w);
        i8x4_to_f16x4(b.z, kv[3].x, kv[3].y);
        i8x4_to_f16x4(b.w, kv[3].z, kv[3].w);
        return true;
    }
    if (tier == 2) {
        if (slot >= (uint32_t)p.n_i4) return false;
        const uint4 w = *reinterpret_cast<const uint4 *>(p.i4_k + r0 * (kD / 2) + 16 * r);
        kscale = p.i4_ks[(int64_t)slot * p.num_kv_heads + g];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint32_t o[4];
            i4x8_to_f16x8(ww[ks], o);
            kv[ks] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        return true;
    }
    return false;
}

// Loads the raw V words of 16 tokens x 8 dims for this lane's row-slot (hot:
// 4 words per token, int8: 2, int4: 1), its tier and V scale.  Returns false
// for an invalid page-table entry.
template <int KV, int MODE>
__device__ __forceinline__ bool load_v_slot(const DecodeParams &p, uint32_t entry, int g, int row0,
                                            int c, uint4 (&vr)[kSlotTok], uint32_t &tier,
                                            float &vscale) {
    vscale = 1.0f;
    tier = 0;
    uint32_t slot = entry;
    if constexpr (MODE == MODE_TIERED) {
        tier = entry >> 30;
        slot = entry & ((1u << 30) - 1u);
    }
    const int P = p.page_tokens;
    if (tier == 0) {
        if (slot >= (uint32_t)p.num_blocks) return false;
        const uint16_t *src = reinterpret_cast<const uint16_t *>(p.v_pool) +
                              (((int64_t)slot * p.num_kv_heads + g) * P + row0) * kD + 8 * c;
#pragma unroll
        for (int u = 0; u < kSlotTok; ++u) vr[u] = *reinterpret_cast<const uint4 *>(src + u * kD);
        return true;
    }
    if constexpr (MODE == MODE_TIERED) {
        if (tier == 1) {
            if (slot >= (uint32_t)p.n_i8) return false;
            const int64_t r0 = ((int64_t)slot * p.num_kv_heads + g) * P + row0;
            const uint2 *src = reinterpret_cast<const uint2 *>(p.i8_v + r0 * kD + 8 * c);
            vscale = p.i8_vs[(int64_t)slot * p.num_kv_heads + g];
#pragma unroll
            for (int u = 0; u < kSlotTok; ++u) {
                const uint2 w = src[u * (kD / 8)];
                vr[u] = make_uint4(w.x, w.y, 0u, 0u);
            }
            return true;
        }
        if (tier == 2) {
            if (slot >= (uint32_t)p.n_i4) return false;
            const int64_t r0 = ((int64_t)slot * p.num_kv_heads + g) * P + row0;
            const uint32_t *src = reinterpret_cast<const uint32_t *>(p.i4_v + r0 * (kD / 2) + 4 * c);
            vscale = p.i4_vs[(int64_t)slot * p.num_kv_heads + g];
#pragma unroll
            for (int u = 0; u < kSlotTok; ++u) vr[u] = make_uint4(src[u * (kD / 8)], 0u, 0u, 0u);
            return true;
        }
    }
    return false;
}

template <int QT, int KV, int G, int MODE>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(const DecodeParams p) {
    constexpr int NR = (G + 3) / 4;  // 16-lane rows holding score heads (4 heads per row)
    constexpr float kSlack = 8.0f;   // lazy rescale threshold (log2 units)
    constexpr float kPScale = 7.0f;  // probabilities kept relative to m_ref - 7
    const float kNegInf = -__builtin_inff();

    __shared__ __attribute__((aligned(16))) float sP[kWaves][kTileTok][G];
    __shared__ float s_acc[kWaves][G][kD];
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
    // splits stage them grouped by tier and walk the pages in that order
    __shared__ int32_t s_pages[kStagedPages];
    __shared__ int16_t s_lp[MODE == MODE_TIERED ? kStagedPages : 1];
    const int32_t *trow = p.page_table + (int64_t)seq * p.max_pages;
    const int P = p.page_tokens;
    const int lp_first = t0 / P;
    const int lp_count = t1 > t0 ? (t1 - 1) / P - lp_first + 1 : 0;
    const bool staged = lp_count <= kStagedPages;
    const bool by_tier = MODE == MODE_TIERED && staged;
    if (by_tier) {
        stage_pages_by_tier(trow + lp_first, lp_count, s_pages, s_lp);
    } else {
        if (staged)
            for (int i = tid; i < lp_count; i += 256) s_pages[i] = trow[lp_first + i];
        __syncthreads();
    }

    // A operand: query head c (zero for c >= G), dims 32 ks + 8 r .. + 8
    uint4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (c < G) {
            // operand ks, lane row r holds dims 32 ks + 8 r (16-bit pages) or
            // 32 r + 8 ks (tiered pages, so each lane's K bytes are one run);
            // a dot product does not depend on how its terms are dealt out
            const int d0 = MODE == MODE_TIERED ? 32 * r + 8 * ks : 32 * ks + 8 * r;
            const int64_t q0 = ((int64_t)row * p.num_heads + g * G + c) * kD + d0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = load_elem(p.q, q0 + 2 * i, p.q_dtype);
                const float x1 = load_elem(p.q, q0 + 2 * i + 1, p.q_dtype);
                if constexpr (QT == KV_BF16) {  // q is bf16: exact
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

    // m_ref / l of the heads 4 r + i held by this lane's row (score layout);
    // acc of all G heads in the row-slot layout
    float m_ref[4], l[4], acc[G][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_ref[i] = kNegInf;
        l[i] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    bool bad = !row_ok;

    // positions walked: tokens t0 .. t1 - 1, or (by tier) every token slot of
    // the split's pages, of which those outside [t0, t1) are masked
    const int n_pos = by_tier ? lp_count * P : t1 - t0;
    const int n_tiles = n_pos > 0 ? (n_pos + kTileTok - 1) / kTileTok : 0;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    for (int tile = wave_u; tile < n_tiles; tile += kWaves) {
        // ---- the 16-position groups of the tile: the page size is a
        // multiple of 16 and tiles start at multiples of 64 positions, so a
        // group lies in one page; its first token, page-table entry and
        // liveness are wave-uniform
        int gtok[4];
        uint32_t gent[4];
        bool glive[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            const int q = tile * kTileTok + 16 * tg;
            if (by_tier) {
                const int pi = q / P;
                glive[tg] = pi < lp_count;
                const int lp = lp_first + (glive[tg] ? s_lp[pi] : 0);
                gtok[tg] = lp * P + (q - pi * P);
                gent[tg] = glive[tg] ? (uint32_t)s_pages[pi] : 0u;
            } else {
                gtok[tg] = t0 + q;
                glive[tg] = gtok[tg] < t1;
                const int lp = gtok[tg] / P;
                gent[tg] = glive[tg] ? (uint32_t)(staged ? s_pages[lp - lp_first] : trow[lp]) : 0u;
            }
            gtok[tg] = __builtin_amdgcn_readfirstlane(gtok[tg]);
            gent[tg] = __builtin_amdgcn_readfirstlane(gent[tg]);
        }
        auto in_range = [&](int tok) { return tok >= t0 && tok < t1; };

        // ---- K: token gtok[tg] + c, dims 32 ks + 8 r .. + 8
        uint4 kb[4][4];
        float kscale[4];
        bool kvalid[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            const int tk = gtok[tg] + c;
            kscale[tg] = 1.0f;
            kvalid[tg] = glive[tg] && in_range(tk);
            bool ok = glive[tg];
            if (ok) {
                const int row0 = gtok[tg] % P;
                if constexpr (MODE == MODE_TIERED) {
                    ok = load_k_row_tiered<KV>(p, gent[tg], g, row0 + c, r, kb[tg], kscale[tg]);
                } else {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        ok = ok && load_k_chunk<KV, MODE>(p, gent[tg], g, row0 + c,
                                                          32 * ks + 8 * r, kb[tg][ks], kscale[tg]);
                }
                if (!ok) {
                    bad = true;
                    kvalid[tg] = false;
                }
            }
            if (!ok) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kb[tg][ks] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        // ---- V rows of this lane's row-slot r = group r (in flight during QK)
        const int v0 = r == 0 ? gtok[0] : r == 1 ? gtok[1] : r == 2 ? gtok[2] : gtok[3];
        const uint32_t vent = r == 0 ? gent[0] : r == 1 ? gent[1] : r == 2 ? gent[2] : gent[3];
        bool slot_live = r == 0 ? glive[0] : r == 1 ? glive[1] : r == 2 ? glive[2] : glive[3];
        uint4 vr[kSlotTok];
        uint32_t vtier = 0;
        float vscale = 1.0f;
        if (slot_live) {
            if (!load_v_slot<KV, MODE>(p, vent, g, v0 % P, c, vr, vtier, vscale)) {
                bad = true;
                slot_live = false;
            }
        }

        // ---- scores: sc[tg][i] = head 4 r + i, token 16 tg + c (log2 domain)
        f32x4_t sc[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            sc[tg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sc[tg] = mfma16<QT>(qf[ks], kb[tg][ks], sc[tg]);
            const float f = kscale[tg] * p.scale_log2;
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[tg][i] = kvalid[tg] ? sc[tg][i] * f : kNegInf;
        }

        // ---- online softmax, one reference max per head (uniform in a row)
        bool move_any = false;
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
            mx = fmaxf(mx, dpp_f<0x128>(mx));
            mx = fmaxf(mx, dpp_f<0x124>(mx));
            mx = fmaxf(mx, dpp_f<0x122>(mx));
            mx = fmaxf(mx, dpp_f<0x121>(mx));
            const bool move = mx > m_ref[i] + kSlack;  // also true on the first tile
            const float m_new = move ? mx : m_ref[i];
            alpha[i] = move ? __builtin_amdgcn_exp2f(m_ref[i] - m_new) : 1.0f;
            move_any = move_any || move;
            m_ref[i] = m_new;
        }
        if (__any(move_any)) {  // wave-uniform
#pragma unroll
            for (int i = 0; i < 4; ++i) l[i] *= alpha[i];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ah = __int_as_float(
                    __builtin_amdgcn_readlane(__float_as_int(alpha[h & 3]), 16 * (h >> 2)));
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * r + i;
            const float m_off = (m_ref[i] == kNegInf) ? 0.0f : m_ref[i] - kPScale;
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                const float pr = __builtin_amdgcn_exp2f(sc[tg][i] - m_off);
                l[i] += pr;
                if (r < NR && h < G) sP[wave][16 * tg + c][h] = pr;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- P.V on the vector ALUs (row-slot layout); the tier is uniform
        // within a row-slot, so each decode path runs straight-line
        if (slot_live) {
            auto pv = [&](auto widen) {
#pragma unroll
                for (int u = 0; u < kSlotTok; ++u) {
                    const bool valid = in_range(v0 + u);
                    float pu[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) pu[h] = sP[wave][kSlotTok * r + u][h] * vscale;
                    float v[8];
                    widen(vr[u], v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = valid ? v[e] : 0.0f;
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pu[h], x, acc[h][e]);
                    }
                }
            };
            if (MODE != MODE_TIERED || vtier == 0) {
                pv([](const uint4 &w, float (&v)[8]) {
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = widen_word<KV>(ww, e);
                });
            } else if (vtier == 1) {
                pv([](const uint4 &w, float (&v)[8]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] = (float)sext_field(e < 4 ? w.x : w.y, 24 - 8 * (e & 3), 8);
                });
            } else {
                pv([](const uint4 &w, float (&v)[8]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (float)sext_field(w.x, 28 - 4 * e, 4);
                });
            }
        }
        __builtin_amdgcn_wave_barrier();  // sP is rewritten by the next tile
    }

    // ---- merge: all lanes share the reference max of a head, so the
    // row-slot accumulators just add; l is summed over the 16 lanes of the
    // row that holds the head
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = acc[h][e];
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            acc[h][e] = a;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i] = row16_sum(l[i]);
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * c + e] = acc[h][e];
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
                for (int w = 0; w < kWaves; ++w) o = fmaf(fw[w], s_acc[w][h][col], o);
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
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(int kv_type, int head_dim, int group, int mode) {
    // G = 8 needs more registers than two waves per SIMD allow (spills):
    // it stays on the vector-ALU kernel
    if (head_dim != kD || (group != 2 && group != 4)) return false;
    if (mode == MODE_PLAIN) return kv_type == KV_BF16 || kv_type == KV_F16;
    if (mode == MODE_TIERED) return kv_type == KV_F16;
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
