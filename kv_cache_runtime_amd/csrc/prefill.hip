// Chunked causal prefill on the matrix cores (gfx950 MFMA), folded over the
// paged keys with an online softmax.
//
// Method: "attend the whole chunk as GEMMs with a causal masked softmax"
// (cortiq README, prefill), computed flash-style: the score tile and the
// probability tile never leave registers, and the softmax is folded key tile
// by key tile (CFR-Atlas README, overview: exact folded online-softmax
// attention).  Regenerated pages are produced once per call by the page
// regenerator into the workspace (inspect.hip) and read here like resident
// pages, so each regenerated value is computed once, not once per query tile.
//
// gfx950 mapping.  A workgroup is 4 wave64s and owns 128 query rows of one kv
// head: (128 / G) positions x the G query heads sharing that kv head, so every
// K/V byte staged in LDS feeds all G heads.  Each wave owns 32 rows and
// computes, per 64-key tile,
//   S^T[key][row]  = K[key][:] . Q[row][:]          (v_mfma_f32_32x32x16_bf16,
//                                                    A = K from LDS, B = Q^T in VGPRs)
//   O^T[d][row]   += V^T[d][key] . P^T[key][row]    (A = V^T from LDS, B = P^T in VGPRs)
// P and V enter the second product as f16 (P scaled by 2^15, bf16 V converted
// exactly while it is staged): f16 keeps 11 significant bits of every
// probability where bf16 would keep 8, which holds the result within 2e-3 of
// exact even for rows that see only a few keys.  bf16 V must therefore lie
// within the f16 range (|v| <= 65504); larger values turn the row into inf/NaN.
// Computing the transposed products keeps every row in one lane pair (lane r
// and lane r+32), so the row max, the rescale of the accumulator and the
// conversion of P to the B operand need no data movement beyond one
// cross-half exchange.  K is staged row-major; V is transposed while it is
// written to LDS (4 keys per 64-bit store) so that its MFMA operand is read
// with two 64-bit loads per lane.  The key order inside a 16-key MFMA step
// is permuted identically in A and B, which leaves the contraction unchanged.
// Workgroups are ordered kv-head-fastest so that, with 8 kv heads on 8 XCDs,
// each XCD's L2 serves the K/V stream of one kv head.
#include "device.h"

namespace atlas {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;              // head_dim
constexpr int kTile = 64;            // keys per tile
constexpr int kKStride = kD + 8;     // LDS row stride of K, 16-bit elements (272 B)
constexpr int kVStride = kTile + 4;  // LDS row stride of V^T, 16-bit elements (136 B)

template <int KV>
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    if constexpr (KV == KV_BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// Two packed bf16 values -> two packed f16 values (exact for magnitudes in
// the f16 normal range; values above 65504 become inf and poison the row).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const f16x2_t h = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, h);
}

// Row index (in units of head_dim elements) of K row `key` of (seq, kv head
// g): a regenerated page in the workspace copy, or a resident page through
// the page table.  Rows key .. key + 3 share the page (page_tokens is a
// multiple of 16).  Sets `bad` for a block id outside the pool (rows of block
// 0 are read instead).
__device__ __forceinline__ int64_t k_row_index(const PrefillParams &p, int seq, int g, int key,
                                               uint32_t lp, int n_regen, bool &bad) {
    const int P = p.page_tokens;
    const int row = key - (int)lp * P;
    if ((int)lp < n_regen) return (((int64_t)seq * p.max_regen + lp) * p.num_kv_heads + g) * P + row;
    int blk = p.page_table[(int64_t)seq * p.max_pages + lp];
    if (blk < 0 || blk >= p.num_blocks) {
        bad = true;
        blk = 0;
    }
    return ((int64_t)blk * p.num_kv_heads + g) * P + row;
}

__device__ __forceinline__ uint32_t page_of(const PrefillParams &p, int key) {
    return (__umulhi((uint32_t)key, p.p_magic) + (uint32_t)key) >> p.p_shift;
}

// ALIBI: scores gain -slope_h * (pos - key).  ROPE: q is rotated by its
// position; the rotated row is kept as a 16-bit hi part plus the rounded
// remainder, and S^T takes one more MFMA per step for the remainder.
template <int KV, int G, int NH, bool ALIBI, bool ROPE>
__global__ __launch_bounds__(256, 3 - NH) void prefill_kernel(const PrefillParams p) {
    constexpr int kPosHalf = 32 / G;         // positions per 32-row half
    constexpr int kPosWave = NH * kPosHalf;  // a wave owns NH halves of 32 rows
    constexpr int kPosWg = 4 * kPosWave;     // positions per workgroup
    // Lazy rescale: the reference max of a row moves only when a tile's max
    // exceeds it by more than 2^8, so probabilities (scaled by 2^7) stay
    // below 2^15 and fit f16.
    constexpr float kSlack = 8.0f;
    constexpr float kPScale = 7.0f;
    const float kNegInf = -__builtin_inff();

    // double-buffered K (row-major) and V^T tiles
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kTile * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][kD * kVStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, half = lane >> 5;

    const int g = blockIdx.x % p.num_kv_heads;
    const int rest = blockIdx.x / p.num_kv_heads;
    const int qb = rest % p.q_blocks;
    const int seq = rest / p.q_blocks;

    const int q0 = p.rows.query_start[seq];
    const int n_q = p.rows.query_start[seq + 1] - q0;
    if (n_q < 1 || n_q > p.max_query_len) return;  // malformed chunk: nothing addressable
    const int t_base = qb * kPosWg;
    if (t_base >= n_q) return;
    const int ctx = p.rows.context_lens[seq];
    const bool ctx_ok = ctx >= n_q && ctx <= p.rows.max_context_len && ctx <= p.rows.max_keys &&
                        q0 >= 0 && q0 + n_q <= p.total_q;

    // this lane's two query rows (one per 32-row half)
    const int head = g * G + (r % G);
    int t[NH], pos[NH];
    bool row_ok[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        t[hh] = t_base + wave * kPosWave + hh * kPosHalf + r / G;
        row_ok[hh] = ctx_ok && t[hh] < n_q;
        pos[hh] = ctx - n_q + t[hh];  // last visible key of the row
    }
    const int t_last = min(n_q - 1, t_base + kPosWg - 1);
    const int key_limit = ctx_ok ? ctx - n_q + t_last + 1 : 0;
    const int wave_min_pos = ctx - n_q + t_base + wave * kPosWave;
    bool all_ok = true;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) all_ok = all_ok && row_ok[hh];
    const bool wave_rows_ok = __all(all_ok);
    int n_regen = 0;
    bool regen_bad = false;
    if (p.regen_pages != nullptr && ctx_ok) {
        n_regen = p.regen_pages[seq];
        if (n_regen < 0 || n_regen > p.max_regen) {  // outside the host bound: fail loudly
            regen_bad = true;
            n_regen = 0;
        }
    }

    // Q^T operands: k-step ks holds dims 16 ks + 8 half .. + 8 of the row
    uint4 qf[NH][8];
    uint4 qlo[NH][ROPE ? 8 : 1];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                               ((int64_t)(q0 + t[hh]) * p.num_heads + head) * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[hh][ks] = row_ok[hh] ? *reinterpret_cast<const uint4 *>(qrow + 16 * ks)
                                    : make_uint4(0, 0, 0, 0);
            if constexpr (ROPE) {
                uint32_t hi[4] = {qf[hh][ks].x, qf[hh][ks].y, qf[hh][ks].z, qf[hh][ks].w};
                uint32_t lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x0 = KV == KV_BF16 ? bf16_lo(hi[i]) : f16_lo(hi[i]);
                    float x1 = KV == KV_BF16 ? bf16_hi(hi[i]) : f16_hi(hi[i]);
                    rope_rotate(x0, x1, pos[hh],
                                rope_turns(8 * ks + 4 * half + i, kD, p.pos.rope_log2_theta));
                    if constexpr (KV == KV_BF16) {
                        const float h0 = bf16_round(x0), h1 = bf16_round(x1);
                        hi[i] = (__float_as_uint(h0) >> 16) | (__float_as_uint(h1) & 0xFFFF0000u);
                        lo[i] = (__float_as_uint(bf16_round(x0 - h0)) >> 16) |
                                (__float_as_uint(bf16_round(x1 - h1)) & 0xFFFF0000u);
                    } else {
                        const f16x2_t h = {(_Float16)x0, (_Float16)x1};
                        const f16x2_t l = {(_Float16)(x0 - (float)h[0]), (_Float16)(x1 - (float)h[1])};
                        hi[i] = __builtin_bit_cast(uint32_t, h);
                        lo[i] = __builtin_bit_cast(uint32_t, l);
                    }
                }
                qf[hh][ks] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                qlo[hh][ks] = row_ok[hh] ? make_uint4(lo[0], lo[1], lo[2], lo[3])
                                         : make_uint4(0, 0, 0, 0);
            }
        }
    }
    // ALiBi slope of this lane's head in raw score units (the scores are
    // scaled by scale * log2(e) later)
    float ab = 0.0f;
    if constexpr (ALIBI) ab = p.pos.alibi[head] / (p.scale_log2 * (1.0f / kLog2e));

    f32x16_t o[NH][4];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[hh][b][j] = 0.0f;
    float m_ref[NH], l[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        m_ref[hh] = kNegInf;
        l[hh] = 0.0f;
    }
    bool bad = false;

    // cooperative staging.  K: thread (kg, dc) moves keys 4 kg .. 4 kg + 3,
    // dims 8 dc .. 8 dc + 7 (one page lookup per thread and tile).  V^T:
    // thread moves keys 8 vk .. 8 vk + 7 of dims vd + 32 i from the
    // transposed copy.
    const int dc = tid & 15, kg = tid >> 4;
    const int vk = tid & 7, vd = tid >> 3;
    const int64_t vt_seq = (int64_t)seq * p.max_pages;
    uint4 kreg[4], vreg[4];
    // Pages of a multiple of 64 tokens hold whole tiles: a full tile then
    // has one (wave-uniform) page, so its K and V^T bases are scalar and every
    // thread adds a fixed offset.
    const bool whole_tiles = p.page_tokens % kTile == 0;
    const int k_off = 4 * kg * kD + 8 * dc;                  // elements from a K row base
    const int v_off = 8 * vk + vd * p.page_tokens;           // elements from a V^T page base
    const int64_t v_step = (int64_t)32 * p.page_tokens;      // dims vd + 32 i
    auto fetch_whole = [&](int k0) {
        const int P = p.page_tokens;
        const int lp = k0 / P;
        const int r0 = k0 - lp * P;
        const uint16_t *kb;
        if (lp < n_regen) {
            kb = reinterpret_cast<const uint16_t *>(p.regen_k) +
                 ((((int64_t)seq * p.max_regen + lp) * p.num_kv_heads + g) * P + r0) * kD;
        } else {
            int blk = p.page_table[(int64_t)seq * p.max_pages + lp];
            if (blk < 0 || blk >= p.num_blocks) {
                bad = true;
                blk = 0;
            }
            kb = reinterpret_cast<const uint16_t *>(p.k_pool) +
                 (((int64_t)blk * p.num_kv_heads + g) * P + r0) * kD;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) kreg[i] = *reinterpret_cast<const uint4 *>(kb + k_off + i * kD);
        const uint16_t *vb = reinterpret_cast<const uint16_t *>(p.vt) +
                             ((vt_seq + lp) * p.num_kv_heads + g) * (int64_t)kD * P + r0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vreg[i] = *reinterpret_cast<const uint4 *>(vb + v_off + i * v_step);
    };
    auto fetch = [&](int k0) {
        if (whole_tiles && k0 + kTile <= key_limit) {  // uniform
            fetch_whole(k0);
            return;
        }
        const int key = k0 + 4 * kg;
        if (key < key_limit) {
            const int64_t row = k_row_index(p, seq, g, key, page_of(p, key), n_regen, bad);
            const uint16_t *kb =
                reinterpret_cast<const uint16_t *>((int)page_of(p, key) < n_regen ? p.regen_k
                                                                                   : p.k_pool) +
                row * kD + 8 * dc;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kreg[i] = key + i < key_limit ? *reinterpret_cast<const uint4 *>(kb + i * kD)
                                              : make_uint4(0, 0, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kreg[i] = make_uint4(0, 0, 0, 0);
        }
        const int vkey = k0 + 8 * vk;
        if (vkey < key_limit) {
            const uint32_t lp = page_of(p, vkey);
            const uint16_t *vb = reinterpret_cast<const uint16_t *>(p.vt) +
                                 ((vt_seq + lp) * p.num_kv_heads + g) * (int64_t)kD * p.page_tokens +
                                 (vkey - (int)lp * p.page_tokens) + (int64_t)vd * p.page_tokens;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vreg[i] = *reinterpret_cast<const uint4 *>(vb + (int64_t)(32 * i) * p.page_tokens);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) vreg[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4 *>(&sK[buf][(4 * kg + i) * kKStride + 8 * dc]) = kreg[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t *dst = &sV[buf][(vd + 32 * i) * kVStride + 8 * vk];
            *reinterpret_cast<uint2 *>(dst) = make_uint2(vreg[i].x, vreg[i].y);
            *reinterpret_cast<uint2 *>(dst + 4) = make_uint2(vreg[i].z, vreg[i].w);
        }
    };

    const int n_tiles = (key_limit + kTile - 1) / kTile;
    if (n_tiles > 0) {
        fetch(0);
        stage(0);
    }
    __syncthreads();
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int k0 = tile * kTile;
        const int buf = tile & 1;
        if (tile + 1 < n_tiles) fetch(k0 + kTile);  // in flight during the math below
        const uint16_t *cK = sK[buf];
        const uint16_t *cV = sV[buf];

        // S^T for keys k0 .. k0 + 63 (two 32-key blocks) and both halves;
        // each K fragment read from LDS feeds two MFMAs
        f32x16_t s[NH][2];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) s[hh][kb][j] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint4 a =
                    *reinterpret_cast<const uint4 *>(&cK[(32 * kb + r) * kKStride + 16 * ks + 8 * half]);
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    s[hh][kb] = mfma32<KV>(a, qf[hh][ks], s[hh][kb]);
                    if constexpr (ROPE) s[hh][kb] = mfma32<KV>(a, qlo[hh][ks], s[hh][kb]);
                }
            }
        }
        // ALiBi, split as ab * (key - pos) = ab * o_j + rb: o_j = key - (k0 +
        // 4 half) is a compile-time offset of the register slot, and the
        // row's tile offset rb = ab * (k0 + 4 half - pos) is added to its max
        // and to the exponent below, once per row instead of per score
        float rb[NH];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) rb[hh] = 0.0f;
        if constexpr (ALIBI) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                rb[hh] = ab * (float)(k0 + 4 * half - pos[hh]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        s[hh][kb][j] = fmaf(ab, (float)(32 * kb + 8 * (j >> 2) + (j & 3)),
                                            s[hh][kb][j]);
            }
        }

        // causal mask only on tiles that reach past some row's position
        if (!wave_rows_ok || k0 + kTile - 1 > wave_min_pos) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = k0 + 32 * kb + 8 * (j >> 2) + 4 * half + (j & 3);
                        s[hh][kb][j] = (row_ok[hh] && key <= pos[hh]) ? s[hh][kb][j] : kNegInf;
                    }
        }
        float mt[NH];
        bool move[NH];
        bool any_move = false;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            float mraw = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mraw = fmaxf(mraw, s[hh][kb][j]);
            if constexpr (ALIBI) mraw += rb[hh];
            {  // the row's other half (lane r + 32) by a VALU swap, no LDS trip
                const auto h = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(mraw), __float_as_uint(mraw), false, false);
                mraw = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
            }
            mt[hh] = mraw * p.scale_log2;  // scale > 0 keeps the order
            move[hh] = mt[hh] > m_ref[hh] + kSlack;  // also true on the first finite tile
            any_move = any_move || move[hh];
        }
        if (__any(any_move)) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) {
                const float m_new = move[hh] ? mt[hh] : m_ref[hh];
                const float alpha = move[hh] ? __builtin_amdgcn_exp2f(m_ref[hh] - m_new) : 1.0f;
                m_ref[hh] = m_new;
                l[hh] *= alpha;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[hh][b][j] *= alpha;
            }
        }

        // P^T operands (f16, p * 2^7 relative to the reference max): PV step
        // st covers keys 16 st .. 16 st + 15 of the tile
        uint4 pb[NH][4];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            float m_off = (m_ref[hh] == kNegInf) ? 0.0f : m_ref[hh] - kPScale;
            if constexpr (ALIBI) m_off = fmaf(-rb[hh], p.scale_log2, m_off);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int kb = st >> 1, j0 = 8 * (st & 1);
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 =
                        __builtin_amdgcn_exp2f(fmaf(s[hh][kb][j0 + 2 * i], p.scale_log2, -m_off));
                    const float p1 =
                        __builtin_amdgcn_exp2f(fmaf(s[hh][kb][j0 + 2 * i + 1], p.scale_log2, -m_off));
                    const f16x2_t h = {(_Float16)p0, (_Float16)p1};
                    // l sums the f16 weights the matrix cores use
                    l[hh] = __builtin_amdgcn_fdot2(h, f16x2_t{(_Float16)1.0f, (_Float16)1.0f},
                                                   l[hh], false);
                    w[i] = __builtin_bit_cast(uint32_t, h);
                }
                pb[hh][st] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }

        // O^T += V^T P^T; each V^T fragment read from LDS feeds two MFMAs
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint16_t *vrow = &cV[(32 * b + r) * kVStride + 4 * half + 16 * st];
                const uint2 va = *reinterpret_cast<const uint2 *>(vrow);
                const uint2 vb = *reinterpret_cast<const uint2 *>(vrow + 8);
                const uint4 a = make_uint4(va.x, va.y, vb.x, vb.y);
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) o[hh][b] = mfma32<KV_F16>(a, pb[hh][st], o[hh][b]);
            }
        }

        if (tile + 1 < n_tiles) stage(buf ^ 1);
        __syncthreads();
    }

    // combine the two halves of each row and write out / lse
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || !ctx_ok || regen_bad;
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        const float l_row = l[hh] + __shfl_xor(l[hh], 32);
        if (t[hh] < n_q) {
            const int64_t orow = (int64_t)(q0 + t[hh]) * p.num_heads + head;
            const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
            float *dst = p.out + orow * kD;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d0 = 32 * b + 8 * jj + 4 * half;
                    float4 v = make_float4(o[hh][b][4 * jj] * inv, o[hh][b][4 * jj + 1] * inv,
                                           o[hh][b][4 * jj + 2] * inv, o[hh][b][4 * jj + 3] * inv);
                    if (any_bad) v = make_float4(qnan, qnan, qnan, qnan);
                    *reinterpret_cast<float4 *>(dst + d0) = v;
                }
            }
            if (half == 0) {
                const float m_off = (m_ref[hh] == kNegInf) ? 0.0f : m_ref[hh] - kPScale;
                const float lse = l_row > 0.0f ? (m_off + log2f(l_row)) * kLn2 : kNegInf;
                p.lse[orow] = any_bad ? qnan : lse;
            }
        }
    }
}

template <int KV, int NH, bool A, bool R>
hipError_t by_group(const PrefillParams &p, int group, hipStream_t s) {
    const int64_t blocks = (int64_t)p.num_kv_heads * p.q_blocks * p.rows.num_seqs;
    if (blocks <= 0) return hipSuccess;
    switch (group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<KV, 1, NH, A, R>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<KV, 2, NH, A, R>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<KV, 4, NH, A, R>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<KV, 8, NH, A, R>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int KV>
hipError_t by_policy(const PrefillParams &p, int group, hipStream_t s) {
    const bool a = p.pos.alibi != nullptr, r = p.pos.rope != 0;
    if (a && r) return by_group<KV, kPrefillHalves, true, true>(p, group, s);
    if (a) return by_group<KV, kPrefillHalves, true, false>(p, group, s);
    if (r) return by_group<KV, kPrefillHalves, false, true>(p, group, s);
    return by_group<KV, kPrefillHalves, false, false>(p, group, s);
}

}  // namespace

int prefill_rows_per_wave() { return 32 * kPrefillHalves; }

hipError_t launch_prefill(const PrefillParams &p, int kv_type, int group, hipStream_t stream) {
    if (kv_type == KV_BF16) return by_policy<KV_BF16>(p, group, stream);
    if (kv_type == KV_F16) return by_policy<KV_F16>(p, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace atlas
