// Chunked causal prefill on the matrix cores (gfx950 MFMA), folded over the
// paged keys with an online softmax.
//
// Method.  A chunk of new query rows attends its whole context as two dense
// products around a causally masked softmax (cortiq README, "Attention that
// stops growing with the context"), computed flash-style: scores and
// probabilities stay in registers and the keys are folded tile by tile into a
// running max, sum and accumulator (CFR-Atlas README, overview: exact folded
// online-softmax attention).  A call may cover one window [key_begin,
// key_end) of the keys; a later window merges its partial result into out/lse
// by log-sum-exp (attnres AGENTS.md, online softmax merge), so that
// regenerated pages can be produced window by window into a bounded ring.
//
// gfx950 mapping.  A workgroup is 8 wave64s and owns 256 query rows of one kv
// head: (256 / G) positions x the G query heads sharing that kv head, so
// every K/V byte staged in LDS feeds all G heads and all 8 waves.  Wave w owns
// 32 rows and computes, per 64-key tile,
//   S^T[key][row]  = K[key][:] . Q[row][:]        (v_mfma_f32_32x32x16_{bf16,f16};
//                                                  A = K from LDS, B = Q^T in VGPRs)
//   O^T[d][row]   += V^T[d][key] . P^T[key][row]  (v_mfma_f32_32x32x16_f16;
//                                                  A = V from LDS by the transposing
//                                                  read, B = P^T in VGPRs)
// so each row lives in one lane pair (r, r + 32) for the softmax.
//
// Phases.  The waves of a workgroup are dealt to the four SIMDs round-robin,
// so waves w and w + 4 share a SIMD.  Waves 0-3 and waves 4-7 run the same
// sequence of clusters -- matrix cluster M_a (P.V of tile a - 1 and the scores
// of tile a), vector cluster V_a (the softmax of tile a and the staging of the
// next tiles) -- but waves 4-7 run one slot behind.  Every slot ends with a
// workgroup barrier, so on each SIMD one wave issues matrix instructions while
// the other runs the exponentials, and the matrix cores do not wait for the
// softmax.
//
// Staging.  LDS holds two buffers, each a 64-key K tile (row-major) and a
// 64-key V tile (row-major, f16: bf16 values are converted while staged, so
// P.V runs with f16 probabilities).  Buffer x % 2 holds K of tile x and V of
// tile x - 1, read by M_x; each wave group stages its 32 keys of the next
// buffer in its vector clusters, from registers loaded one cluster earlier.
// P is kept relative to the reference max minus 7 and is at most 2^15, so
// P * V stays finite for |v| <= 65504, the f16 range that bf16 V must lie in.
#include "device.h"

namespace atlas {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head_dim
constexpr int kTile = 64;        // keys per tile
constexpr int kWaves = 8;        // waves per workgroup
constexpr int kKPitch = 136;     // K tile row pitch, 16-bit elements (68 dwords)
constexpr int kVPitch = 160;     // V tile row pitch, 16-bit elements (80 dwords)

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

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// s gives the address of 4 consecutive 16-bit elements; with lane s pointing
// at row k0 + s / 4, column n0 + 4 (s % 4) of a row-major tile, lane i
// receives column n0 + i of rows k0 .. k0 + 3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *ptr) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(ptr));
    return __builtin_bit_cast(uint2, v);
}

// Two packed bf16 values -> two packed f16 values (round to nearest even;
// exact for magnitudes in the f16 normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const f16x2_t h = {(_Float16)__uint_as_float(w << 16),
                       (_Float16)__uint_as_float(w & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, h);
}

// Barrier between slots: LDS traffic settled, global loads left in flight.
__device__ __forceinline__ void slot_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ALIBI: scores gain -slope_h * (pos - key).  ROPE: q is rotated by its
// position; the rotated row is kept as a 16-bit hi part plus the rounded
// remainder, and S^T takes one more MFMA per step for the remainder.
template <int KV, int G, bool ALIBI, bool ROPE>
__global__ __launch_bounds__(512, 1) void prefill_kernel(const PrefillParams p) {
    constexpr int kPosWave = 32 / G;         // positions per wave
    constexpr int kPosWg = kWaves * kPosWave;
    // Lazy rescale: the reference max of a row moves only when a tile's max
    // exceeds it by more than 2^8, so probabilities (scaled by 2^7) stay
    // at most 2^15 and fit f16.
    constexpr float kSlack = 8.0f;
    constexpr float kPScale = 7.0f;
    const float kNegInf = -__builtin_inff();

    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kTile * kKPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][kTile * kVPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (scalar) so that the cluster branches below are uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;   // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
    const int r = lane & 31, half = lane >> 5;

    const int g = blockIdx.x % p.num_kv_heads;
    const int rest = blockIdx.x / p.num_kv_heads;
    const int qb = rest % p.q_blocks;
    const int seq = rest / p.q_blocks;

    const int q0 = p.rows.query_start[seq];
    const int n_q = p.rows.query_start[seq + 1] - q0;
    // a chunk whose rows cannot be addressed is left alone (the validator
    // counts it)
    if (n_q < 1 || n_q > p.max_query_len || q0 < 0 || q0 + n_q > p.total_q) return;
    const int t_base = qb * kPosWg;
    if (t_base >= n_q) return;
    const int ctx = p.rows.context_lens[seq];
    const bool ctx_ok = ctx >= n_q && ctx <= p.rows.max_context_len && ctx <= p.rows.max_keys;

    // this lane's query row
    const int head = g * G + (r % G);
    const int t = t_base + wave * kPosWave + r / G;
    const bool row_ok = ctx_ok && t < n_q;
    const int pos = ctx - n_q + t;  // last visible key of the row
    const int t_last = min(n_q - 1, t_base + kPosWg - 1);
    const int key_limit = ctx_ok ? ctx - n_q + t_last + 1 : 0;
    const int wave_min_pos = ctx - n_q + t_base + wave * kPosWave;
    const bool wave_rows_ok = __all(row_ok);

    int n_regen = 0;
    bool regen_bad = false;
    if (p.regen_pages != nullptr && ctx_ok) {
        n_regen = p.regen_pages[seq];
        if (n_regen < 0 || n_regen > p.max_regen) {  // outside the host bound: fail loudly
            regen_bad = true;
            n_regen = 0;
        }
    }

    // keys of this call: the window, cut at the last key any row here sees
    const int kb0 = p.key_begin;
    const int kb1 = min(p.key_end, key_limit);
    const int n_tiles = kb1 > kb0 ? (kb1 - kb0 + kTile - 1) / kTile : 0;
    const int64_t orow0 = (int64_t)(q0 + t) * p.num_heads + head;
    const float qnan = __builtin_nanf("");
    if (n_tiles == 0) {  // uniform: no key of this window is visible here
        if (!p.carry && t < n_q) {  // the first window still owns the rows
            const float o_fill = ctx_ok && !regen_bad ? 0.0f : qnan;
            float *dst = p.out + orow0 * kD;
            for (int d = 4 * half; d < kD; d += 8)
                *reinterpret_cast<float4 *>(dst + d) = make_float4(o_fill, o_fill, o_fill, o_fill);
            if (half == 0) p.lse[orow0] = ctx_ok && !regen_bad ? kNegInf : qnan;
        }
        return;
    }

    // Q^T operands: k-step ks holds dims 16 ks + 8 half .. + 8 of the row
    uint4 qf[8];
    uint4 qlo[ROPE ? 8 : 1];
    {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) + orow0 * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = row_ok ? *reinterpret_cast<const uint4 *>(qrow + 16 * ks)
                            : make_uint4(0, 0, 0, 0);
            if constexpr (ROPE) {
                uint32_t hi[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
                uint32_t lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x0 = KV == KV_BF16 ? bf16_lo(hi[i]) : f16_lo(hi[i]);
                    float x1 = KV == KV_BF16 ? bf16_hi(hi[i]) : f16_hi(hi[i]);
                    rope_rotate(x0, x1, pos, rope_turns(8 * ks + 4 * half + i, kD,
                                                        p.pos.rope_log2_theta));
                    if constexpr (KV == KV_BF16) {
                        const float h0 = bf16_round(x0), h1 = bf16_round(x1);
                        hi[i] = (__float_as_uint(h0) >> 16) | (__float_as_uint(h1) & 0xFFFF0000u);
                        lo[i] = (__float_as_uint(bf16_round(x0 - h0)) >> 16) |
                                (__float_as_uint(bf16_round(x1 - h1)) & 0xFFFF0000u);
                    } else {
                        const f16x2_t h = {(_Float16)x0, (_Float16)x1};
                        const f16x2_t l2 = {(_Float16)(x0 - (float)h[0]),
                                            (_Float16)(x1 - (float)h[1])};
                        hi[i] = __builtin_bit_cast(uint32_t, h);
                        lo[i] = __builtin_bit_cast(uint32_t, l2);
                    }
                }
                qf[ks] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                qlo[ks] = row_ok ? make_uint4(lo[0], lo[1], lo[2], lo[3]) : make_uint4(0, 0, 0, 0);
            }
        }
    }
    // ALiBi slope of this lane's head in raw score units (the scores are
    // scaled by scale * log2(e) later)
    float ab = 0.0f;
    if constexpr (ALIBI) ab = p.pos.alibi[head] / (p.scale_log2 * (1.0f / kLog2e));

    f32x16_t o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[b][j] = 0.0f;
    f32x16_t s[2];
    uint4 pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) pb[st] = make_uint4(0, 0, 0, 0);
    float m_ref = kNegInf, l = 0.0f;
    bool bad = false;

    // ---- staging: this thread moves 16 dims of key 32 grp + tg / 8 of a
    // tile, for K and for V.  K dims 16 cp .. 16 cp + 15; V dims of chunks c0
    // and c0 + 4 (8 dims each), which keeps the 16 lanes of one LDS write
    // phase on distinct banks with the 80-dword V pitch.
    const int tg = tid & 255;
    const int srow = 32 * grp + (tg >> 3);
    const int cp = tg & 7;
    const int vc0 = (cp & 3) + 8 * (cp >> 2);
    const int P = p.page_tokens;
    const int64_t trow = (int64_t)seq * p.max_pages;
    const int64_t ring_row0 = ((int64_t)seq * p.num_kv_heads + g) * p.ring_tokens;
    // Element offset of key `key`'s row of this kv head, in the ring or in the
    // pool through the page table.  `ent` is the page-table entry of the key's
    // page (read ahead by the caller).
    auto row_offset = [&](int key, int ent, const uint16_t *&base) -> int64_t {
        const int lp = (int)((__umulhi((uint32_t)key, p.p_magic) + (uint32_t)key) >> p.p_shift);
        if (lp < n_regen) {
            base = reinterpret_cast<const uint16_t *>(p.ring_k);
            return (ring_row0 + (key - kb0)) * kD;
        }
        int blk = ent;
        if (blk < 0 || blk >= p.num_blocks) {
            bad = true;
            blk = 0;
        }
        base = nullptr;
        return (((int64_t)blk * p.num_kv_heads + g) * P + (key - lp * P)) * kD;
    };
    auto entry_of = [&](int key) -> int {
        const int lp = (int)((__umulhi((uint32_t)key, p.p_magic) + (uint32_t)key) >> p.p_shift);
        return lp >= n_regen ? p.page_table[trow + lp] : 0;
    };
    uint4 kst[2], vst[2];
    int ent_k = 0, ent_v = 0;  // entries of the next content's keys
    // Loads this group's half of content x (K of tile x, V of tile x - 1)
    // into kst / vst; keys past the visible range load zeros.
    auto load_content = [&](int x) {
        const int kk = kb0 + kTile * x + srow;
        const int kv = kk - kTile;
        if (x < n_tiles && kk < kb1) {
            const uint16_t *base;
            int64_t off = row_offset(kk, ent_k, base);
            const uint16_t *src = (base ? base : reinterpret_cast<const uint16_t *>(p.k_pool)) +
                                  off + 16 * cp;
            kst[0] = *reinterpret_cast<const uint4 *>(src);
            kst[1] = *reinterpret_cast<const uint4 *>(src + 8);
        } else {
            kst[0] = kst[1] = make_uint4(0, 0, 0, 0);
        }
        if (x >= 1 && x <= n_tiles && kv < kb1) {
            const uint16_t *base;
            int64_t off = row_offset(kv, ent_v, base);
            const uint16_t *src = (base ? reinterpret_cast<const uint16_t *>(p.ring_v)
                                        : reinterpret_cast<const uint16_t *>(p.v_pool)) +
                                  off + 8 * vc0;
            vst[0] = *reinterpret_cast<const uint4 *>(src);
            vst[1] = *reinterpret_cast<const uint4 *>(src + 32);
        } else {
            vst[0] = vst[1] = make_uint4(0, 0, 0, 0);
        }
        // entries of content x + 1 (the next call), read ahead
        const int nk = kk + kTile, nv = kv + kTile;
        ent_k = (x + 1 < n_tiles && nk < kb1) ? entry_of(nk) : 0;
        ent_v = (x + 1 <= n_tiles && nv < kb1) ? entry_of(nv) : 0;
    };
    auto write_content = [&](int x) {
        const int buf = x & 1;
        uint16_t *kd = &sK[buf][srow * kKPitch + 16 * cp];
        *reinterpret_cast<uint4 *>(kd) = kst[0];
        *reinterpret_cast<uint4 *>(kd + 8) = kst[1];
        uint4 v0 = vst[0], v1 = vst[1];
        if constexpr (KV == KV_BF16) {
            v0 = make_uint4(bf16x2_to_f16x2(v0.x), bf16x2_to_f16x2(v0.y), bf16x2_to_f16x2(v0.z),
                            bf16x2_to_f16x2(v0.w));
            v1 = make_uint4(bf16x2_to_f16x2(v1.x), bf16x2_to_f16x2(v1.y), bf16x2_to_f16x2(v1.z),
                            bf16x2_to_f16x2(v1.w));
        }
        uint16_t *vd = &sV[buf][srow * kVPitch + 8 * vc0];
        *reinterpret_cast<uint4 *>(vd) = v0;
        *reinterpret_cast<uint4 *>(vd + 32) = v1;
    };

    // prologue: content 0 (K of tile 0) from both groups, then the first
    // content each group writes inside the loop (content 1)
    {
        ent_k = kb0 + srow < kb1 ? entry_of(kb0 + srow) : 0;
        load_content(0);
        write_content(0);
        load_content(1);
    }
    slot_barrier();

    // ---- matrix cluster M_a: P.V of tile a - 1, scores of tile a
    auto matrix_cluster = [&](int a) {
        const uint16_t *cK = sK[a & 1];
        const uint16_t *cV = sV[a & 1];
        if (a >= 1) {
            // A = V^T: lane (dim 32 b + r, half) takes keys 16 st + 4 half ..
            // + 3 and 16 st + 8 + 4 half .. + 3 (two transposing reads), the
            // key order of P^T's registers
            const int q16 = lane >> 4, s16 = lane & 15;
            const int kq = 4 * (q16 >> 1) + (s16 >> 2);     // row within the 16-key step
            const int nq = 16 * (q16 & 1) + 4 * (s16 & 3);  // dim within the 32-dim block
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint16_t *vp = cV + (16 * st + kq) * kVPitch + 32 * b + nq;
                    const uint2 x0 = lds_read_tr16(vp);
                    const uint2 x1 = lds_read_tr16(vp + 8 * kVPitch);
                    o[b] = mfma32<KV_F16>(make_uint4(x0.x, x0.y, x1.x, x1.y), pb[st], o[b]);
                }
            }
        }
        if (a < n_tiles) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) s[kb][j] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint4 av = *reinterpret_cast<const uint4 *>(
                        &cK[(32 * kb + r) * kKPitch + 16 * ks + 8 * half]);
                    s[kb] = mfma32<KV>(av, qf[ks], s[kb]);
                    if constexpr (ROPE) s[kb] = mfma32<KV>(av, qlo[ks], s[kb]);
                }
            }
        }
    };
    // ---- vector cluster V_a: staging (group 0 writes content a + 1, group 1
    // content a + 2), then the softmax of tile a (a = -1: staging only)
    auto vector_cluster = [&](int a) {
        const int x = a + 1 + grp;
        if (x <= n_tiles) {
            write_content(x);
            load_content(x + 1);
        }
        if (a < 0) return;
        // S^T register j of block kb holds key k0 + 32 kb + 8 (j / 4) +
        // 4 half + j % 4 of row r
        const int k0 = kb0 + kTile * a;
        float rb = 0.0f;
        if constexpr (ALIBI) {
            // ab * (key - pos) = ab * o_j + rb with o_j a fixed offset of the
            // register slot and rb the row's tile offset
            rb = ab * (float)(k0 + 4 * half - pos);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    s[kb][j] = fmaf(ab, (float)(32 * kb + 8 * (j >> 2) + (j & 3)), s[kb][j]);
        }
        if (!wave_rows_ok || k0 + kTile - 1 > wave_min_pos) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = k0 + 32 * kb + 8 * (j >> 2) + 4 * half + (j & 3);
                    s[kb][j] = (row_ok && key <= pos) ? s[kb][j] : kNegInf;
                }
        }
        float mraw = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mraw = fmaxf(mraw, s[kb][j]);
        if constexpr (ALIBI) mraw += rb;
        {  // the row's other half (lane r + 32)
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw),
                                                            __float_as_uint(mraw), false, false);
            mraw = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
        }
        const float mt = mraw * p.scale_log2;    // scale > 0 keeps the order
        const bool move = mt > m_ref + kSlack;  // also true on the first finite tile
        if (__any(move)) {
            const float m_new = move ? mt : m_ref;
            const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
            m_ref = m_new;
            l *= alpha;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[b][j] *= alpha;
        }
        // P^T operands (f16, relative to m_ref - 7); step st covers keys 16 st
        // .. 16 st + 15 of the tile: registers 8 (st % 2) .. + 7 of block st / 2
        float m_off = (m_ref == kNegInf) ? 0.0f : m_ref - kPScale;
        if constexpr (ALIBI) m_off = fmaf(-rb, p.scale_log2, m_off);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int kb = st >> 1, j0 = 8 * (st & 1);
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 =
                    __builtin_amdgcn_exp2f(fmaf(s[kb][j0 + 2 * i], p.scale_log2, -m_off));
                const float p1 =
                    __builtin_amdgcn_exp2f(fmaf(s[kb][j0 + 2 * i + 1], p.scale_log2, -m_off));
                const f16x2_t h = {(_Float16)p0, (_Float16)p1};
                // l sums the f16 weights the matrix cores use
                l = __builtin_amdgcn_fdot2(h, f16x2_t{(_Float16)1.0f, (_Float16)1.0f}, l, false);
                w[i] = __builtin_bit_cast(uint32_t, h);
            }
            pb[st] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    };

    // ---- slots: M_0, V_0, M_1, ..., V_{n-1}, M_n, each followed by a
    // barrier; waves 4-7 run one slot behind (a staging-only slot first),
    // waves 0-3 end with an empty slot, so every wave passes 2 n + 2 barriers
    if (grp == 1) {
        vector_cluster(-1);
        slot_barrier();
    }
    for (int a = 0; a < n_tiles; ++a) {
        matrix_cluster(a);
        slot_barrier();
        vector_cluster(a);
        slot_barrier();
    }
    matrix_cluster(n_tiles);
    slot_barrier();
    if (grp == 0) slot_barrier();

    // ---- combine the two halves of each row and write (or merge) out / lse
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || !ctx_ok || regen_bad;
    const float l_row = l + __shfl_xor(l, 32);
    if (t >= n_q) return;
    float *dst = p.out + orow0 * kD;
    const float m_off = (m_ref == kNegInf) ? 0.0f : m_ref - kPScale;
    // this window's lse (natural log), -inf when the row saw no key here
    const float lse_w = l_row > 0.0f ? (m_off + log2f(l_row)) * kLn2 : kNegInf;
    float wa = 0.0f, wb = l_row > 0.0f ? 1.0f / l_row : 0.0f, lse_new = lse_w;
    if (p.carry) {
        // merge with the earlier windows: out = e^(lse_p - lse) out_p +
        // e^(lse_w - lse) o / l
        const float lse_p = p.lse[orow0];
        const float mx = fmaxf(lse_p, lse_w);
        if (mx == kNegInf) {
            wa = 0.0f;
            wb = 0.0f;
            lse_new = kNegInf;
        } else {
            const float ea = __expf(lse_p - mx), eb = __expf(lse_w - mx);
            const float sum = ea + eb;
            lse_new = mx + __logf(sum);
            wa = ea / sum;
            wb = l_row > 0.0f ? (eb / sum) / l_row : 0.0f;
        }
        if (lse_p != lse_p) lse_new = qnan;  // an earlier window failed
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d0 = 32 * b + 8 * jj + 4 * half;
            float4 v = make_float4(o[b][4 * jj] * wb, o[b][4 * jj + 1] * wb,
                                   o[b][4 * jj + 2] * wb, o[b][4 * jj + 3] * wb);
            if (p.carry) {
                const float4 op = *reinterpret_cast<const float4 *>(dst + d0);
                v = make_float4(fmaf(op.x, wa, v.x), fmaf(op.y, wa, v.y), fmaf(op.z, wa, v.z),
                                fmaf(op.w, wa, v.w));
            }
            if (any_bad || lse_new != lse_new) v = make_float4(qnan, qnan, qnan, qnan);
            *reinterpret_cast<float4 *>(dst + d0) = v;
        }
    }
    if (half == 0) p.lse[orow0] = any_bad ? qnan : lse_new;
}

template <int KV, bool A, bool R>
hipError_t by_group(const PrefillParams &p, int group, hipStream_t s) {
    const int64_t blocks = (int64_t)p.num_kv_heads * p.q_blocks * p.rows.num_seqs;
    if (blocks <= 0) return hipSuccess;
    switch (group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<KV, 1, A, R>), dim3((unsigned)blocks), dim3(512), 0, s, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<KV, 2, A, R>), dim3((unsigned)blocks), dim3(512), 0, s, p); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<KV, 4, A, R>), dim3((unsigned)blocks), dim3(512), 0, s, p); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<KV, 8, A, R>), dim3((unsigned)blocks), dim3(512), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int KV>
hipError_t by_policy(const PrefillParams &p, int group, hipStream_t s) {
    const bool a = p.pos.alibi != nullptr, r = p.pos.rope != 0;
    if (a && r) return by_group<KV, true, true>(p, group, s);
    if (a) return by_group<KV, true, false>(p, group, s);
    if (r) return by_group<KV, false, true>(p, group, s);
    return by_group<KV, false, false>(p, group, s);
}

}  // namespace

int prefill_rows_per_workgroup() { return 32 * kWaves; }

hipError_t launch_prefill(const PrefillParams &p, int kv_type, int group, hipStream_t stream) {
    if (kv_type == KV_BF16) return by_policy<KV_BF16>(p, group, stream);
    if (kv_type == KV_F16) return by_policy<KV_F16>(p, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace atlas
