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

// Base of K or V rows [key, key + 4) of (seq, kv head g) (four consecutive
// keys never straddle a page since page_tokens is a multiple of 16): a
// regenerated page in the workspace copy, or a resident page through the page
// table.  Sets `bad` for a block id outside the pool (rows of block 0 are
// read instead).
__device__ __forceinline__ int64_t kv_row_index(const PrefillParams &p, int seq, int g, int key,
                                                int n_regen, bool &in_regen, bool &bad) {
    const int P = p.page_tokens;
    const uint32_t lp = (__umulhi((uint32_t)key, p.p_magic) + (uint32_t)key) >> p.p_shift;
    const int row = key - (int)lp * P;
    in_regen = (int)lp < n_regen;
    if (in_regen) return (((int64_t)seq * p.max_regen + lp) * p.num_kv_heads + g) * P + row;
    int blk = p.page_table[(int64_t)seq * p.max_pages + lp];
    if (blk < 0 || blk >= p.num_blocks) {
        bad = true;
        blk = 0;
    }
    return ((int64_t)blk * p.num_kv_heads + g) * P + row;
}

template <int KV, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillParams p) {
    constexpr int kPosWave = 32 / G;       // positions per wave (32 rows)
    constexpr int kPosWg = 4 * kPosWave;   // positions per workgroup
    // Lazy rescale: the reference max of a row moves only when a tile's max
    // exceeds it by more than 2^8, so probabilities (scaled by 2^7) stay
    // below 2^15 and fit f16.
    constexpr float kSlack = 8.0f;
    constexpr float kPScale = 7.0f;
    const float kNegInf = -__builtin_inff();

    __shared__ __attribute__((aligned(16))) uint16_t sK[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kD * kVStride];

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

    // this lane's query row
    const int t = t_base + wave * kPosWave + r / G;
    const int head = g * G + (r % G);
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

    // Q^T operand: k-step ks holds dims 16 ks + 8 half .. + 8 of this row
    uint4 qf[8];
    {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                               ((int64_t)(q0 + t) * p.num_heads + head) * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = row_ok ? *reinterpret_cast<const uint4 *>(qrow + 16 * ks) : make_uint4(0, 0, 0, 0);
    }

    f32x16_t o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[b][j] = 0.0f;
    float m_ref = kNegInf, l = 0.0f;
    bool bad = false;

    // cooperative staging: thread (kg, dc) moves keys 4 kg .. 4 kg + 3, dims
    // 8 dc .. 8 dc + 7 of both K and V (one page lookup per thread and tile)
    const int dc = tid & 15;
    const int kg = tid >> 4;
    uint4 kreg[4], vreg[4];
    auto fetch = [&](int k0) {
        const int key = k0 + 4 * kg;
        if (key < key_limit) {
            bool in_regen;
            const int64_t row = kv_row_index(p, seq, g, key, n_regen, in_regen, bad);
            const uint16_t *kb = reinterpret_cast<const uint16_t *>(in_regen ? p.regen_k : p.k_pool) +
                                 row * kD + 8 * dc;
            const uint16_t *vb = reinterpret_cast<const uint16_t *>(in_regen ? p.regen_v : p.v_pool) +
                                 row * kD + 8 * dc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = key + i < key_limit;
                kreg[i] = ok ? *reinterpret_cast<const uint4 *>(kb + i * kD) : make_uint4(0, 0, 0, 0);
                vreg[i] = ok ? *reinterpret_cast<const uint4 *>(vb + i * kD) : make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kreg[i] = vreg[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4 *>(&sK[(4 * kg + i) * kKStride + 8 * dc]) = kreg[i];
        // transpose V (as f16): dims 8 dc + e, keys 4 kg .. 4 kg + 3
        if constexpr (KV == KV_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vreg[i].x = bf16x2_to_f16x2(vreg[i].x);
                vreg[i].y = bf16x2_to_f16x2(vreg[i].y);
                vreg[i].z = bf16x2_to_f16x2(vreg[i].z);
                vreg[i].w = bf16x2_to_f16x2(vreg[i].w);
            }
        }
        const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&vreg[0]);
        const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&vreg[1]);
        const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&vreg[2]);
        const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&vreg[3]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo01 = __builtin_amdgcn_perm(w1[w], w0[w], 0x05040100u);
            const uint32_t lo23 = __builtin_amdgcn_perm(w3[w], w2[w], 0x05040100u);
            const uint32_t hi01 = __builtin_amdgcn_perm(w1[w], w0[w], 0x07060302u);
            const uint32_t hi23 = __builtin_amdgcn_perm(w3[w], w2[w], 0x07060302u);
            const int d = 8 * dc + 2 * w;
            *reinterpret_cast<uint2 *>(&sV[d * kVStride + 4 * kg]) = make_uint2(lo01, lo23);
            *reinterpret_cast<uint2 *>(&sV[(d + 1) * kVStride + 4 * kg]) = make_uint2(hi01, hi23);
        }
    };

    const int n_tiles = (key_limit + kTile - 1) / kTile;
    if (n_tiles > 0) fetch(0);
    for (int tile = 0; tile < n_tiles; ++tile) {
        const int k0 = tile * kTile;
        __syncthreads();  // previous tile fully consumed
        stage();
        __syncthreads();
        if (tile + 1 < n_tiles) fetch(k0 + kTile);  // in flight during the math below

        // S^T for keys k0 .. k0 + 63 (two 32-key blocks), unscaled q.k
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint4 a = *reinterpret_cast<const uint4 *>(
                    &sK[(32 * kb + r) * kKStride + 16 * ks + 8 * half]);
                s[kb] = mfma32<KV>(a, qf[ks], s[kb]);
            }
        }

        // causal mask only on tiles that reach past some row's position
        if (!wave_rows_ok || k0 + kTile - 1 > wave_min_pos) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = k0 + 32 * kb + 8 * (j >> 2) + 4 * half + (j & 3);
                    s[kb][j] = (row_ok && key <= pos) ? s[kb][j] : kNegInf;
                }
            }
        }
        float mraw = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mraw = fmaxf(mraw, s[kb][j]);
        mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
        const float mt = mraw * p.scale_log2;  // scale > 0 keeps the order

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

        // P^T operands (f16, p * 2^7 relative to the reference max): PV step
        // st covers keys 16 st .. 16 st + 15 of the tile
        const float m_off = (m_ref == kNegInf) ? 0.0f : m_ref - kPScale;
        uint4 pb[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int kb = st >> 1, j0 = 8 * (st & 1);
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][j0 + 2 * i], p.scale_log2, -m_off));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][j0 + 2 * i + 1], p.scale_log2, -m_off));
                l += p0 + p1;
                const f16x2_t h = {(_Float16)p0, (_Float16)p1};
                w[i] = __builtin_bit_cast(uint32_t, h);
            }
            pb[st] = make_uint4(w[0], w[1], w[2], w[3]);
        }

        // O^T += V^T P^T (consecutive MFMAs use different accumulators)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint16_t *vrow = &sV[(32 * b + r) * kVStride + 4 * half + 16 * st];
                const uint2 va = *reinterpret_cast<const uint2 *>(vrow);
                const uint2 vb = *reinterpret_cast<const uint2 *>(vrow + 8);
                o[b] = mfma32<KV_F16>(make_uint4(va.x, va.y, vb.x, vb.y), pb[st], o[b]);
            }
        }
    }

    // combine the two halves of the row and write out / lse
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0 || !ctx_ok || regen_bad;
    const float l_row = l + __shfl_xor(l, 32);
    if (t < n_q) {
        const int64_t orow = (int64_t)(q0 + t) * p.num_heads + head;
        const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
        const float qnan = __builtin_nanf("");
        float *dst = p.out + orow * kD;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * b + 8 * jj + 4 * half;
                float4 v = make_float4(o[b][4 * jj] * inv, o[b][4 * jj + 1] * inv,
                                       o[b][4 * jj + 2] * inv, o[b][4 * jj + 3] * inv);
                if (any_bad) v = make_float4(qnan, qnan, qnan, qnan);
                *reinterpret_cast<float4 *>(dst + d0) = v;
            }
        }
        if (half == 0) {
            const float m_off = (m_ref == kNegInf) ? 0.0f : m_ref - kPScale;
            float lse = l_row > 0.0f ? (m_off + log2f(l_row)) * kLn2 : kNegInf;
            p.lse[orow] = any_bad ? qnan : lse;
        }
    }
}

template <int KV>
hipError_t by_group(const PrefillParams &p, int group, hipStream_t s) {
    const int64_t blocks = (int64_t)p.num_kv_heads * p.q_blocks * p.rows.num_seqs;
    if (blocks <= 0) return hipSuccess;
    switch (group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<KV, 1>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<KV, 2>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<KV, 4>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<KV, 8>), dim3((unsigned)blocks), dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int prefill_positions_per_block(int group) { return 128 / group; }

hipError_t launch_prefill(const PrefillParams &p, int kv_type, int group, hipStream_t stream) {
    if (kv_type == KV_BF16) return by_group<KV_BF16>(p, group, stream);
    if (kv_type == KV_F16) return by_group<KV_F16>(p, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace atlas
