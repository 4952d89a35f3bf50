// Paged decode attention on the vector ALUs, split-K over pages, and the
// log-sum-exp merge of the splits.
//
// Method (CFR-Atlas README, overview; ARGUS "Latency & Throughput Impact"):
// the keys of one (query row, kv head) are folded tile by tile with an
// online softmax -- running max m, running sum l, running accumulator acc,
// rescaled by exp(m_old - m_new) whenever the max grows -- so the K/V pages
// are never concatenated.  The context is cut into splits of a fixed number
// of tokens (cortiq README, "split-K flash-decoding"); every split is one
// workgroup and writes a normalised partial (o, lse); a second kernel merges
// the partials of every row by log-sum-exp (attnres AGENTS.md, "online
// softmax merge").  Merging inside the attention kernel would need a
// device-scope release per workgroup, which on this chip writes back the L2
// and costs far more than the extra launch.
//
// gfx950 mapping.  A workgroup is 4 wave64s and owns one (row, kv head,
// split).  Inside a wave the 64 lanes form 4 row-slots of 16 lanes; a
// row-slot walks U consecutive tokens of one page and its 16 lanes split the
// head_dim of each K/V row, so every load is a 16-lane-contiguous 128-bit (or
// narrower) vector load of one row: fully coalesced whatever the page size.
// The 16 partial dot products of a row are summed with DPP row rotations.
// All G query heads that share the kv head are computed from the same loaded
// K/V registers (GQA/MQA: K/V bytes are read once per kv head).
// Tokens past the visible range are excluded by selects, never by multiplying
// by zero, so NaN poison in page tails cannot leak.
//
// Tiered mode (ARGUS "Visual Architecture", "Why It Works"): a page's tier
// comes from its page-table entry; int8 / int4 / FP8 / INT2 codes are
// widened in registers, the K scale multiplies the finished dot product and the V scale
// multiplies the probability, so no dequantised page is ever written.
// Regen mode (CFR-Atlas README, overview and KvRegenerator): leading pages are
// regenerated inside the kernel from the counter-based SplitMix64 definition,
// each value exactly once per call.
#include "device.h"

namespace atlas {

namespace {

constexpr int kWaves = 4;
constexpr int kStagedPages = kDecodeStagedPages;

template <int KV>
constexpr int hot_bytes() { return KV == KV_F32 ? 4 : 2; }

struct SlotData {
    float kscale, vscale;
};

// Loads U rows x E elements of K and V for one row-slot, widened to f32.
// Returns false if the page-table entry is invalid (caller marks the row bad).
template <int KV, int D, int U, int MODE>
__device__ __forceinline__ bool load_slot(const DecodeParams &p, uint32_t entry, int g, int tok0,
                                          int lp, int n_regen, int c, float (&kf)[U][D / 16],
                                          float (&vf)[U][D / 16], SlotData &sd,
                                          const double (&rt)[D / 32]) {
    constexpr int E = D / 16;
    const int P = p.page_tokens;
    const int off = tok0 % P;
    sd.kscale = 1.0f;
    sd.vscale = 1.0f;

    if constexpr (MODE == MODE_REGEN) {
        if (lp < n_regen) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int dim = c * E + e;
                    kf[u][e] = regen_value(p.seed, regen_counter(p.layer, g, tok0 + u, dim, 0));
                    vf[u][e] = regen_value(p.seed, regen_counter(p.layer, g, tok0 + u, dim, 1));
                }
            }
            if (p.pos.rope) {
                // regenerated keys are replayed unrotated; the cached key
                // they stand for is the rotated key in bf16
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < E / 2; ++m) {
                        rope_rotate(kf[u][2 * m], kf[u][2 * m + 1], tok0 + u, rt[m]);
                        kf[u][2 * m] = bf16_round(kf[u][2 * m]);
                        kf[u][2 * m + 1] = bf16_round(kf[u][2 * m + 1]);
                    }
            }
            return true;
        }
    }

    uint32_t tier = 0, slot = entry;
    if constexpr (MODE == MODE_TIERED) tier = (uint32_t)entry_class(entry, slot);

    if (tier == 0) {
        if (slot >= (uint32_t)p.num_blocks) return false;
        constexpr int NB = E * hot_bytes<KV>();
        const int64_t row0 = ((int64_t)slot * p.num_kv_heads + g) * P + off;
        const char *kb = reinterpret_cast<const char *>(p.k_pool) +
                         (row0 * D + c * E) * hot_bytes<KV>();
        const char *vb = reinterpret_cast<const char *>(p.v_pool) +
                         (row0 * D + c * E) * hot_bytes<KV>();
        uint32_t kw[U][(NB + 3) / 4], vw[U][(NB + 3) / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            load_words<NB>(kw[u], kb + (int64_t)u * D * hot_bytes<KV>());
            load_words<NB>(vw[u], vb + (int64_t)u * D * hot_bytes<KV>());
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kf[u][e] = widen_word<KV>(kw[u], e);
                vf[u][e] = widen_word<KV>(vw[u], e);
            }
        }
        return true;
    }

    if constexpr (MODE == MODE_TIERED) {
        if (tier == 1) {
            if (slot >= (uint32_t)p.n_i8) return false;
            const int64_t row0 = ((int64_t)slot * p.num_kv_heads + g) * P + off;
            const int8_t *kb = p.i8_k + row0 * D + c * E;
            const int8_t *vb = p.i8_v + row0 * D + c * E;
            uint32_t kw[U][(E + 3) / 4], vw[U][(E + 3) / 4];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_words<E>(kw[u], kb + (int64_t)u * D);
                load_words<E>(vw[u], vb + (int64_t)u * D);
            }
            sd.kscale = p.i8_ks[(int64_t)slot * p.num_kv_heads + g];
            sd.vscale = p.i8_vs[(int64_t)slot * p.num_kv_heads + g];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int sh = 24 - 8 * (e & 3);
                    kf[u][e] = (float)sext_field(kw[u][e >> 2], sh, 8);
                    vf[u][e] = (float)sext_field(vw[u][e >> 2], sh, 8);
                }
            }
            return true;
        }
        if (tier == 2) {
            if (slot >= (uint32_t)p.n_i4) return false;
            constexpr int NB = E / 2;
            const int64_t row0 = ((int64_t)slot * p.num_kv_heads + g) * P + off;
            const uint8_t *kb = p.i4_k + row0 * (D / 2) + c * (E / 2);
            const uint8_t *vb = p.i4_v + row0 * (D / 2) + c * (E / 2);
            uint32_t kw[U][(NB + 3) / 4], vw[U][(NB + 3) / 4];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_words<NB>(kw[u], kb + (int64_t)u * (D / 2));
                load_words<NB>(vw[u], vb + (int64_t)u * (D / 2));
            }
            sd.kscale = p.i4_ks[(int64_t)slot * p.num_kv_heads + g];
            sd.vscale = p.i4_vs[(int64_t)slot * p.num_kv_heads + g];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    // element e is nibble e of the little-endian word
                    const int sh = 28 - 4 * (e & 7);
                    kf[u][e] = (float)sext_field(kw[u][e >> 3], sh, 4);
                    vf[u][e] = (float)sext_field(vw[u][e >> 3], sh, 4);
                }
            }
            return true;
        }
        if (tier == CLS_I2) {  // INT2 codes, four per byte
            if (slot >= (uint32_t)p.n_i2) return false;
            constexpr int NB = E / 4;
            const int64_t row0 = ((int64_t)slot * p.num_kv_heads + g) * P + off;
            const uint8_t *kb = p.i2_k + row0 * (D / 4) + c * NB;
            const uint8_t *vb = p.i2_v + row0 * (D / 4) + c * NB;
            uint32_t kw[U][1], vw[U][1];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_words<NB>(kw[u], kb + (int64_t)u * (D / 4));
                load_words<NB>(vw[u], vb + (int64_t)u * (D / 4));
            }
            sd.kscale = p.i2_ks[(int64_t)slot * p.num_kv_heads + g];
            sd.vscale = p.i2_vs[(int64_t)slot * p.num_kv_heads + g];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int e = 0; e < E; ++e) {  // element e: bits 2e, 2e + 1
                    kf[u][e] = (float)sext_field(kw[u][0], 30 - 2 * e, 2);
                    vf[u][e] = (float)sext_field(vw[u][0], 30 - 2 * e, 2);
                }
            }
            return true;
        }
        if (tier == CLS_F8) {  // FP8 E4M3 codes, widened by the hardware conversion
            if (slot >= (uint32_t)p.n_f8) return false;
            const int64_t row0 = ((int64_t)slot * p.num_kv_heads + g) * P + off;
            const uint8_t *kb = p.f8_k + row0 * D + c * E;
            const uint8_t *vb = p.f8_v + row0 * D + c * E;
            uint32_t kw[U][(E + 3) / 4], vw[U][(E + 3) / 4];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_words<E>(kw[u], kb + (int64_t)u * D);
                load_words<E>(vw[u], vb + (int64_t)u * D);
            }
            sd.kscale = p.f8_ks[(int64_t)slot * p.num_kv_heads + g];
            sd.vscale = p.f8_vs[(int64_t)slot * p.num_kv_heads + g];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int wi = 0; wi < E / 4; ++wi) {  // bytes 0, 1 then 2, 3 of each word
                    typedef float f2 __attribute__((ext_vector_type(2)));
                    const f2 k01 = __builtin_amdgcn_cvt_pk_f32_fp8(kw[u][wi], false);
                    const f2 k23 = __builtin_amdgcn_cvt_pk_f32_fp8(kw[u][wi], true);
                    const f2 v01 = __builtin_amdgcn_cvt_pk_f32_fp8(vw[u][wi], false);
                    const f2 v23 = __builtin_amdgcn_cvt_pk_f32_fp8(vw[u][wi], true);
                    kf[u][4 * wi] = k01[0];
                    kf[u][4 * wi + 1] = k01[1];
                    kf[u][4 * wi + 2] = k23[0];
                    kf[u][4 * wi + 3] = k23[1];
                    vf[u][4 * wi] = v01[0];
                    vf[u][4 * wi + 1] = v01[1];
                    vf[u][4 * wi + 2] = v23[0];
                    vf[u][4 * wi + 3] = v23[1];
                }
            }
            return true;
        }
    }
    return false;
}

// Log-sum-exp merge of `nsplit` normalised partials of one output row
// (attnres AGENTS.md, "online softmax merge"): lse = M + log sum_s
// exp(lse_s - M), out = sum_s exp(lse_s - lse) o_s.  One wave per row: lane
// l owns dims l + 64 k (k < KD).  The splits are folded in chunks of 32 / KD
// with a running max, every load of a chunk issued before its first use, so
// a row costs one memory round trip per chunk and no barrier.  The order is
// fixed (deterministic).  Any NaN partial makes the row NaN; a row whose
// splits are all empty gets out 0 and lse -inf.
template <int KD>
__device__ void merge_row_wave(const float *pl, int64_t l_stride, const float *po,
                               int64_t o_stride, int nsplit, int D, float *out, float *lse_out,
                               int lane) {
    constexpr int C = 32 / KD;
    const float kNegInf = -__builtin_inff();
    float M = kNegInf, L = 0.0f, acc[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) acc[k] = 0.0f;
    bool nan = false;
    for (int c0 = 0; c0 < nsplit; c0 += C) {
        float ls[C], ov[C][KD];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const bool in = c0 + j < nsplit;
            ls[j] = in ? pl[(int64_t)(c0 + j) * l_stride] : kNegInf;
#pragma unroll
            for (int k = 0; k < KD; ++k) {
                const int d = lane + 64 * k;
                ov[j][k] = (in && d < D) ? po[(int64_t)(c0 + j) * o_stride + d] : 0.0f;
            }
        }
        float mc = kNegInf;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            nan = nan || (ls[j] != ls[j]);
            mc = fmaxf(mc, ls[j]);
        }
        const float m_new = fmaxf(M, mc);
        if (m_new == kNegInf) continue;  // every split so far is empty
        const float f = (M == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((M - m_new) * kLog2e);
        L *= f;
#pragma unroll
        for (int k = 0; k < KD; ++k) acc[k] *= f;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const float w =
                (ls[j] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((ls[j] - m_new) * kLog2e);
            L += w;
#pragma unroll
            for (int k = 0; k < KD; ++k) acc[k] = fmaf(w, ov[j][k], acc[k]);
        }
        M = m_new;
    }
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int k = 0; k < KD; ++k) {
        const int d = lane + 64 * k;
        if (d < D) out[d] = nan ? qnan : (L > 0.0f ? acc[k] / L : 0.0f);
    }
    if (lane == 0) *lse_out = nan ? qnan : (L > 0.0f ? M + logf(L) : kNegInf);
}

template <int KV, int D, int G, int MODE>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    constexpr int E = D / 16;           // head_dim elements per lane
    constexpr int U = (E >= 8 || G >= 4) ? 8 : 16;  // tokens per row-slot per tile
    constexpr int TILE = 4 * U;         // tokens per wave per tile
    const float kNegInf = -__builtin_inff();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane >> 4;
    const int c = lane & 15;

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

    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    // positional policy: the row sits at its own key, qpos
    const int qpos = nvis - 1;
    double rt[E / 2];  // rotary turns per position of this lane's dim pairs
#pragma unroll
    for (int m = 0; m < E / 2; ++m)
        rt[m] = p.pos.rope ? rope_turns(c * E / 2 + m, D, p.pos.rope_log2_theta) : 0.0;
    const bool alibi = p.pos.alibi != nullptr;
    float ab[G];  // ALiBi slope of each head, log2 units
#pragma unroll
    for (int h = 0; h < G; ++h) ab[h] = alibi ? p.pos.alibi[g * G + h] * kLog2e : 0.0f;

    float qv[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int64_t qo = ((int64_t)row * p.num_heads + g * G + h) * D + c * E;
#pragma unroll
        for (int e = 0; e < E; ++e) qv[h][e] = load_elem(p.q, qo + e, p.q_dtype);
        if (p.pos.rope) {
#pragma unroll
            for (int m = 0; m < E / 2; ++m) rope_rotate(qv[h][2 * m], qv[h][2 * m + 1], qpos, rt[m]);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) qv[h][e] *= p.scale_log2;
    }

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }
    bool bad = !row_ok;

    const int n_tiles = t1 > t0 ? (t1 - t0 + TILE - 1) / TILE : 0;
    const int32_t *trow = p.page_table + (int64_t)seq * p.max_pages;
    // page-table entries of this split, staged once (a dependent global load
    // per tile would add a memory round trip before every K/V load)
    __shared__ int32_t s_pages[kStagedPages];
    const int lp_first = t0 / p.page_tokens;
    const int lp_count = t1 > t0 ? (t1 - 1) / p.page_tokens - lp_first + 1 : 0;
    const bool staged = lp_count <= kStagedPages;
    if (staged)
        for (int i = threadIdx.x; i < lp_count; i += 256) s_pages[i] = trow[lp_first + i];
    __syncthreads();
    int n_regen = 0;
    if constexpr (MODE == MODE_REGEN) {
        n_regen = row_ok ? p.regen_pages[seq] : 0;
        if (n_regen < 0 || n_regen > p.max_regen) {  // outside the host bound: fail loudly
            bad = true;
            n_regen = 0;
        }
    }

    // Resident pages with few registers per token (at most 16 bytes per row
    // and lane, at most 8 accumulators per lane): software pipeline over
    // 32-token tiles (8 tokens per row-slot), two register sets used in
    // turn, so the next tile's K/V loads are in flight while this tile is
    // folded.  Wider shapes keep the single-buffered loop (their second
    // register set would halve the waves per SIMD).
    constexpr int NB = E * hot_bytes<KV>();  // bytes per row and lane
    constexpr int NW = (NB + 3) / 4;
    constexpr bool kPipe = MODE == MODE_PLAIN && NW <= 4 && G * E <= 8;
    if constexpr (kPipe) {
        constexpr int UP = 8;
        constexpr int TP = 4 * UP;
        const int n_tiles_p = t1 > t0 ? (t1 - t0 + TP - 1) / TP : 0;
        const int P = p.page_tokens;
        struct Raw {
            uint32_t k[UP][NW], v[UP][NW];
            int tok0;
            bool live;
        };
        auto load = [&](int tile, Raw &R) {
            R.tok0 = t0 + tile * TP + r * UP;  // UP tokens of one page (P % 16 == 0)
            R.live = tile < n_tiles_p && R.tok0 < t1;
            if (R.live) {
                const int lp = R.tok0 / P;
                const uint32_t slot = (uint32_t)(staged ? s_pages[lp - lp_first] : trow[lp]);
                if (slot >= (uint32_t)p.num_blocks) {
                    bad = true;
                    R.live = false;
                } else {
                    const int64_t row0 = ((int64_t)slot * p.num_kv_heads + g) * P + (R.tok0 - lp * P);
                    const char *kb = reinterpret_cast<const char *>(p.k_pool) +
                                     (row0 * D + c * E) * hot_bytes<KV>();
                    const char *vb = reinterpret_cast<const char *>(p.v_pool) +
                                     (row0 * D + c * E) * hot_bytes<KV>();
#pragma unroll
                    for (int u = 0; u < UP; ++u) {
                        load_words<NB>(R.k[u], kb + (int64_t)u * D * hot_bytes<KV>());
                        load_words<NB>(R.v[u], vb + (int64_t)u * D * hot_bytes<KV>());
                    }
                }
            }
        };
        auto fold = [&](const Raw &R) {
            float s[G][UP];
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                const bool valid = R.live && (R.tok0 + u < t1);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float part = 0.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        part = fmaf(qv[h][e], widen_word<KV>(R.k[u], e), part);
                    const float dot = row16_sum(part);
                    s[h][u] = valid ? dot : kNegInf;
                    if (alibi) s[h][u] = fmaf(ab[h], (float)(R.tok0 + u - qpos), s[h][u]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float mt = s[h][0];
#pragma unroll
                for (int u = 1; u < UP; ++u) mt = fmaxf(mt, s[h][u]);
                const float m_new = fmaxf(m[h], mt);
                const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m[h] - m_use);
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
#pragma unroll
                for (int u = 0; u < UP; ++u) {
                    const bool valid = R.live && (R.tok0 + u < t1);
                    const float pr = __builtin_amdgcn_exp2f(s[h][u] - m_use);
                    l[h] += pr;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float x = valid ? widen_word<KV>(R.v[u], e) : 0.0f;
                        acc[h][e] = fmaf(pr, x, acc[h][e]);
                    }
                }
                m[h] = m_new;
            }
        };
        Raw A, B;
        load(wave, A);
        for (int tile = wave; tile < n_tiles_p; tile += 2 * kWaves) {
            load(tile + kWaves, B);
            fold(A);
            if (tile + kWaves >= n_tiles_p) break;
            load(tile + 2 * kWaves, A);
            fold(B);
        }
    } else {
        for (int tile = wave; tile < n_tiles; tile += kWaves) {
            const int tok0 = t0 + tile * TILE + r * U;  // first token of this row-slot
            float kf[U][E], vf[U][E];
            SlotData sd{1.0f, 1.0f};
            bool live = tok0 < t1;
            if (live) {
                const int lp = tok0 / p.page_tokens;
                uint32_t entry = 0;
                if (!(MODE == MODE_REGEN && lp < n_regen))
                    entry = (uint32_t)(staged ? s_pages[lp - lp_first] : trow[lp]);
                if (!load_slot<KV, D, U, MODE>(p, entry, g, tok0, lp, n_regen, c, kf, vf, sd, rt)) {
                    bad = true;
                    live = false;
                }
            }
            if (!live) {
    #pragma unroll
                for (int u = 0; u < U; ++u)
    #pragma unroll
                    for (int e = 0; e < E; ++e) kf[u][e] = vf[u][e] = 0.0f;
            }

            // scores in the log2 domain, masked past the visible range
            float s[G][U];
    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool valid = live && (tok0 + u < t1);
    #pragma unroll
                for (int h = 0; h < G; ++h) {
                    float part = 0.0f;
    #pragma unroll
                    for (int e = 0; e < E; ++e) part = fmaf(qv[h][e], kf[u][e], part);
                    const float dot = row16_sum(part) * sd.kscale;
                    s[h][u] = valid ? dot : kNegInf;
                    if (alibi) s[h][u] = fmaf(ab[h], (float)(tok0 + u - qpos), s[h][u]);
                }
    #pragma unroll
                for (int e = 0; e < E; ++e) vf[u][e] = valid ? vf[u][e] : 0.0f;
            }

            // online softmax update of this row-slot's state
    #pragma unroll
            for (int h = 0; h < G; ++h) {
                float mt = s[h][0];
    #pragma unroll
                for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[h][u]);
                const float m_new = fmaxf(m[h], mt);
                const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m[h] - m_use);
                l[h] *= alpha;
    #pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
    #pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float pr = __builtin_amdgcn_exp2f(s[h][u] - m_use);
                    l[h] += pr;
                    const float pv = pr * sd.vscale;
    #pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pv, vf[u][e], acc[h][e]);
                }
                m[h] = m_new;
            }
        }
    }

    // merge the 4 row-slots of the wave (lanes c, c+16, c+32, c+48)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = fmaxf(m[h], __shfl_xor(m[h], 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float M_use = (M == kNegInf) ? 0.0f : M;
        const float f = __builtin_amdgcn_exp2f(m[h] - M_use);
        float lw = l[h] * f;
        lw += __shfl_xor(lw, 16);
        lw += __shfl_xor(lw, 32);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float a = acc[h][e] * f;
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            acc[h][e] = a;
        }
        m[h] = M;
        l[h] = lw;
    }
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[wave][h][c * E + e] = acc[h][e];
            if (c == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
    }
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;

    // merge the waves in a fixed order: this split's normalised result
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
            for (int col = lane; col < D; col += 64) {
                float o = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) o = fmaf(fw[w], s_acc[w][h][col], o);
                o = L > 0.0f ? o / L : 0.0f;
                if (any_bad) o = qnan;
                if (final_here) p.out[orow * D + col] = o;
                else p.part_o[(orow * p.max_splits + split) * D + col] = o;
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

// Split merge: one wave per merged row, four rows per workgroup.  With
// fixed_splits == 0 the number of splits of a row follows from its visible
// keys (decode path).
template <int KD>
__global__ __launch_bounds__(256) void fold_kernel(const FoldParams f) {
    const int lane = threadIdx.x & 63;
    const int idx = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (idx >= f.rows) return;
    int nsplit = f.fixed_splits;
    if (nsplit <= 0) {
        int seq, vis;
        map_row(f.map, idx / f.num_heads, seq, vis);
        nsplit = splits_of(vis, f.split_tokens);
        if (nsplit == 1) return;  // written directly by the attention kernel
    }
    merge_row_wave<KD>(f.part_lse + (int64_t)idx * f.l_row_stride, f.l_split_stride,
                       f.part_o + (int64_t)idx * f.o_row_stride, f.o_split_stride, nsplit,
                       f.head_dim, f.out + (int64_t)idx * f.head_dim, f.lse + idx, lane);
}

template <int KV, int D, int G, int MODE>
hipError_t launch_one(const DecodeParams &p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.total_q * p.num_kv_heads * p.max_splits;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<KV, D, G, MODE>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <int KV, int D, int MODE>
hipError_t by_group(const DecodeParams &p, int group, hipStream_t s) {
    switch (group) {
        case 1: return launch_one<KV, D, 1, MODE>(p, s);
        case 2: return launch_one<KV, D, 2, MODE>(p, s);
        case 4: return launch_one<KV, D, 4, MODE>(p, s);
        case 8: return launch_one<KV, D, 8, MODE>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int KV, int MODE>
hipError_t by_dim(const DecodeParams &p, int head_dim, int group, hipStream_t s) {
    switch (head_dim) {
        case 64: return by_group<KV, 64, MODE>(p, group, s);
        case 128: return by_group<KV, 128, MODE>(p, group, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int kv_type, int head_dim, int group, int mode,
                         hipStream_t stream) {
    if (mode == MODE_PLAIN) {
        switch (kv_type) {
            case KV_F32: return by_dim<KV_F32, MODE_PLAIN>(p, head_dim, group, stream);
            case KV_BF16: return by_dim<KV_BF16, MODE_PLAIN>(p, head_dim, group, stream);
            case KV_F16: return by_dim<KV_F16, MODE_PLAIN>(p, head_dim, group, stream);
        }
    } else if (mode == MODE_TIERED) {
        switch (kv_type) {
            case KV_BF16: return by_dim<KV_BF16, MODE_TIERED>(p, head_dim, group, stream);
            case KV_F16: return by_dim<KV_F16, MODE_TIERED>(p, head_dim, group, stream);
        }
    } else if (mode == MODE_REGEN) {
        if (kv_type == KV_BF16) return by_dim<KV_BF16, MODE_REGEN>(p, head_dim, group, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fold(const FoldParams &f, hipStream_t stream) {
    if (f.rows <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((f.rows + 3) / 4);
    if (f.head_dim <= 64)
        hipLaunchKernelGGL(fold_kernel<1>, dim3(blocks), dim3(256), 0, stream, f);
    else if (f.head_dim <= 128)
        hipLaunchKernelGGL(fold_kernel<2>, dim3(blocks), dim3(256), 0, stream, f);
    else
        hipLaunchKernelGGL(fold_kernel<4>, dim3(blocks), dim3(256), 0, stream, f);
    return hipGetLastError();
}

}  // namespace atlas
