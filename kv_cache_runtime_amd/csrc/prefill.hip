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
//                                                  A = V^T from LDS, one 16-byte
//                                                  read, B = P^T in VGPRs)
// so each row lives in one lane pair (r, r + 32) for the softmax.
//
// Schedule.  The waves of a workgroup are dealt to the four SIMDs
// round-robin, so two waves share each SIMD and its matrix core.  An
// exponential in one wave holds up the matrix instructions of the other, so
// each wave interleaves its own work instead: keys are folded in units of 32,
// and while the matrix core computes the scores of unit u + 1 the wave takes
// the exponentials of unit u between the products, whose second half
// alternates with the first P.V products of unit u.  The issue order inside
// a unit is fixed with scheduling barriers.  No row max is taken per unit:
// the reference max moves only when a half unit's f16 weights overflow
// (a score more than 9 log2 units above it), which the sum of that half's
// weights shows; the half is then redone.
//
// Staging.  The keys of the call come from a ring the window preparation
// kernel fills: K in the kv type, 64 contiguous key rows per tile, and V in
// f16, each 64-key tile stored dims-major (V^T, 128 rows of 64 keys) with
// the keys of every 16 ordered so that the eight a lane's P.V operand takes
// are adjacent.  A single 16-byte LDS read then yields that operand, where
// the key-major layout took two transposing 8-byte reads; the 16-byte reads
// sustain a higher LDS rate.
// They move from memory straight into LDS by DMA (global_load_lds), with no
// registers in between.  LDS holds five buffers of one K tile and one V tile
// each; a tile is issued four tiles ahead and the workgroup meets once per
// tile.  Rows are not padded: the 16-byte chunks of each row are permuted
// so that the fragment reads of the matrix operands hit distinct banks.
// P is kept relative to the reference max minus 7 and is at most 2^15, so
// P * V stays finite for |v| <= 65504, the f16 range that bf16 V must lie in.
#include <type_traits>

#include "device.h"

namespace atlas {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head_dim
constexpr int kTile = 64;        // keys per tile
constexpr int kWaves = 8;        // waves per workgroup
constexpr int kRowBytes = kD * 2;             // one staged K or V row
constexpr int kTileBytes = kTile * kRowBytes;  // one staged K or V tile
constexpr int kVtRowBytes = kTile * 2;         // one dim of a staged V^T tile

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

// Two packed bf16 values -> two packed f16 values (round to nearest even;
// exact for magnitudes in the f16 normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const f16x2_t h = {(_Float16)__uint_as_float(w << 16),
                       (_Float16)__uint_as_float(w & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, h);
}

// 16 bytes per lane from memory straight into LDS (buffer_load_dwordx4 ...
// lds): lane l reads the buffer at byte soffset + voffset and writes bytes
// 16 l .. 16 l + 15 after the wave-uniform LDS address dst; reads past the
// buffer's byte count return zeros.  Counted by vmcnt like any load.  The
// buffer form (not the global one) matters: the compiler treats a pending
// global-to-LDS load as an access of both memory kinds and then waits for
// every outstanding LDS read at each use of one, while a pending buffer load
// leaves its in-order LDS-read waits alone.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(const void *base, uint32_t bytes) {
    // last word: 32-bit data format (the untyped loads used here ignore it)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                          uint32_t soffset, uint16_t *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void *)(dst), 16, voffset,
        soffset, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): the tile DMAs issued before the last N
// loads have landed in LDS and this wave's LDS reads have returned.
template <int N>
__device__ __forceinline__ void tile_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Barrier between tiles.  Inside the key loop LDS is written only by the
// tile DMAs, whose completion tile_wait establishes, so no fence is used (a
// workgroup fence would also wait for the DMA still in flight).  The empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

    // five LDS buffers, each a K tile and a V tile; separate objects, so
    // that the compiler sees a DMA into one buffer does not alias reads of
    // another and adds no wait for it
    __shared__ __attribute__((aligned(1024))) uint16_t sB0[2 * kTile * kD], sB1[2 * kTile * kD],
        sB2[2 * kTile * kD], sB3[2 * kTile * kD], sB4[2 * kTile * kD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (scalar) so that the cluster branches below are uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // a regenerated-page count outside the host bound fails loudly (the
    // window preparation leaves such a sequence's ring rows alone)
    bool regen_bad = false;
    if (p.regen_pages != nullptr && ctx_ok) {
        const int n_regen = p.regen_pages[seq];
        regen_bad = n_regen < 0 || n_regen > p.max_regen;
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
    float m_ref = kNegInf, l = 0.0f;

    // ---- staging.  Tiles come from the window's ring [seq][kv head][key -
    // key_begin][D] (K in the kv type, rows past the context zero), so a K
    // tile is 64 contiguous rows of 256 bytes; the V ring holds the same
    // 16 KiB per tile as V^T, 128 dim rows of 64 f16 keys in the order
    // described at the window preparation kernel.  Tiles go straight from
    // memory into LDS by DMA (global_load_lds_dwordx4: lane l of a wave's
    // load fills bytes 16 l .. 16 l + 15 of a 1 KiB stretch, from any address
    // it names), four loads per thread per tile pair.  Rows are not padded;
    // instead the 16-byte chunks of a row are permuted so that the matrix
    // operand reads hit distinct banks: chunk c of K row k sits at position
    // c ^ (k % 16), chunk c of V^T row d at c ^ ((d / 2) % 8).
    // Content x is K of tile x and V of tile x - 1; it lives in buffer x % 5
    // and is issued three tiles before it is read.
    // buffer B: K tile at element 0, V tile at element kTile * kD
    auto kbuf = [&](auto b_c) __attribute__((always_inline)) -> uint16_t * {
        constexpr int B = decltype(b_c)::value % 5;
        if constexpr (B == 0) return sB0;
        else if constexpr (B == 1) return sB1;
        else if constexpr (B == 2) return sB2;
        else if constexpr (B == 3) return sB3;
        else return sB4;
    };
    auto vbuf = [&](auto b_c) __attribute__((always_inline)) -> uint16_t * {
        return kbuf(b_c) + kTile * kD;
    };
    const int64_t ring0 = ((int64_t)seq * p.num_kv_heads + g) * p.ring_tokens * kD;
    // this (sequence, kv head)'s ring rows as buffers (tile byte offsets go
    // in the scalar offset)
    const uint32_t ring_bytes = (uint32_t)p.ring_tokens * kRowBytes;
    const __amdgpu_buffer_rsrc_t rk =
        ring_rsrc(reinterpret_cast<const char *>(p.ring_k) + 2 * ring0, ring_bytes);
    const __amdgpu_buffer_rsrc_t rv =
        ring_rsrc(reinterpret_cast<const char *>(p.ring_v) + 2 * ring0, ring_bytes);
    // thread's DMA rows: K row 8 wave + 4 i + lane / 16 (i = 0, 1), position
    // lane % 16; V^T row (dim) 16 wave + 8 i + lane / 8, position lane % 8.
    // The byte offsets within a tile are recomputed at each use from a lane
    // index the compiler cannot hoist (keeping them costs registers the
    // products need)
    auto dma_offsets = [&](uint32_t (&ko)[2], uint32_t (&vo)[2]) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = 8 * wave + 4 * i + (ln >> 4), at = ln & 15;
            ko[i] = row * kRowBytes + ((at ^ (row & 15)) << 4);
            const int dim = 16 * wave + 8 * i + (ln >> 3), vat = ln & 7;
            vo[i] = dim * kVtRowBytes + ((vat ^ ((dim >> 1) & 7)) << 4);
        }
    };
    // Every content issues exactly four loads (past the tiles of the call
    // they read a clamped, valid tile that is never used), so a wait for
    // "all but the last four" means "all but the newest content".
    auto dma_content = [&](int x, auto b_c) __attribute__((always_inline)) {
        const int xk = min(x, n_tiles - 1);
        const int xv = max(min(x - 1, n_tiles - 1), 0);
        uint32_t kofs[2], vofs[2];
        dma_offsets(kofs, vofs);
        const uint32_t ks = (uint32_t)xk * kTileBytes, vs = (uint32_t)xv * kTileBytes;
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16(rk, kofs[i], ks, kbuf(b_c) + (8 * wave + 4 * i) * kD);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            lds_dma16(rv, vofs[i], vs, vbuf(b_c) + (16 * wave + 8 * i) * kTile);
    };

    // The keys are folded in units of 32 (unit u = keys 32 u .. 32 u + 31 of
    // the call, half u % 2 of tile u / 2), one 32 x 32 score block each.
    // ---- scores of unit u (K of tile u / 2, buffer B = (u / 2) % 5).  Lane
    // (r, half) reads chunk 2 ks + half of row 32 (u % 2) + r, which sits at
    // byte (r * 256 + ((half ^ r % 16) << 4)) ^ (ks << 5) of its half tile.
    const uint32_t kaddr = r * kRowBytes + ((half ^ (r & 15)) << 4);
    // the eight K read addresses of the key loop, kept (eight registers, one
    // XOR per read less); the V ones are rebuilt at each use
    uint32_t kaddrs[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kaddrs[ks] = kaddr ^ (ks << 5);
    auto scores = [&](int u, f32x16_t &dst, auto b_c) __attribute__((always_inline)) {
        const char *cK = reinterpret_cast<const char *>(kbuf(b_c)) + (u & 1) * (32 * kRowBytes);
        // the eight read addresses are rebuilt here from an opaque copy of
        // kaddr: hoisted out of the loop they would take eight registers
        uint32_t ka = kaddr;
        asm volatile("" : "+v"(ka));
        uint4 kf[2];
        kf[0] = *reinterpret_cast<const uint4 *>(cK + ka);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks < 7)
                kf[(ks + 1) & 1] = *reinterpret_cast<const uint4 *>(cK + (ka ^ ((ks + 1) << 5)));
            // the first step starts from a zero accumulator operand
            dst = mfma32<KV>(kf[ks & 1], qf[ks], ks == 0 ? f32x16_t{} : dst);
            if constexpr (ROPE) dst = mfma32<KV>(kf[ks & 1], qlo[ks], dst);
        }
    };
    // ---- P.V of unit u (V of tile u / 2, content u / 2 + 1, buffer B).  A =
    // V^T: lane (dim 32 b + r, half) takes keys 16 st + 4 half .. + 3 and
    // 16 st + 8 + 4 half .. + 3 of the unit, the key order of P^T's
    // registers.  The V^T tile holds those eight keys in one 16-byte chunk:
    // chunk 4 (u % 2) + 2 st + half of row 32 b + r, stored at chunk position
    // c ^ ((row / 2) % 8), i.e. byte vaddr ^ (st << 5) ^ ((u % 2) << 6) + 32 b * 128.
    // The LDS has 64 banks and serves a 16-byte read 16 lanes at a time: rows
    // r = 0 .. 15 of 128 bytes then land on bank groups 8 (r % 2) + position,
    // all distinct.
    const uint32_t vaddr = r * kVtRowBytes + ((half ^ ((r >> 1) & 7)) << 4);
    uint4 pb[2];  // P^T operands of the unit being folded
    // ---- softmax, part 1 (unit u): ALiBi, the causal mask (mask: the unit
    // reaches past some row's position), the row max and the new reference;
    // the rescale it implies is owed to the accumulators.  Score register j
    // holds key k0 + 8 (j / 4) + 4 half + j % 4 of row r.
    auto alibi_bias = [&](f32x16_t &sx) __attribute__((always_inline)) {
        if constexpr (ALIBI) {
#pragma unroll
            for (int j = 0; j < 16; ++j) sx[j] = fmaf(ab, (float)(8 * (j >> 2) + (j & 3)), sx[j]);
        }
    };
    auto causal_mask = [&](int u, f32x16_t &sx) __attribute__((always_inline)) {
        // register j is visible when its key offset 8 (j / 4) + j % 4 stays
        // within lim (a row outside the chunk sees nothing)
        const int lim = row_ok ? pos - kb0 - 32 * u - 4 * half : -1;
#pragma unroll
        for (int j = 0; j < 16; ++j) sx[j] = 8 * (j >> 2) + (j & 3) <= lim ? sx[j] : kNegInf;
    };
    // the first unit's reference: its row max (nothing is accumulated yet,
    // so nothing is rescaled)
    auto first_reference = [&](f32x16_t &sx, bool mask) __attribute__((always_inline)) {
        if (mask) causal_mask(0, sx);  // wave-uniform
        float mraw = kNegInf;
#pragma unroll
        for (int j = 0; j < 16; ++j) mraw = fmaxf(mraw, sx[j]);
        if constexpr (ALIBI) mraw += ab * (float)(kb0 + 4 * half - pos);
        {  // the row's other half (lane r + 32)
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw),
                                                            __float_as_uint(mraw), false, false);
            mraw = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
        }
        m_ref = mraw * p.scale_log2;  // scale > 0 keeps the order
    };
    // a unit needs the causal mask when it reaches past the first position of
    // the wave (or the wave holds rows past the chunk)
    auto masked = [&](int u) { return !wave_rows_ok || kb0 + 32 * u + 31 > wave_min_pos; };
    // One unit, in an explicit issue order (the compiler may not move code
    // across the scheduling barriers): the scores of unit u + 1 on the matrix
    // cores, each product beside one exponential pair of unit u and the read
    // of a K fragment two products ahead; the last four alternate with the
    // first four P.V products of unit u; then the other four P.V products.
    // sc holds unit u's scores, sn receives unit u + 1's.  MORE: a unit
    // follows; KB / VB: the buffers of the K tile of unit u + 1 and of the V
    // tile of unit u.
    auto unit = [&](int u, f32x16_t &sc, f32x16_t &sn, auto more_c, auto kb_c,
                    auto vb_c) __attribute__((always_inline)) {
        constexpr bool MORE = decltype(more_c)::value;
        constexpr int kAhead = 2;  // K fragments in flight
        // (no rescale is owed here: the reference moves only inside a unit,
        // which rescales at once; the first unit's reference finds o = 0)
        const char *cK =
            reinterpret_cast<const char *>(kbuf(kb_c)) + ((u + 1) & 1) * (32 * kRowBytes);
        const char *cV = reinterpret_cast<const char *>(vbuf(vb_c));
        // the V read addresses are rebuilt here from an opaque copy: hoisted
        // out of the loop they would take more registers than are left
        uint32_t va = vaddr ^ ((u & 1) << 6);
        asm volatile("" : "+v"(va));
        uint4 kf[8];
        uint4 vf[2][4];
        auto kread = [&](int ks) __attribute__((always_inline)) {
            kf[ks] = *reinterpret_cast<const uint4 *>(cK + kaddrs[ks]);
        };
        auto vread = [&](int st, int b) __attribute__((always_inline)) {
            vf[st][b] = *reinterpret_cast<const uint4 *>(cV + (va ^ (st << 5)) + 32 * b * kVtRowBytes);
        };
        if constexpr (ALIBI) {
            // The bias makes a row's scores climb toward its own position, so
            // the overflow check below would fire (and redo a half) in most
            // units.  Under ALiBi the reference instead follows the unit's
            // row max, lazily (only past the slack), with a rescale that
            // costs no exponential of the unit's weights.
            float mraw = kNegInf;
#pragma unroll
            for (int j = 0; j < 16; ++j) mraw = fmaxf(mraw, sc[j]);
            mraw += ab * (float)(kb0 + 32 * u + 4 * half - pos);
            const auto hm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw),
                                                             __float_as_uint(mraw), false, false);
            mraw = fmaxf(__uint_as_float(hm[0]), __uint_as_float(hm[1]));
            const float mt = mraw * p.scale_log2;
            const bool move = mt > m_ref + kSlack;
            if (__any(move)) {  // wave-uniform
                const float m_new = move ? mt : m_ref;
                const float a = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
                m_ref = m_new;
                l *= a;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[b][j] *= a;
            }
        }
        // probabilities of unit u as f16 P^T operands, relative to m_ref - 7;
        // pair i is registers 2 i, 2 i + 1 (step i / 4 of the P.V).  l sums
        // the f16 weights the matrix cores use.
        float m_off = (m_ref == kNegInf) ? 0.0f : m_ref - kPScale;
        if constexpr (ALIBI)
            m_off = fmaf(-ab * (float)(kb0 + 32 * u + 4 * half - pos), p.scale_log2, m_off);
        uint32_t w[8];
        float lh = 0.0f;  // the f16 weights of the current half unit
        auto pexp = [&](int i) __attribute__((always_inline)) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[2 * i], p.scale_log2, -m_off));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[2 * i + 1], p.scale_log2, -m_off));
            const f16x2_t h = {(_Float16)p0, (_Float16)p1};
            lh = __builtin_amdgcn_fdot2(h, f16x2_t{(_Float16)1.0f, (_Float16)1.0f}, lh, false);
            w[i] = __builtin_bit_cast(uint32_t, h);
            // keep the pair here, beside its matrix product (the compiler
            // would otherwise sink it to its use after the mask branch)
            asm volatile("" : "+v"(w[i]), "+v"(lh));
        };
        // A half unit whose weights overflowed f16 (a key more than 9 log2
        // units above the reference) is redone: the reference moves to the
        // unit's row max, the accumulators are rescaled, and the half's
        // weights are recomputed.  Rare: it needs a score far above every
        // earlier one of the row.
        auto check_half = [&](int h) __attribute__((always_inline)) {
            if (__any(!(lh < __builtin_inff()))) {  // wave-uniform; NaN lands here too
                float mraw = kNegInf;  // over this half's scores (the other half
#pragma unroll                                 // checks its own)
                for (int j = 8 * h; j < 8 * h + 8; ++j) mraw = fmaxf(mraw, sc[j]);
                if constexpr (ALIBI) mraw += ab * (float)(kb0 + 32 * u + 4 * half - pos);
                const auto hm = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(mraw), __float_as_uint(mraw), false, false);
                mraw = fmaxf(__uint_as_float(hm[0]), __uint_as_float(hm[1]));
                const float mt = mraw * p.scale_log2;
                const bool move = mt > m_ref + kSlack;
                const float m_new = move ? mt : m_ref;
                const float a = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
                m_ref = m_new;
                l *= a;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[b][j] *= a;
                m_off = (m_ref == kNegInf) ? 0.0f : m_ref - kPScale;
                if constexpr (ALIBI)
                    m_off = fmaf(-ab * (float)(kb0 + 32 * u + 4 * half - pos), p.scale_log2, m_off);
                lh = 0.0f;
#pragma unroll
                for (int i = 4 * h; i < 4 * h + 4; ++i) pexp(i);
            }
            l += lh;
            lh = 0.0f;
        };
        if constexpr (MORE) {
#pragma unroll
            for (int ks = 0; ks < kAhead; ++ks) kread(ks);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the score products of unit u + 1 (a chain through sn) alternate
        // with the P.V products of unit u (independent accumulators) from the
        // fifth on, so that a score product never waits for the one before
        auto score = [&](int i) __attribute__((always_inline)) {
            if constexpr (MORE) {
                // the first step starts from a zero accumulator operand
                sn = mfma32<KV>(kf[i], qf[i], i == 0 ? f32x16_t{} : sn);
                if constexpr (ROPE) sn = mfma32<KV>(kf[i], qlo[i], sn);
                if (i + kAhead < 8) kread(i + kAhead);
            }
        };
        // The two waves of a SIMD contend for its issue slots.  A wave takes
        // a higher priority while it issues its matrix products and drops it
        // for its exponentials, so that a product ready to go is not held
        // behind the other wave's vector work (about 1 % on the 2,048 x
        // 131,072 prefill).
        auto prio = [&](auto v_c) __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(decltype(v_c)::value);
            __builtin_amdgcn_sched_barrier(0);
        };
        using Hi = std::integral_constant<int, 1>;
        using Lo = std::integral_constant<int, 0>;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            prio(Hi{});
            score(i);
            __builtin_amdgcn_sched_barrier(0);
            prio(Lo{});
            pexp(i);
            vread(0, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        check_half(0);
        pb[0] = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
        for (int i = 4; i < 8; ++i) {
            prio(Hi{});
            score(i);
            o[i - 4] = mfma32<KV_F16>(vf[0][i - 4], pb[0], o[i - 4]);
            __builtin_amdgcn_sched_barrier(0);
            prio(Lo{});
            pexp(i);
            vread(1, i - 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        check_half(1);
        pb[1] = make_uint4(w[4], w[5], w[6], w[7]);
        if constexpr (MORE) {
            alibi_bias(sn);
            if (masked(u + 1)) causal_mask(u + 1, sn);
        }
        prio(Hi{});
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            o[b] = mfma32<KV_F16>(vf[1][b], pb[1], o[b]);
            __builtin_amdgcn_sched_barrier(0);
        }
        prio(Lo{});
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    using B3 = std::integral_constant<int, 3>;
    using B4 = std::integral_constant<int, 4>;

    // ---- prologue: contents 0, 1 and 2 in LDS, the scores of unit 0.  All
    // three have landed before the loop, so that its first tile starts from
    // the same pending state as every later one (the compiler tracks the LDS
    // DMAs for the waits it adds to LDS reads, and a DMA of unknown age
    // there would cost a full wait).
    f32x16_t sa, sb;
    dma_content(0, B0{});
    dma_content(1, B1{});
    dma_content(2, B2{});
    dma_content(3, B3{});
    tile_wait<0>();
    tile_barrier();
    scores(0, sa, B0{});
    alibi_bias(sa);
    first_reference(sa, masked(0));

    // ---- iteration t folds tile t (units 2t, 2t + 1) from contents t and
    // t + 1 (buffers P = t % 5 and P + 1).
    auto iteration = [&](int t, auto ph_c, auto more_c) __attribute__((always_inline)) {
        constexpr int P = decltype(ph_c)::value;
        using BK = std::integral_constant<int, P>;
        using BN = std::integral_constant<int, (P + 1) % 5>;
        unit(2 * t, sa, sb, std::true_type{}, BK{}, BN{});
        unit(2 * t + 1, sb, sa, more_c, BN{}, BN{});
    };
    // Every tile but the last issues content t + 4 into the buffer of content
    // t - 1, free since the last barrier, and ends once content t + 2 has
    // landed: one barrier per tile.  The loop is unrolled by the five buffer
    // phases and holds one DMA per phase, with no branch around a DMA, so the
    // compiler tells the buffers apart and adds no wait of its own.
    auto step = [&](int t, auto ph_c) __attribute__((always_inline)) {
        constexpr int P = decltype(ph_c)::value;
        dma_content(t + 4, std::integral_constant<int, (P + 4) % 5>{});
        iteration(t, ph_c, std::true_type{});
        tile_wait<8>();
        tile_barrier();
    };
    int tl = 0;  // tiles folded so far
    for (; tl + 5 < n_tiles; tl += 5) {
        step(tl, B0{});
        step(tl + 1, B1{});
        step(tl + 2, B2{});
        step(tl + 3, B3{});
        step(tl + 4, B4{});
    }
    // the remaining 1 .. 5 tiles: all but the last as above, then the last
    const int rem = n_tiles - tl;
    if (rem > 1) step(tl, B0{});
    if (rem > 2) step(tl + 1, B1{});
    if (rem > 3) step(tl + 2, B2{});
    if (rem > 4) step(tl + 3, B3{});
    switch (rem) {
        case 1: iteration(tl, B0{}, std::false_type{}); break;
        case 2: iteration(tl + 1, B1{}, std::false_type{}); break;
        case 3: iteration(tl + 2, B2{}, std::false_type{}); break;
        case 4: iteration(tl + 3, B3{}, std::false_type{}); break;
        default: iteration(tl + 4, B4{}, std::false_type{}); break;
    }
    tile_wait<0>();  // no DMA may still be writing LDS when the wave ends

    // ---- combine the two halves of each row and write (or merge) out / lse
    __syncthreads();
    const bool any_bad = !ctx_ok || regen_bad;
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
    float4 prev[16];  // the earlier windows' output, all loads issued together
    if (p.carry) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            prev[i] = *reinterpret_cast<const float4 *>(dst + 32 * (i >> 2) + 8 * (i & 3) + 4 * half);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d0 = 32 * b + 8 * jj + 4 * half;
            float4 v = make_float4(o[b][4 * jj] * wb, o[b][4 * jj + 1] * wb,
                                   o[b][4 * jj + 2] * wb, o[b][4 * jj + 3] * wb);
            if (p.carry) {
                const float4 op = prev[4 * b + jj];
                v = make_float4(fmaf(op.x, wa, v.x), fmaf(op.y, wa, v.y), fmaf(op.z, wa, v.z),
                                fmaf(op.w, wa, v.w));
            }
            if (any_bad || lse_new != lse_new) v = make_float4(qnan, qnan, qnan, qnan);
            *reinterpret_cast<float4 *>(dst + d0) = v;
        }
    }
    if (half == 0) p.lse[orow0] = any_bad ? qnan : lse_new;
}

// Window preparation: every key of the window [key_begin, key_begin +
// window_tokens) of every (sequence, kv head) is written into the ring the
// prefill kernel reads, K in the kv type and V in f16: regenerated keys from
// the SplitMix64 regenerator (once per call; K rotated by its position under
// RoPE), other keys gathered through the page table (CFR-Atlas README: cold
// pages regenerated into scratch buffers that are reused, here one ring per
// window), keys past the context as zeros, and the keys of a page whose block
// id lies outside the pool as NaN, so the rows that see them fail loudly.
// One workgroup per (sequence, kv head, 64 keys); four lanes per key row, each
// moving 32 dims (64 contiguous bytes of K).  V is written per 64-key tile as
// V^T, 128 dim rows of 64 keys (128 bytes each), key k of the tile in slot
// 16 (k / 16) + s(k % 16), where s swaps bits 2 and 3 (keys 0-3, 8-11, 4-7,
// 12-15 of every 16): the order in which a lane of the prefill kernel holds
// its eight keys of a P.V step.  The tile is transposed through LDS and
// stored in 16-byte chunks.
__global__ __launch_bounds__(256) void window_prepare_kernel(const WindowParams r) {
    __shared__ uint16_t vt[kD * kTile];  // [dim][slot]
    constexpr int D = kD;
    const int groups = r.window_tokens / 64;
    const int gi = blockIdx.x % groups;
    const int rest = blockIdx.x / groups;
    const int g = rest % r.num_kv_heads;
    const int seq = rest / r.num_kv_heads;
    const int ctx = r.context_lens[seq];
    // sequences the prefill kernel turns into NaN rows need no ring rows
    if (ctx < 0 || ctx > r.max_context_len || ctx > r.max_keys) return;
    const int n_regen = r.regen_pages != nullptr ? r.regen_pages[seq] : 0;
    if (n_regen < 0 || n_regen > r.max_regen) return;
    const int P = r.page_tokens;
    const int64_t regen_keys = (int64_t)n_regen * P;
    const int row = threadIdx.x >> 2;      // key row within the 64
    const int d0 = 32 * (threadIdx.x & 3);  // first dim of this lane
    const int key = r.key_begin + 64 * gi + row;
    const int64_t at = (((int64_t)seq * r.num_kv_heads + g) * r.window_tokens + 64 * gi + row) * D + d0;
    uint32_t kw[16], vw[16];  // 32 dims of K and V as 16-bit pairs
    if (key >= ctx) {
#pragma unroll
        for (int i = 0; i < 16; ++i) kw[i] = vw[i] = 0u;
    } else if ((int64_t)key < regen_keys) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int dim = d0 + 2 * i;
            uint32_t k0 = regen_bf16_bits(r.seed, regen_counter(r.layer, g, key, dim, 0));
            uint32_t k1 = regen_bf16_bits(r.seed, regen_counter(r.layer, g, key, dim + 1, 0));
            if (r.pos.rope) {  // cached keys are rotated by their position
                float x0 = __uint_as_float(k0 << 16), x1 = __uint_as_float(k1 << 16);
                rope_rotate(x0, x1, key, rope_turns(dim / 2, D, r.pos.rope_log2_theta));
                k0 = __float_as_uint(bf16_round(x0)) >> 16;
                k1 = __float_as_uint(bf16_round(x1)) >> 16;
            }
            kw[i] = k0 | (k1 << 16);
            // f16 holds a regenerated value exactly (at most 8 significant
            // bits, within [-1, 1])
            const float v0 = regen_value(r.seed, regen_counter(r.layer, g, key, dim, 1));
            const float v1 = regen_value(r.seed, regen_counter(r.layer, g, key, dim + 1, 1));
            const f16x2_t vh = {(_Float16)v0, (_Float16)v1};
            vw[i] = __builtin_bit_cast(uint32_t, vh);
        }
    } else {
        const int lp = key / P;
        const int blk = r.page_table[(int64_t)seq * r.max_pages + lp];
        if (blk < 0 || blk >= r.num_blocks) {
            const uint32_t knan = r.kv_f16 ? 0x7E007E00u : 0x7FC07FC0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                kw[i] = knan;
                vw[i] = 0x7E007E00u;
            }
        } else {
            const int64_t src = (((int64_t)blk * r.num_kv_heads + g) * P + (key - lp * P)) * D + d0;
            const uint4 *ks = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(r.k_pool) + src);
            const uint4 *vs = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(r.v_pool) + src);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 a = ks[c], b = vs[c];
                kw[4 * c] = a.x; kw[4 * c + 1] = a.y; kw[4 * c + 2] = a.z; kw[4 * c + 3] = a.w;
                vw[4 * c] = b.x; vw[4 * c + 1] = b.y; vw[4 * c + 2] = b.z; vw[4 * c + 3] = b.w;
            }
            if (!r.kv_f16) {
#pragma unroll
                for (int i = 0; i < 16; ++i) vw[i] = bf16x2_to_f16x2(vw[i]);
            }
        }
    }
    uint4 *kd = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(r.ring_k) + at);
#pragma unroll
    for (int c = 0; c < 4; ++c)
        kd[c] = make_uint4(kw[4 * c], kw[4 * c + 1], kw[4 * c + 2], kw[4 * c + 3]);
    // V^T: this lane's 32 dims of key `row` into its slot of each dim row
    const int slot = (row & ~15) | (row & 3) | ((row & 4) << 1) | ((row & 8) >> 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        vt[(d0 + 2 * i) * kTile + slot] = (uint16_t)(vw[i] & 0xFFFFu);
        vt[(d0 + 2 * i + 1) * kTile + slot] = (uint16_t)(vw[i] >> 16);
    }
    __syncthreads();
    // the tile's 1,024 chunks of 16 bytes, four per lane, row-major
    const int64_t tile0 = (((int64_t)seq * r.num_kv_heads + g) * r.window_tokens + 64 * gi) * D;
    uint4 *vd = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(r.ring_v) + tile0);
    const uint4 *vs = reinterpret_cast<const uint4 *>(vt);
#pragma unroll
    for (int c = 0; c < 4; ++c) vd[threadIdx.x + 256 * c] = vs[threadIdx.x + 256 * c];
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

hipError_t launch_window_prepare(const WindowParams &r, hipStream_t stream) {
    const int64_t blocks = (int64_t)r.num_seqs * r.num_kv_heads * (r.window_tokens / 64);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(window_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, r);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams &p, int kv_type, int group, hipStream_t stream) {
    if (kv_type == KV_BF16) return by_policy<KV_BF16>(p, group, stream);
    if (kv_type == KV_F16) return by_policy<KV_F16>(p, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace atlas
