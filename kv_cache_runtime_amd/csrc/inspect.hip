// Page-walk, regeneration and decode kernels without attention arithmetic:
// the page gather (inspection), the page regenerator that writes bf16 values
// into pools or into the workspace copy used by chunked prefill, and the
// tier decoder (inspection).
#include "device.h"

namespace atlas {

namespace {

// One workgroup per (token, kv head) row: copy head_dim elements.
__global__ __launch_bounds__(128) void gather_kernel(const char *k_pool, const char *v_pool,
                                                     const int32_t *table_row, int32_t hkv,
                                                     int32_t d, int32_t P, int32_t num_blocks,
                                                     int32_t eb, int32_t num_tokens, char *k_out,
                                                     char *v_out) {
    const int64_t rowid = blockIdx.x;  // token * hkv + g
    const int tok = (int)(rowid / hkv);
    const int g = (int)(rowid % hkv);
    if (tok >= num_tokens) return;
    const int32_t blk = table_row[tok / P];
    const bool ok = blk >= 0 && blk < num_blocks;
    const int64_t src = (((int64_t)(ok ? blk : 0) * hkv + g) * P + tok % P) * d;
    const int64_t dst = rowid * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        if (eb == 4) {
            const uint32_t nanw = 0x7FC00000u;
            reinterpret_cast<uint32_t *>(k_out)[dst + i] =
                ok ? reinterpret_cast<const uint32_t *>(k_pool)[src + i] : nanw;
            reinterpret_cast<uint32_t *>(v_out)[dst + i] =
                ok ? reinterpret_cast<const uint32_t *>(v_pool)[src + i] : nanw;
        } else {
            const uint16_t nanh = 0x7FFFu;
            reinterpret_cast<uint16_t *>(k_out)[dst + i] =
                ok ? reinterpret_cast<const uint16_t *>(k_pool)[src + i] : nanh;
            reinterpret_cast<uint16_t *>(v_out)[dst + i] =
                ok ? reinterpret_cast<const uint16_t *>(v_pool)[src + i] : nanh;
        }
    }
}

// One workgroup per (page entry, kv head); each thread writes pairs of
// consecutive head_dim elements (one 32-bit bf16x2 or two f32 stores).
__global__ __launch_bounds__(256) void regen_fill_kernel(const RegenFillParams r) {
    const int i = blockIdx.x / r.num_kv_heads;
    const int g = blockIdx.x % r.num_kv_heads;
    if (i >= r.n) return;
    int lp, blk;
    if (r.regen_pages != nullptr) {
        // workspace copy: block i holds logical page i % pages_per_seq of
        // sequence i / pages_per_seq, if that page is regenerated
        const int seq = i / r.pages_per_seq;
        lp = i % r.pages_per_seq;
        if (lp >= r.regen_pages[seq]) return;
        blk = i;
    } else {
        lp = r.logical_pages[i];
        blk = r.dst_blocks[i];
        if (lp < 0 || blk < 0 || blk >= r.num_blocks) return;
    }
    const int P = r.page_tokens, D = r.head_dim;
    const int64_t base = (((int64_t)blk * r.num_kv_heads + g) * P) * D;
    const int pairs = P * D / 2;
    for (int t = threadIdx.x; t < pairs; t += blockDim.x) {
        const int e = 2 * t;
        const int row = e / D, dim = e % D;
        const int tok = lp * P + row;
        uint32_t k0 = regen_bf16_bits(r.seed, regen_counter(r.layer, g, tok, dim, 0));
        uint32_t k1 = regen_bf16_bits(r.seed, regen_counter(r.layer, g, tok, dim + 1, 0));
        uint32_t v0 = regen_bf16_bits(r.seed, regen_counter(r.layer, g, tok, dim, 1));
        uint32_t v1 = regen_bf16_bits(r.seed, regen_counter(r.layer, g, tok, dim + 1, 1));
        if (r.kv_f32) {
            float2 kk = make_float2(__uint_as_float(k0 << 16), __uint_as_float(k1 << 16));
            float2 vv = make_float2(__uint_as_float(v0 << 16), __uint_as_float(v1 << 16));
            reinterpret_cast<float2 *>(reinterpret_cast<float *>(r.k_dst) + base)[t] = kk;
            reinterpret_cast<float2 *>(reinterpret_cast<float *>(r.v_dst) + base)[t] = vv;
        } else {
            reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(r.k_dst) + base)[t] =
                k0 | (k1 << 16);
            reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(r.v_dst) + base)[t] =
                v0 | (v1 << 16);
        }
    }
}

// One workgroup per (entry, kv head): f32 values of every element of the page.
__global__ __launch_bounds__(256) void dequant_kernel(const DecodeParams p, int kv_type, int D,
                                                      const int32_t *entries, int32_t n,
                                                      float *k_out, float *v_out) {
    const int i = blockIdx.x / p.num_kv_heads;
    const int g = blockIdx.x % p.num_kv_heads;
    if (i >= n) return;
    const uint32_t e = (uint32_t)entries[i];
    const uint32_t tier = e >> 30, slot = e & ((1u << 30) - 1u);
    const int P = p.page_tokens;
    const int64_t dst = (((int64_t)i * p.num_kv_heads + g) * P) * D;
    const int64_t src_row = ((int64_t)slot * p.num_kv_heads + g) * P;
    const float qnan = __builtin_nanf("");
    for (int t = threadIdx.x; t < P * D; t += blockDim.x) {
        float kv = qnan, vv = qnan;
        if (tier == 0 && slot < (uint32_t)p.num_blocks) {
            kv = load_elem(p.k_pool, src_row * D + t, kv_type);
            vv = load_elem(p.v_pool, src_row * D + t, kv_type);
        } else if (tier == 1 && slot < (uint32_t)p.n_i8) {
            const float ks = p.i8_ks[(int64_t)slot * p.num_kv_heads + g];
            const float vs = p.i8_vs[(int64_t)slot * p.num_kv_heads + g];
            kv = (float)p.i8_k[src_row * D + t] * ks;
            vv = (float)p.i8_v[src_row * D + t] * vs;
        } else if (tier == 2 && slot < (uint32_t)p.n_i4) {
            const float ks = p.i4_ks[(int64_t)slot * p.num_kv_heads + g];
            const float vs = p.i4_vs[(int64_t)slot * p.num_kv_heads + g];
            const uint32_t bk = p.i4_k[src_row * (D / 2) + t / 2];
            const uint32_t bv = p.i4_v[src_row * (D / 2) + t / 2];
            const int sh = (t & 1) ? 24 : 28;  // high nibble for odd elements
            kv = (float)sext_field(bk, sh, 4) * ks;
            vv = (float)sext_field(bv, sh, 4) * vs;
        }
        k_out[dst + t] = kv;
        v_out[dst + t] = vv;
    }
}

}  // namespace

hipError_t launch_gather(const void *k_pool, const void *v_pool, const int32_t *table_row,
                         int32_t num_kv_heads, int32_t head_dim, int32_t page_tokens,
                         int32_t num_blocks, int32_t elem_bytes, int32_t num_tokens, void *k_out,
                         void *v_out, hipStream_t stream) {
    const int64_t rows = (int64_t)num_tokens * num_kv_heads;
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)rows), dim3(128), 0, stream,
                       (const char *)k_pool, (const char *)v_pool, table_row, num_kv_heads,
                       head_dim, page_tokens, num_blocks, elem_bytes, num_tokens, (char *)k_out,
                       (char *)v_out);
    return hipGetLastError();
}

hipError_t launch_regen_fill(const RegenFillParams &r, hipStream_t stream) {
    const int64_t blocks = (int64_t)r.n * r.num_kv_heads;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(regen_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, r);
    return hipGetLastError();
}

hipError_t launch_dequant(const DecodeParams &p, int kv_type, int head_dim,
                          const int32_t *entries, int32_t n, float *k_out, float *v_out,
                          hipStream_t stream) {
    const int64_t blocks = (int64_t)n * p.num_kv_heads;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, kv_type,
                       head_dim, entries, n, k_out, v_out);
    return hipGetLastError();
}

}  // namespace atlas
