/*
 * Plain f64 CPU oracle for exact causal scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the attention library links, calls or
 * includes this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code with the GPU path.
 *
 * What it computes (RustAttention README, "Mathematical Framework Covered"):
 *   Attention(Q, K, V) = softmax(Q K^T * scale + Mask) V
 * with the causal mask of the same README ("GPT-Style Causal Masking": keys
 * after the query position get weight exactly zero) and the max subtraction
 * of its "Numerically Stable Softmax" bullet.  Everything is accumulated in
 * double precision, over the whole (unpaged) key range of one head.
 *
 * The folded variant walks the same keys page by page with an online softmax
 * (running max, running sum, running accumulator rescaled per page), which is
 * the computation the CFR-Atlas README describes as "exact folded
 * online-softmax attention" and ARGUS describes as "page-by-page online
 * softmax (Milakov & Gimelshein 2018)" in its "Latency & Throughput Impact"
 * section.  It is used only to check the folded == full-KV contract of the
 * CFR-Atlas README ("Its core contract is ...").
 *
 * The regenerator is SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): the n-th output of a stream
 * seeded with `seed` is mix64(seed + n * 0x9E3779B97F4A7C15).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Keys [0, visible[r]) are visible to row r; the rest are masked out.
 *
 * slope (NULL, or [n_rows]): ALiBi (Press, Smith, Lewis, "Train Short, Test
 * Long", ICLR 2022), the positional policy the CFR-Atlas README lists beside
 * RoPE: score j of row r gains -slope[r] * (pos_r - j), where pos_r =
 * visible[r] - 1 is the row's own position, so a key i tokens back is
 * penalised linearly in i. */
void oracle_attend(int64_t n_rows, int64_t d, int64_t n_keys,
                   const double *q,      /* [n_rows][d] */
                   const double *k,      /* [n_keys][d] */
                   const double *v,      /* [n_keys][d] */
                   const int64_t *visible, /* [n_rows] */
                   double scale,
                   const double *slope,  /* [n_rows] or NULL */
                   double *out,          /* [n_rows][d] */
                   double *lse)          /* [n_rows] */
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t n = visible[r];
        if (n > n_keys) n = n_keys;
        double *o = out + r * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        if (n <= 0) {
            lse[r] = -INFINITY;
            continue;
        }
        const double *qr = q + r * d;
        const double sl = slope ? slope[r] : 0.0;
        const int64_t pos = visible[r] - 1;
        /* m = max_j s_j with s_j = scale * q . k_j - slope * (pos - j)
         * (scores are recomputed below rather than stored, so the memory
         * stays O(d) per row) */
        double m = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            const double *kj = k + j * d;
            for (int64_t c = 0; c < d; ++c) acc += qr[c] * kj[c];
            acc = acc * scale - sl * (double)(pos - j);
            if (acc > m) m = acc;
        }
        /* weights w_j = exp(s_j - m), their sum Z, and sum_j w_j v_j */
        double z = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            const double *kj = k + j * d;
            for (int64_t c = 0; c < d; ++c) acc += qr[c] * kj[c];
            double w = exp(acc * scale - sl * (double)(pos - j) - m);
            z += w;
            const double *vj = v + j * d;
            for (int64_t c = 0; c < d; ++c) o[c] += w * vj[c];
        }
        for (int64_t c = 0; c < d; ++c) o[c] /= z;
        lse[r] = m + log(z);
    }
}

/* Same rows, folded page by page with an online softmax. */
void oracle_attend_folded(int64_t n_rows, int64_t d, int64_t n_keys,
                          const double *q, const double *k, const double *v,
                          const int64_t *visible, double scale,
                          int64_t page_tokens, double *out, double *lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t n = visible[r];
        if (n > n_keys) n = n_keys;
        double *o = out + r * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        const double *qr = q + r * d;
        double m = -INFINITY, l = 0.0;
        for (int64_t p0 = 0; p0 < n; p0 += page_tokens) {
            int64_t p1 = p0 + page_tokens < n ? p0 + page_tokens : n;
            double pm = -INFINITY;
            for (int64_t j = p0; j < p1; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c) acc += qr[c] * k[j * d + c];
                acc *= scale;
                if (acc > pm) pm = acc;
            }
            double m_new = pm > m ? pm : m;
            double alpha = exp(m - m_new); /* exp(-inf) = 0 on the first page */
            l *= alpha;
            for (int64_t c = 0; c < d; ++c) o[c] *= alpha;
            for (int64_t j = p0; j < p1; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c) acc += qr[c] * k[j * d + c];
                double w = exp(acc * scale - m_new);
                l += w;
                for (int64_t c = 0; c < d; ++c) o[c] += w * v[j * d + c];
            }
            m = m_new;
        }
        if (n <= 0) {
            lse[r] = -INFINITY;
            continue;
        }
        for (int64_t c = 0; c < d; ++c) o[c] /= l;
        lse[r] = m + log(l);
    }
}

/* ---- SplitMix64 and the page regenerator's value definition ------------- */

static const uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ull;

static uint64_t sm64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* The n-th output (n >= 1) of SplitMix64 seeded with `seed`. */
uint64_t oracle_splitmix64(uint64_t seed, uint64_t n)
{
    return sm64_mix(seed + n * SM64_GAMMA);
}

/* Round an f32 to bf16 (nearest, ties to even) and widen it back to f32.
 * Inputs here are finite. */
static float round_to_bf16(float x)
{
    uint32_t b;
    memcpy(&b, &x, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;
    float y;
    memcpy(&y, &b, 4);
    return y;
}

/*
 * Regenerated K (kv = 0) or V (kv = 1) value of (layer, kv_head, token, dim):
 *   c = layer<<48 | kv_head<<40 | token<<9 | dim<<1 | kv
 *   z = the (c+1)-th SplitMix64 output for `seed`
 *   x = 2 * (z>>40) * 2^-24 - 1   (uniform on [-1, 1), exact in f32)
 *   value = bf16(x), round to nearest even.
 * Writes [n_tokens][d] values for tokens token0 .. token0+n_tokens-1 as f32.
 */
void oracle_regen_values(uint64_t seed, uint64_t layer, uint64_t kv_head,
                         int64_t token0, int64_t n_tokens, int64_t d,
                         int64_t kv, float *dst)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int64_t c = 0; c < d; ++c) {
            uint64_t ctr = (layer << 48) | (kv_head << 40) |
                           ((uint64_t)(token0 + t) << 9) | ((uint64_t)c << 1) |
                           (uint64_t)kv;
            uint64_t z = oracle_splitmix64(seed, ctr + 1);
            int64_t u24 = (int64_t)(z >> 40);
            float x = (float)(u24 - (1 << 23)) * (1.0f / 8388608.0f);
            dst[t * d + c] = round_to_bf16(x);
        }
    }
}
