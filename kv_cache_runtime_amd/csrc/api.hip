// C ABI of libatlas.so: host-side argument checks, split planning, workspace
// layout and kernel dispatch.  No device memory is read or allocated here;
// every check runs before the first launch, so an error leaves all outputs
// untouched (CFR-Atlas README, test list: rejection of invalid configs and
// ranges, transactional behaviour).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "atlas.h"
#include "internal.h"

using namespace atlas;

// Device scratch of atlas_paged_attention_noalloc: a file-scope device array,
// one copy per GPU.  Host code never uses the name as an address; it keeps
// the address hipGetSymbolAddress reports for each device.
static __device__ __align__(256) char scratch[ATLAS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // per device, set on its first call

atlas_status fail(atlas_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

atlas_status ok() {
    g_last_error.clear();
    return ATLAS_OK;
}

atlas_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(ATLAS_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Everything a call needs that follows from the host-side arguments.
struct Plan {
    int group = 1;
    int split_tokens = 0;
    int max_splits = 1;
    bool direct = true;      // one split per row: the decode kernel writes out/lse
    bool mfma = false;       // chunked prefill on matrix cores
    int q_blocks = 0;        // query tiles per sequence (matrix-core prefill)
    size_t part_o_bytes = 0;
    size_t part_lse_bytes = 0;
    int window_tokens = 0;   // matrix-core prefill: keys per window
    int windows = 1;
    size_t ring_bytes = 0;   // the K ring (and the V ring) of one window's keys
    size_t total = 0;
};

int env_split_tokens() {
    const char *s = std::getenv("ATLAS_SPLIT_TOKENS");
    if (!s || !*s) return 0;
    return std::atoi(s);
}

// Tokens per split-K work item.  Fixed in tokens (never derived from the page
// size or placement) so the arithmetic order, hence the result bits, depend
// only on the logical problem.  The largest power of two in [256, 4096] that
// still yields about 4 workgroups per compute unit when every row has the
// largest context (longer splits amortise each workgroup's setup and shrink
// the merge; measured on the decode workloads, 2048-4096 is best whenever the
// grid stays that full).
int choose_split_tokens(const atlas_attn_args *a) {
    int t = a->split_tokens > 0 ? a->split_tokens : env_split_tokens();
    if (t > 0) return t;
    const int64_t rows = (int64_t)a->total_q * a->num_kv_heads;
    const int64_t want = 1024;
    for (int cand = 4096; cand >= 256; cand >>= 1) {
        const int64_t items = rows * ((a->max_context_len + cand - 1) / cand);
        if (items >= want) return cand;
    }
    return 256;
}

bool dtype_ok(int32_t d) { return d == ATLAS_F32 || d == ATLAS_BF16 || d == ATLAS_F16; }

// sizing: atlas_workspace_size, which serves plain and tiered calls alike,
// so the hot-pool checks that only a plain call needs are left to the call.
atlas_status check_common(const atlas_attn_args *a, bool tiered, const atlas_regen_spec *rg,
                          Plan *plan, bool sizing = false) {
    if (!a) return fail(ATLAS_EINVAL, "args is NULL");
    if (a->struct_size != sizeof(atlas_attn_args))
        return fail(ATLAS_EINVAL, "args->struct_size %u != %zu", a->struct_size,
                    sizeof(atlas_attn_args));
    if (!dtype_ok(a->q_dtype) || !dtype_ok(a->kv_dtype))
        return fail(ATLAS_EINVAL, "unknown dtype (q %d, kv %d)", a->q_dtype, a->kv_dtype);
    if (a->num_seqs < 1) return fail(ATLAS_EINVAL, "num_seqs %d < 1", a->num_seqs);
    if (a->num_heads < 1 || a->num_kv_heads < 1)
        return fail(ATLAS_EINVAL, "num_heads %d / num_kv_heads %d must be >= 1", a->num_heads,
                    a->num_kv_heads);
    if (a->num_heads % a->num_kv_heads)
        return fail(ATLAS_EINVAL, "num_heads %d is not a multiple of num_kv_heads %d",
                    a->num_heads, a->num_kv_heads);
    const int group = a->num_heads / a->num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(ATLAS_EUNSUPPORTED, "heads per kv head %d not in {1, 2, 4, 8}", group);
    if (a->head_dim < 1) return fail(ATLAS_EINVAL, "head_dim %d < 1", a->head_dim);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(ATLAS_EUNSUPPORTED, "head_dim %d not in {64, 128}", a->head_dim);
    if (a->page_tokens < 1) return fail(ATLAS_EINVAL, "page_tokens %d < 1", a->page_tokens);
    if (a->page_tokens % 16)
        return fail(ATLAS_EUNSUPPORTED, "page_tokens %d is not a multiple of 16", a->page_tokens);
    if (a->max_pages_per_seq < 1)
        return fail(ATLAS_EINVAL, "max_pages_per_seq %d < 1", a->max_pages_per_seq);
    if (a->num_blocks < (tiered || sizing ? 0 : 1))
        return fail(ATLAS_EINVAL, "num_blocks %d out of range", a->num_blocks);
    const int64_t max_keys = (int64_t)a->max_pages_per_seq * a->page_tokens;
    if (max_keys > INT32_MAX)
        return fail(ATLAS_EINVAL, "max_pages_per_seq * page_tokens overflows int32");
    if (a->max_context_len < 0 || a->max_context_len > max_keys)
        return fail(ATLAS_EINVAL, "max_context_len %d outside [0, %lld]", a->max_context_len,
                    (long long)max_keys);
    if (a->query_start == nullptr) {
        if (a->total_q != a->num_seqs)
            return fail(ATLAS_EINVAL, "decode needs total_q (%d) == num_seqs (%d)", a->total_q,
                        a->num_seqs);
    } else {
        if (a->total_q < 1) return fail(ATLAS_EINVAL, "total_q %d < 1", a->total_q);
        if (a->max_query_len < 1 || a->max_query_len > a->total_q ||
            a->max_query_len > a->max_context_len)
            return fail(ATLAS_EINVAL, "max_query_len %d outside [1, min(total_q, max_context_len)]",
                        a->max_query_len);
    }
    if (!std::isfinite(a->scale)) return fail(ATLAS_EINVAL, "scale is not finite");
    if (!std::isfinite(a->rope_theta) || (a->rope_theta != 0.0f && !(a->rope_theta > 1.0f)))
        return fail(ATLAS_EINVAL, "rope_theta must be 0 or a finite value > 1");
    if (a->reserved != 0) return fail(ATLAS_EINVAL, "reserved field must be 0");
    if (a->split_tokens < 0 || (a->split_tokens > 0 && a->split_tokens % 64))
        return fail(ATLAS_EINVAL, "split_tokens %d must be 0 or a positive multiple of 64",
                    a->split_tokens);
    if (!a->q || !a->page_table || !a->context_lens || !a->out || !a->lse)
        return fail(ATLAS_EINVAL, "NULL q, page_table, context_lens, out or lse");
    if (!tiered && !sizing && (!a->k_pool || !a->v_pool))
        return fail(ATLAS_EINVAL, "NULL k_pool or v_pool");
    if (tiered && a->num_blocks > 0 && (!a->k_pool || !a->v_pool))
        return fail(ATLAS_EINVAL, "NULL hot k_pool or v_pool with num_blocks > 0");
    if ((int64_t)a->total_q * a->num_heads * a->head_dim > ((int64_t)1 << 40))
        return fail(ATLAS_EINVAL, "output too large");

    plan->group = group;
    const bool prefill = a->query_start != nullptr;
    const bool sixteen = a->kv_dtype == ATLAS_BF16 || a->kv_dtype == ATLAS_F16;
    plan->mfma = prefill && !tiered && sixteen && a->q_dtype == a->kv_dtype &&
                 a->head_dim == 128 && std::getenv("ATLAS_NO_MFMA") == nullptr;

    if (!plan->mfma) {
        int st = choose_split_tokens(a);
        if (st < 64 || st % 64)
            return fail(ATLAS_EINVAL, "split tokens %d must be a positive multiple of 64", st);
        plan->split_tokens = st;
        plan->max_splits = a->max_context_len > 0 ? (a->max_context_len + st - 1) / st : 1;
        if (plan->max_splits < 1) plan->max_splits = 1;
        plan->direct = plan->max_splits == 1;
        const int64_t blocks = (int64_t)a->total_q * a->num_kv_heads * plan->max_splits;
        if (blocks > INT32_MAX)
            return fail(ATLAS_EUNSUPPORTED, "too many split-K work items (%lld)",
                        (long long)blocks);
        if (!plan->direct) {
            const int64_t parts = (int64_t)a->total_q * a->num_heads * plan->max_splits;
            plan->part_o_bytes = align_up((size_t)parts * a->head_dim * sizeof(float));
            plan->part_lse_bytes = align_up((size_t)parts * sizeof(float));
        }
    }

    if (rg) {
        if (rg->struct_size != sizeof(atlas_regen_spec))
            return fail(ATLAS_EINVAL, "regen->struct_size %u != %zu", rg->struct_size,
                        sizeof(atlas_regen_spec));
        if (a->kv_dtype != ATLAS_BF16)
            return fail(ATLAS_EUNSUPPORTED, "regenerated pages need kv_dtype BF16");
        if (rg->layer >= (1u << 16)) return fail(ATLAS_EINVAL, "layer %u >= 2^16", rg->layer);
        if (a->num_kv_heads > 256) return fail(ATLAS_EINVAL, "num_kv_heads > 256 with regen");
        if (!rg->regen_pages) return fail(ATLAS_EINVAL, "NULL regen_pages");
        if (rg->max_regen_pages < 0 || rg->max_regen_pages > a->max_pages_per_seq)
            return fail(ATLAS_EINVAL, "max_regen_pages %d outside [0, max_pages_per_seq]",
                        rg->max_regen_pages);
    }
    if (plan->mfma) {
        const int pos_per_block = kPrefillRows / group;
        plan->q_blocks = (a->max_query_len + pos_per_block - 1) / pos_per_block;
        const int64_t blocks = (int64_t)a->num_kv_heads * plan->q_blocks * a->num_seqs;
        if (blocks > INT32_MAX)
            return fail(ATLAS_EUNSUPPORTED, "too many prefill workgroups (%lld)", (long long)blocks);
        // The keys are taken in windows fixed in tokens, each gathered (or
        // regenerated) into one ring that every window reuses, so the scratch
        // does not grow with the context and the result bits do not depend
        // on the page size or on which pages are regenerated.
        int w = a->split_tokens > 0 ? a->split_tokens : kPrefillWindow;
        if (w > kPrefillMaxWindow) w = kPrefillMaxWindow;
        const int ctx64 = (a->max_context_len + 63) / 64 * 64;
        if (ctx64 > 0 && w > ctx64) w = ctx64;  // one window holds the whole context
        plan->window_tokens = w;
        plan->windows = a->max_context_len > 0 ? (a->max_context_len + w - 1) / w : 1;
        plan->ring_bytes = align_up((size_t)a->num_seqs * a->num_kv_heads * w * a->head_dim * 2);
    }
    plan->total = plan->part_o_bytes + plan->part_lse_bytes + 2 * plan->ring_bytes;
    return ok();
}

atlas_status check_workspace(const atlas_attn_args *a, const Plan &plan) {
    if (plan.total == 0) return ok();
    if (!a->workspace) return fail(ATLAS_EWORKSPACE, "workspace is NULL, %zu bytes needed",
                                   plan.total);
    if (a->workspace_bytes < plan.total)
        return fail(ATLAS_EWORKSPACE, "workspace %zu bytes < %zu needed", a->workspace_bytes,
                    plan.total);
    if (reinterpret_cast<uintptr_t>(a->workspace) % kAlign)
        return fail(ATLAS_EINVAL, "workspace must be %zu-byte aligned", kAlign);
    return ok();
}

PosParams pos_params(float rope_theta, const float *alibi) {
    PosParams q;
    std::memset(&q, 0, sizeof(q));
    q.alibi = alibi;
    q.rope = rope_theta > 0.0f ? 1 : 0;
    q.rope_log2_theta = q.rope ? std::log2((double)rope_theta) : 0.0;
    return q;
}

// Sizes and pointers of the cold-tier pools (a pool with slots needs all four
// of its pointers).
atlas_status check_pools(const atlas_tier_pools *t) {
    if (!t) return fail(ATLAS_EINVAL, "pools is NULL");
    if (t->struct_size != sizeof(atlas_tier_pools))
        return fail(ATLAS_EINVAL, "pools->struct_size %u != %zu", t->struct_size,
                    sizeof(atlas_tier_pools));
    if (t->num_int8 < 0 || t->num_int4 < 0 || t->num_fp8 < 0 || t->num_int2 < 0)
        return fail(ATLAS_EINVAL, "negative tier pool size");
    if (t->num_fp8 > (1 << 28) || t->num_int2 > (1 << 28))
        return fail(ATLAS_EINVAL, "FP8 / INT2 pools hold at most 2^28 slots");
    if (t->reserved != 0 || t->reserved2 != 0 || t->reserved3 != 0)
        return fail(ATLAS_EINVAL, "reserved field must be 0");
    if (t->num_int8 > 0 && (!t->int8_k || !t->int8_v || !t->int8_k_scale || !t->int8_v_scale))
        return fail(ATLAS_EINVAL, "NULL int8 pool pointer");
    if (t->num_int4 > 0 && (!t->int4_k || !t->int4_v || !t->int4_k_scale || !t->int4_v_scale))
        return fail(ATLAS_EINVAL, "NULL int4 pool pointer");
    if (t->num_fp8 > 0 && (!t->fp8_k || !t->fp8_v || !t->fp8_k_scale || !t->fp8_v_scale))
        return fail(ATLAS_EINVAL, "NULL fp8 pool pointer");
    if (t->num_int2 > 0 && (!t->int2_k || !t->int2_v || !t->int2_k_scale || !t->int2_v_scale))
        return fail(ATLAS_EINVAL, "NULL int2 pool pointer");
    if (t->num_1bit < 0 || t->num_1bit > (1 << 28))
        return fail(ATLAS_EINVAL, "1-bit pool size %d outside [0, 2^28]", t->num_1bit);
    if (t->outliers_1bit < 0 || t->outliers_1bit > ATLAS_1BIT_MAX_OUTLIERS)
        return fail(ATLAS_EINVAL, "outliers_1bit %d outside [0, %d]", t->outliers_1bit,
                    ATLAS_1BIT_MAX_OUTLIERS);
    if (t->num_1bit > 0 && (!t->bit_k || !t->bit_v || !t->bit_k_scale || !t->bit_v_scale ||
                            (t->outliers_1bit > 0 && (!t->bit_k_out || !t->bit_v_out))))
        return fail(ATLAS_EINVAL, "NULL 1-bit pool pointer");
    return ok();
}

// 1-bit blocks index their elements with 16 bits.
atlas_status check_1bit_block(const atlas_attn_args *a, const atlas_tier_pools *t) {
    if (t->num_1bit > 0 && (int64_t)a->page_tokens * a->head_dim > 65536)
        return fail(ATLAS_EUNSUPPORTED, "1-bit pages need page_tokens * head_dim <= 65536");
    return ok();
}

template <typename P>
void set_pools(P &p, const atlas_tier_pools *t) {
    p.i8_k = t->int8_k;
    p.i8_v = t->int8_v;
    p.i8_ks = t->int8_k_scale;
    p.i8_vs = t->int8_v_scale;
    p.i4_k = t->int4_k;
    p.i4_v = t->int4_v;
    p.i4_ks = t->int4_k_scale;
    p.i4_vs = t->int4_v_scale;
    p.f8_k = t->fp8_k;
    p.f8_v = t->fp8_v;
    p.f8_ks = t->fp8_k_scale;
    p.f8_vs = t->fp8_v_scale;
    p.i2_k = t->int2_k;
    p.i2_v = t->int2_v;
    p.i2_ks = t->int2_k_scale;
    p.i2_vs = t->int2_v_scale;
    p.n_i8 = t->num_int8;
    p.n_i4 = t->num_int4;
    p.n_f8 = t->num_fp8;
    p.n_i2 = t->num_int2;
}

void set_1bit(DecodeParams &p, const atlas_tier_pools *t) {
    p.b1_k = t->bit_k;
    p.b1_v = t->bit_v;
    p.b1_ks = t->bit_k_scale;
    p.b1_vs = t->bit_v_scale;
    p.b1_ko = t->bit_k_out;
    p.b1_vo = t->bit_v_out;
    p.n_b1 = t->num_1bit;
    p.b1_nout = t->outliers_1bit;
}

RowMap row_map(const atlas_attn_args *a) {
    RowMap m;
    m.context_lens = a->context_lens;
    m.query_start = a->query_start;
    m.num_seqs = a->num_seqs;
    m.max_context_len = a->max_context_len;
    m.max_keys = a->max_pages_per_seq * a->page_tokens;
    return m;
}

// Division by page_tokens as a multiply-high: x / P == (umulhi(x, magic) +
// x) >> shift for every x < 2^31 (round-up reciprocal with a 2^shift >= P
// pre-scale; the sum stays below 2^32 because magic < 2^32 and x < 2^31).
void page_divider(int32_t page_tokens, uint32_t &magic, uint32_t &shift) {
    uint32_t sh = 0;
    while ((1u << sh) < (uint32_t)page_tokens) ++sh;
    shift = sh;
    magic = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << sh) - page_tokens)) / page_tokens + 1);
}

DecodeParams decode_params(const atlas_attn_args *a, const Plan &plan) {
    DecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.rows = row_map(a);
    p.pos = pos_params(a->rope_theta, a->alibi_slopes);
    p.q = a->q;
    p.q_dtype = a->q_dtype;
    p.k_pool = a->k_pool;
    p.v_pool = a->v_pool;
    p.page_table = a->page_table;
    p.num_heads = a->num_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.page_tokens = a->page_tokens;
    p.max_pages = a->max_pages_per_seq;
    p.num_blocks = a->num_blocks;
    p.total_q = a->total_q;
    p.split_tokens = plan.split_tokens;
    p.max_splits = plan.max_splits;
    page_divider(a->page_tokens, p.p_magic, p.p_shift);
    p.scale_log2 = a->scale * 1.4426950408889634f;
    char *ws = reinterpret_cast<char *>(a->workspace);
    // (callers that launch nothing, such as the validator, may pass no
    // workspace: no pointer is formed from a null base)
    p.part_o = plan.direct || !ws ? nullptr : reinterpret_cast<float *>(ws);
    p.part_lse = plan.direct || !ws ? nullptr : reinterpret_cast<float *>(ws + plan.part_o_bytes);
    p.out = a->out;
    p.lse = a->lse;
    p.direct = plan.direct ? 1 : 0;
    return p;
}

// Optional caller events around the main kernel (profiling hook).
hipError_t mark(const atlas_attn_args *a, int which, hipStream_t stream) {
    if (!a->profile_events[which]) return hipSuccess;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(a->profile_events[which]), stream);
}

atlas_status run_decode(const atlas_attn_args *a, const Plan &plan, DecodeParams &p, int mode) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(a->stream);
    hipError_t e = mark(a, 0, stream);
    if (e != hipSuccess) return device_status(e, "profile event record");
    if (decode_mfma_supported(a->kv_dtype, a->head_dim, plan.group, mode, a->page_tokens,
                              plan.split_tokens) &&
        std::getenv("ATLAS_DECODE_VALU") == nullptr)
        e = launch_decode_mfma(p, a->kv_dtype, plan.group, mode, stream);
    else
        e = launch_decode(p, a->kv_dtype, a->head_dim, plan.group, mode, stream);
    if (e != hipSuccess) return device_status(e, "decode launch");
    e = mark(a, 1, stream);
    if (e != hipSuccess) return device_status(e, "profile event record");
    if (!plan.direct) {
        FoldParams f;
        std::memset(&f, 0, sizeof(f));
        f.part_o = p.part_o;
        f.part_lse = p.part_lse;
        f.out = a->out;
        f.lse = a->lse;
        f.o_row_stride = (int64_t)plan.max_splits * a->head_dim;
        f.o_split_stride = a->head_dim;
        f.l_row_stride = plan.max_splits;
        f.l_split_stride = 1;
        f.rows = a->total_q * a->num_heads;
        f.head_dim = a->head_dim;
        f.fixed_splits = 0;
        f.map = p.rows;
        f.num_heads = a->num_heads;
        f.split_tokens = plan.split_tokens;
        e = launch_fold(f, stream);
        if (e != hipSuccess) return device_status(e, "fold launch");
    }
    return ok();
}

// Chunked prefill on the matrix cores, window by window: the window's keys
// are gathered (or regenerated) into the ring, then the prefill kernel folds
// the window and merges it into out / lse.
atlas_status run_prefill(const atlas_attn_args *a, const Plan &plan, const atlas_regen_spec *rg) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(a->stream);
    char *ws = reinterpret_cast<char *>(a->workspace);
    PrefillParams p;
    std::memset(&p, 0, sizeof(p));
    p.rows = row_map(a);
    p.pos = pos_params(a->rope_theta, a->alibi_slopes);
    p.q = a->q;
    p.ring_k = ws;
    p.ring_v = ws + plan.ring_bytes;
    p.ring_tokens = plan.window_tokens;
    p.regen_pages = rg ? rg->regen_pages : nullptr;
    p.max_regen = rg ? rg->max_regen_pages : 0;
    p.num_heads = a->num_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.total_q = a->total_q;
    p.max_query_len = a->max_query_len;
    p.q_blocks = plan.q_blocks;
    p.scale_log2 = a->scale * 1.4426950408889634f;
    p.out = a->out;
    p.lse = a->lse;
    WindowParams r;
    std::memset(&r, 0, sizeof(r));
    r.pos = p.pos;
    r.seed = rg ? rg->seed : 0;
    r.layer = rg ? rg->layer : 0;
    r.num_seqs = a->num_seqs;
    r.num_kv_heads = a->num_kv_heads;
    r.page_tokens = a->page_tokens;
    r.max_pages = a->max_pages_per_seq;
    r.num_blocks = a->num_blocks;
    r.k_pool = a->k_pool;
    r.v_pool = a->v_pool;
    r.page_table = a->page_table;
    r.kv_f16 = a->kv_dtype == ATLAS_F16 ? 1 : 0;
    r.regen_pages = p.regen_pages;
    r.max_regen = p.max_regen;
    r.context_lens = a->context_lens;
    r.max_context_len = a->max_context_len;
    r.max_keys = a->max_pages_per_seq * a->page_tokens;
    r.window_tokens = plan.window_tokens;
    r.ring_k = ws;
    r.ring_v = ws + plan.ring_bytes;
    hipError_t e = mark(a, 0, stream);
    if (e != hipSuccess) return device_status(e, "profile event record");
    for (int w = 0; w < plan.windows; ++w) {
        const int64_t k0 = (int64_t)w * plan.window_tokens;
        r.key_begin = (int32_t)k0;
        e = launch_window_prepare(r, stream);
        if (e != hipSuccess) return device_status(e, "window preparation launch");
        p.key_begin = (int32_t)k0;
        p.key_end = (int32_t)std::min<int64_t>(k0 + plan.window_tokens, INT32_MAX);
        p.carry = w > 0 ? 1 : 0;
        e = launch_prefill(p, a->kv_dtype, plan.group, stream);
        if (e != hipSuccess) return device_status(e, "prefill launch");
    }
    e = mark(a, 1, stream);
    if (e != hipSuccess) return device_status(e, "profile event record");
    return ok();
}

}  // namespace

namespace atlas {
// Error reporting for the library's other host sources (the same
// thread-local message atlas_last_error returns).
int32_t report_error(int32_t st, const char *msg) {
    g_last_error = msg;
    return st;
}
int32_t report_ok() { return ok(); }
}  // namespace atlas

extern "C" {

uint32_t atlas_abi_version(void) { return ATLAS_ABI_VERSION; }

const char *atlas_status_string(atlas_status s) {
    switch (s) {
        case ATLAS_OK: return "ok";
        case ATLAS_EINVAL: return "invalid argument";
        case ATLAS_EUNSUPPORTED: return "unsupported configuration";
        case ATLAS_EWORKSPACE: return "workspace missing or too small";
        case ATLAS_EDEVICE: return "device error";
        case ATLAS_ECAPACITY: return "pool capacity exceeded";
        default: return "unknown status";
    }
}

const char *atlas_last_error(void) { return g_last_error.c_str(); }

atlas_status atlas_workspace_size(const atlas_attn_args *args, const atlas_regen_spec *regen,
                                  size_t *bytes) {
    if (!bytes) return fail(ATLAS_EINVAL, "bytes is NULL");
    Plan plan;
    atlas_status st = check_common(args, false, regen, &plan, /*sizing=*/true);
    if (st != ATLAS_OK) return st;
    *bytes = plan.total;
    return ok();
}

atlas_status atlas_paged_attention(const atlas_attn_args *args) {
    Plan plan;
    atlas_status st = check_common(args, false, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if ((st = check_workspace(args, plan)) != ATLAS_OK) return st;
    if (plan.mfma) return run_prefill(args, plan, nullptr);
    DecodeParams p = decode_params(args, plan);
    return run_decode(args, plan, p, MODE_PLAIN);
}

atlas_status atlas_paged_attention_noalloc(const atlas_attn_args *args) {
    Plan plan;
    atlas_status st = check_common(args, false, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if (plan.total > ATLAS_NOALLOC_SCRATCH_BYTES)
        return fail(ATLAS_EWORKSPACE,
                    "the call needs %zu workspace bytes, the built-in scratch holds %zu",
                    plan.total, (size_t)ATLAS_NOALLOC_SCRATCH_BYTES);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(ATLAS_EUNSUPPORTED, "device %d", dev);
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        if (!g_scratch_ptr[dev]) {  // first call on this device, with it current
            e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
            if (e != hipSuccess) {
                g_scratch_ptr[dev] = nullptr;
                return device_status(e, "scratch address lookup");
            }
        }
        ptr = g_scratch_ptr[dev];
    }
    atlas_attn_args a = *args;
    a.workspace = ptr;
    a.workspace_bytes = ATLAS_NOALLOC_SCRATCH_BYTES;
    if (plan.mfma) return run_prefill(&a, plan, nullptr);
    DecodeParams p = decode_params(&a, plan);
    return run_decode(&a, plan, p, MODE_PLAIN);
}

atlas_status atlas_paged_attention_tiered(const atlas_attn_args *args,
                                          const atlas_tier_pools *pools) {
    Plan plan;
    atlas_status st = check_common(args, true, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if ((st = check_pools(pools)) != ATLAS_OK) return st;
    if (args->query_start != nullptr)
        return fail(ATLAS_EUNSUPPORTED, "tiered pages support decode only (query_start NULL)");
    if (args->kv_dtype != ATLAS_F16 && args->kv_dtype != ATLAS_BF16)
        return fail(ATLAS_EUNSUPPORTED, "tiered hot pages must be F16 or BF16");
    if ((st = check_workspace(args, plan)) != ATLAS_OK) return st;
    DecodeParams p = decode_params(args, plan);
    set_pools(p, pools);
    return run_decode(args, plan, p, MODE_TIERED);
}

atlas_status atlas_paged_attention_regen(const atlas_attn_args *args,
                                         const atlas_regen_spec *regen) {
    if (!regen) return fail(ATLAS_EINVAL, "regen is NULL");
    Plan plan;
    atlas_status st = check_common(args, false, regen, &plan);
    if (st != ATLAS_OK) return st;
    if ((st = check_workspace(args, plan)) != ATLAS_OK) return st;
    if (plan.mfma) return run_prefill(args, plan, regen);
    DecodeParams p = decode_params(args, plan);
    p.seed = regen->seed;
    p.layer = regen->layer;
    p.regen_pages = regen->regen_pages;
    p.max_regen = regen->max_regen_pages;
    return run_decode(args, plan, p, MODE_REGEN);
}

atlas_status atlas_fold_partials(const float *part_out, const float *part_lse, int32_t splits,
                                 int32_t rows, int32_t head_dim, float *out, float *lse,
                                 void *stream) {
    if (!part_out || !part_lse || !out || !lse)
        return fail(ATLAS_EINVAL, "NULL pointer argument");
    if (splits < 1) return fail(ATLAS_EINVAL, "splits %d < 1", splits);
    if (rows < 0) return fail(ATLAS_EINVAL, "rows %d < 0", rows);
    if (head_dim < 1 || head_dim > 256)
        return fail(ATLAS_EUNSUPPORTED, "head_dim %d outside [1, 256]", head_dim);
    FoldParams f;
    std::memset(&f, 0, sizeof(f));
    f.part_o = part_out;
    f.part_lse = part_lse;
    f.out = out;
    f.lse = lse;
    f.o_row_stride = head_dim;
    f.o_split_stride = (int64_t)rows * head_dim;
    f.l_row_stride = 1;
    f.l_split_stride = rows;
    f.rows = rows;
    f.head_dim = head_dim;
    f.fixed_splits = splits;
    f.num_heads = 1;
    f.split_tokens = 1;
    return device_status(launch_fold(f, reinterpret_cast<hipStream_t>(stream)), "fold launch");
}

atlas_status atlas_gather_pages(const atlas_attn_args *args, int32_t seq, int32_t num_tokens,
                                void *k_out, void *v_out) {
    Plan plan;
    atlas_status st = check_common(args, false, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if (seq < 0 || seq >= args->num_seqs)
        return fail(ATLAS_EINVAL, "seq %d outside [0, %d)", seq, args->num_seqs);
    if (num_tokens < 0 || (int64_t)num_tokens > (int64_t)args->max_pages_per_seq * args->page_tokens)
        return fail(ATLAS_EINVAL, "num_tokens %d outside [0, max_pages * page_tokens]",
                    num_tokens);
    if (!k_out || !v_out) return fail(ATLAS_EINVAL, "NULL output");
    const int eb = args->kv_dtype == ATLAS_F32 ? 4 : 2;
    return device_status(
        launch_gather(args->k_pool, args->v_pool,
                      args->page_table + (int64_t)seq * args->max_pages_per_seq,
                      args->num_kv_heads, args->head_dim, args->page_tokens, args->num_blocks, eb,
                      num_tokens, k_out, v_out, reinterpret_cast<hipStream_t>(args->stream)),
        "gather launch");
}

atlas_status atlas_regenerate_pages(uint64_t seed, uint32_t layer, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t page_tokens, int32_t kv_dtype,
                                    float rope_theta, const int32_t *logical_pages, const int32_t *dst_blocks,
                                    int32_t n, int32_t num_blocks, void *k_pool, void *v_pool,
                                    void *stream, int32_t *nonfinite) {
    if (layer >= (1u << 16)) return fail(ATLAS_EINVAL, "layer %u >= 2^16", layer);
    if (num_kv_heads < 1 || num_kv_heads > 256)
        return fail(ATLAS_EINVAL, "num_kv_heads %d outside [1, 256]", num_kv_heads);
    if (head_dim < 2 || head_dim > 256 || head_dim % 2)
        return fail(ATLAS_EINVAL, "head_dim %d must be even and in [2, 256]", head_dim);
    if (page_tokens < 1) return fail(ATLAS_EINVAL, "page_tokens %d < 1", page_tokens);
    if (kv_dtype != ATLAS_BF16 && kv_dtype != ATLAS_F32)
        return fail(ATLAS_EUNSUPPORTED, "regenerated pages are written as BF16 or F32");
    if (n < 0 || num_blocks < 0) return fail(ATLAS_EINVAL, "negative n or num_blocks");
    if (n > 0 && (!logical_pages || !dst_blocks || !k_pool || !v_pool))
        return fail(ATLAS_EINVAL, "NULL pointer argument");
    if (!std::isfinite(rope_theta) || (rope_theta != 0.0f && !(rope_theta > 1.0f)))
        return fail(ATLAS_EINVAL, "rope_theta must be 0 or a finite value > 1");
    RegenFillParams r;
    std::memset(&r, 0, sizeof(r));
    r.pos = pos_params(rope_theta, nullptr);
    r.seed = seed;
    r.layer = layer;
    r.num_kv_heads = num_kv_heads;
    r.head_dim = head_dim;
    r.page_tokens = page_tokens;
    r.logical_pages = logical_pages;
    r.dst_blocks = dst_blocks;
    r.n = n;
    r.num_blocks = num_blocks;
    r.kv_f32 = kv_dtype == ATLAS_F32;
    r.k_dst = k_pool;
    r.v_dst = v_pool;
    const int eb = kv_dtype == ATLAS_F32 ? 4 : 2;
    if (nonfinite && ((int64_t)page_tokens * head_dim * eb) % 16)
        return fail(ATLAS_EINVAL, "nonfinite counts need page_tokens * head_dim * %d "
                                  "to be a multiple of 16 bytes", eb);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_regen_fill(r, st);
    if (e != hipSuccess) return device_status(e, "regenerate launch");
    if (nonfinite)
        e = launch_count_nonfinite(k_pool, v_pool, dst_blocks, n, num_blocks, num_kv_heads,
                                   page_tokens, head_dim, eb, 0, nonfinite, st);
    return device_status(e, "finite check launch");
}

atlas_status atlas_dequant_pages(const atlas_attn_args *args, const atlas_tier_pools *pools,
                                 const int32_t *entries, int32_t n, float *k_out, float *v_out) {
    Plan plan;
    atlas_status st = check_common(args, true, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if ((st = check_pools(pools)) != ATLAS_OK) return st;
    if ((st = check_1bit_block(args, pools)) != ATLAS_OK) return st;
    if (args->kv_dtype != ATLAS_F16 && args->kv_dtype != ATLAS_BF16)
        return fail(ATLAS_EUNSUPPORTED, "tiered hot pages must be F16 or BF16");
    if (n < 0) return fail(ATLAS_EINVAL, "n %d < 0", n);
    if (n > 0 && (!entries || !k_out || !v_out)) return fail(ATLAS_EINVAL, "NULL pointer");
    DecodeParams p = decode_params(args, plan);
    set_pools(p, pools);
    set_1bit(p, pools);
    return device_status(launch_dequant(p, args->kv_dtype, args->head_dim, entries, n, k_out,
                                        v_out, reinterpret_cast<hipStream_t>(args->stream)),
                         "dequant launch");
}

atlas_status atlas_validate_tables(const atlas_attn_args *args, const atlas_tier_pools *pools,
                                   const atlas_regen_spec *regen, int32_t check_values,
                                   uint32_t *report_dev, uint32_t *report_host) {
    if (pools && regen) return fail(ATLAS_EINVAL, "pools and regen are exclusive");
    Plan plan;
    atlas_status st = check_common(args, pools != nullptr, regen, &plan);
    if (st != ATLAS_OK) return st;
    if (!report_dev) return fail(ATLAS_EINVAL, "report_dev is NULL");
    if (pools && pools->struct_size != sizeof(atlas_tier_pools))
        return fail(ATLAS_EINVAL, "pools->struct_size mismatch");
    if (pools && (pools->num_int8 < 0 || pools->num_int4 < 0 || pools->num_fp8 < 0 ||
                  pools->num_int2 < 0))
        return fail(ATLAS_EINVAL, "negative tier pool size");
    ValidateParams v;
    std::memset(&v, 0, sizeof(v));
    v.p = decode_params(args, plan);
    v.p.part_o = nullptr;
    v.p.part_lse = nullptr;
    v.mode = pools ? MODE_TIERED : regen ? MODE_REGEN : MODE_PLAIN;
    if (pools) {
        v.p.i8_ks = pools->int8_k_scale;
        v.p.i8_vs = pools->int8_v_scale;
        v.p.i4_ks = pools->int4_k_scale;
        v.p.i4_vs = pools->int4_v_scale;
        v.p.n_i8 = pools->num_int8;
        v.p.n_i4 = pools->num_int4;
        v.p.f8_k = pools->fp8_k;
        v.p.f8_v = pools->fp8_v;
        v.p.f8_ks = pools->fp8_k_scale;
        v.p.f8_vs = pools->fp8_v_scale;
        v.p.n_f8 = pools->num_fp8;
        v.p.i2_ks = pools->int2_k_scale;
        v.p.i2_vs = pools->int2_v_scale;
        v.p.n_i2 = pools->num_int2;
        if (check_values && ((v.p.n_i8 > 0 && (!v.p.i8_ks || !v.p.i8_vs)) ||
                             (v.p.n_i4 > 0 && (!v.p.i4_ks || !v.p.i4_vs)) ||
                             (v.p.n_f8 > 0 && (!v.p.f8_ks || !v.p.f8_vs)) ||
                             (v.p.n_i2 > 0 && (!v.p.i2_ks || !v.p.i2_vs))))
            return fail(ATLAS_EINVAL, "NULL tier scale pointer");
    }
    if (regen) {
        v.p.regen_pages = regen->regen_pages;
        v.p.max_regen = regen->max_regen_pages;
    }
    v.kv_type = args->kv_dtype;
    v.head_dim = args->head_dim;
    v.check_values = check_values ? 1 : 0;
    v.max_query_len = args->max_query_len;
    v.report = report_dev;
    hipStream_t stream = reinterpret_cast<hipStream_t>(args->stream);
    hipError_t e = launch_validate(v, stream);
    if (e != hipSuccess) return device_status(e, "validate launch");
    if (report_host) {
        e = hipMemcpyAsync(report_host, report_dev, 4 * sizeof(uint32_t), hipMemcpyDeviceToHost,
                           stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return device_status(e, "validate report copy");
    }
    return ok();
}

atlas_status atlas_read_probe(const void *src, size_t bytes, uint32_t *out, int32_t blocks,
                              void *stream) {
    if (!src || !out) return fail(ATLAS_EINVAL, "NULL pointer argument");
    if (bytes % 16) return fail(ATLAS_EINVAL, "bytes %zu is not a multiple of 16", bytes);
    if (reinterpret_cast<uintptr_t>(src) % 16) return fail(ATLAS_EINVAL, "src is not 16-byte aligned");
    if (blocks < 1 || blocks > (1 << 20)) return fail(ATLAS_EINVAL, "blocks %d outside [1, 2^20]", blocks);
    return device_status(launch_read_probe(src, (int64_t)bytes, out, blocks,
                                           reinterpret_cast<hipStream_t>(stream)),
                         "read probe launch");
}

atlas_status atlas_issue_probe(int32_t mix, int32_t waves_per_simd, int32_t iters,
                               uint64_t *clocks, float *sink, void *stream) {
    if (!clocks || !sink) return fail(ATLAS_EINVAL, "NULL pointer argument");
    if (mix < 0 || mix > 7) return fail(ATLAS_EINVAL, "mix %d outside [0, 7]", mix);
    if (waves_per_simd != 1 && waves_per_simd != 2)
        return fail(ATLAS_EINVAL, "waves_per_simd %d is not 1 or 2", waves_per_simd);
    if (iters < 1 || iters > (1 << 20)) return fail(ATLAS_EINVAL, "iters %d outside [1, 2^20]", iters);
    return device_status(launch_issue_probe(mix, waves_per_simd, iters, clocks, sink,
                                            reinterpret_cast<hipStream_t>(stream)),
                         "issue probe launch");
}

atlas_status atlas_write_kv(const atlas_attn_args *args, const void *k_new, const void *v_new) {
    Plan plan;
    atlas_status st = check_common(args, false, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if (!k_new || !v_new) return fail(ATLAS_EINVAL, "NULL k_new or v_new");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16 ||
        reinterpret_cast<uintptr_t>(args->k_pool) % 16 ||
        reinterpret_cast<uintptr_t>(args->v_pool) % 16)
        return fail(ATLAS_EINVAL, "k_new, v_new and the pools must be 16-byte aligned");
    WriteKvParams w;
    std::memset(&w, 0, sizeof(w));
    w.rows = row_map(args);
    w.pos = pos_params(args->rope_theta, nullptr);
    w.k_new = k_new;
    w.v_new = v_new;
    w.k_pool = const_cast<void *>(args->k_pool);
    w.v_pool = const_cast<void *>(args->v_pool);
    w.page_table = args->page_table;
    w.num_kv_heads = args->num_kv_heads;
    w.head_dim = args->head_dim;
    w.page_tokens = args->page_tokens;
    w.max_pages = args->max_pages_per_seq;
    w.num_blocks = args->num_blocks;
    w.total_q = args->total_q;
    w.elem_bytes = args->kv_dtype == ATLAS_F32 ? 4 : 2;
    w.kv_type = args->kv_dtype;
    return device_status(launch_write_kv(w, reinterpret_cast<hipStream_t>(args->stream)),
                         "write launch");
}

atlas_status atlas_demote_pages(const atlas_attn_args *args, const atlas_tier_pools *pools,
                                const int32_t *src_slots, const int32_t *dst_entries, int32_t n,
                                int32_t *rejected) {
    Plan plan;
    atlas_status st = check_common(args, true, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if ((st = check_pools(pools)) != ATLAS_OK) return st;
    if ((st = check_1bit_block(args, pools)) != ATLAS_OK) return st;
    if (args->kv_dtype != ATLAS_F16 && args->kv_dtype != ATLAS_BF16)
        return fail(ATLAS_EUNSUPPORTED, "hot pages must be F16 or BF16");
    if (n < 0) return fail(ATLAS_EINVAL, "n %d < 0", n);
    if (n == 0) return ok();
    if (!src_slots || !dst_entries) return fail(ATLAS_EINVAL, "NULL src_slots or dst_entries");
    if ((int64_t)n * args->num_kv_heads * 2 > INT32_MAX) return fail(ATLAS_EINVAL, "n too large");
    DemoteParams d;
    std::memset(&d, 0, sizeof(d));
    d.k_pool = args->k_pool;
    d.v_pool = args->v_pool;
    d.kv_type = args->kv_dtype;
    d.num_kv_heads = args->num_kv_heads;
    d.head_dim = args->head_dim;
    d.page_tokens = args->page_tokens;
    d.num_blocks = args->num_blocks;
    d.src_slots = src_slots;
    d.dst_entries = dst_entries;
    d.n = n;
    d.i8_k = const_cast<int8_t *>(pools->int8_k);
    d.i8_v = const_cast<int8_t *>(pools->int8_v);
    d.i8_ks = const_cast<float *>(pools->int8_k_scale);
    d.i8_vs = const_cast<float *>(pools->int8_v_scale);
    d.i4_k = const_cast<uint8_t *>(pools->int4_k);
    d.i4_v = const_cast<uint8_t *>(pools->int4_v);
    d.i4_ks = const_cast<float *>(pools->int4_k_scale);
    d.i4_vs = const_cast<float *>(pools->int4_v_scale);
    d.f8_k = const_cast<uint8_t *>(pools->fp8_k);
    d.f8_v = const_cast<uint8_t *>(pools->fp8_v);
    d.f8_ks = const_cast<float *>(pools->fp8_k_scale);
    d.f8_vs = const_cast<float *>(pools->fp8_v_scale);
    d.i2_k = const_cast<uint8_t *>(pools->int2_k);
    d.i2_v = const_cast<uint8_t *>(pools->int2_v);
    d.i2_ks = const_cast<float *>(pools->int2_k_scale);
    d.i2_vs = const_cast<float *>(pools->int2_v_scale);
    d.n_i8 = pools->num_int8;
    d.n_i4 = pools->num_int4;
    d.n_f8 = pools->num_fp8;
    d.n_i2 = pools->num_int2;
    d.b1_k = const_cast<uint8_t *>(pools->bit_k);
    d.b1_v = const_cast<uint8_t *>(pools->bit_v);
    d.b1_ks = const_cast<float *>(pools->bit_k_scale);
    d.b1_vs = const_cast<float *>(pools->bit_v_scale);
    d.b1_ko = const_cast<uint32_t *>(pools->bit_k_out);
    d.b1_vo = const_cast<uint32_t *>(pools->bit_v_out);
    d.n_b1 = pools->num_1bit;
    d.b1_nout = pools->outliers_1bit;
    d.rejected = rejected;
    return device_status(launch_demote(d, reinterpret_cast<hipStream_t>(args->stream)),
                         "demote launch");
}

atlas_status atlas_promote_pages(const atlas_attn_args *args, const atlas_tier_pools *pools,
                                 const int32_t *src_entries, const int32_t *dst_blocks, int32_t n,
                                 int32_t *rejected, int32_t *nonfinite) {
    Plan plan;
    atlas_status st = check_common(args, true, nullptr, &plan);
    if (st != ATLAS_OK) return st;
    if ((st = check_pools(pools)) != ATLAS_OK) return st;
    if ((st = check_1bit_block(args, pools)) != ATLAS_OK) return st;
    if (args->num_blocks < 1 || !args->k_pool || !args->v_pool)
        return fail(ATLAS_EINVAL, "promotion needs a hot pool (num_blocks >= 1)");
    if (n < 0) return fail(ATLAS_EINVAL, "n %d < 0", n);
    if (n == 0) return ok();
    if (!src_entries || !dst_blocks) return fail(ATLAS_EINVAL, "NULL src_entries or dst_blocks");
    if ((int64_t)n * args->num_kv_heads * 2 > INT32_MAX) return fail(ATLAS_EINVAL, "n too large");
    PromoteParams q;
    std::memset(&q, 0, sizeof(q));
    q.p.k_pool = args->k_pool;
    q.p.v_pool = args->v_pool;
    q.p.num_kv_heads = args->num_kv_heads;
    q.p.page_tokens = args->page_tokens;
    q.p.num_blocks = args->num_blocks;
    set_pools(q.p, pools);
    set_1bit(q.p, pools);
    q.k_dst = const_cast<void *>(args->k_pool);
    q.v_dst = const_cast<void *>(args->v_pool);
    q.kv_type = args->kv_dtype;
    q.head_dim = args->head_dim;
    q.src_entries = src_entries;
    q.dst_blocks = dst_blocks;
    q.n = n;
    q.rejected = rejected;
    hipStream_t stream = reinterpret_cast<hipStream_t>(args->stream);
    hipError_t e = launch_promote(q, stream);
    if (e != hipSuccess) return device_status(e, "promote launch");
    if (nonfinite) {
        const int eb = args->kv_dtype == ATLAS_F32 ? 4 : 2;
        e = launch_count_nonfinite(args->k_pool, args->v_pool, dst_blocks, n, args->num_blocks,
                                   args->num_kv_heads, args->page_tokens, args->head_dim, eb,
                                   args->kv_dtype == ATLAS_F16 ? 1 : 0, nonfinite, stream);
    }
    return device_status(e, "finite check launch");
}

}  // extern "C"
