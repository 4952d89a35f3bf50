// Host residency runtime: which pages of each sequence are hot, regenerated or
// stored in a cold tier, and the page tables the attention calls read.
//
// CFR-Atlas README: a bounded hot-page cache with LRU replacement, the
// KeepRecent { recent_tokens } policy and the admission of regenerated pages
// into the cache.  argus-cache, "Visual Architecture" and its configuration
// (max_active_pages, max_fp8_pages, sink_tokens): an FP16 active pool, the
// compression cascade FP8 -> INT8 -> INT4 -> INT2 -> 1-bit for older pages,
// attention sinks kept in FP16, and archived pages rebuilt in FP16 for the
// call that needs them (its overview: transient FP16 reconstruction).
//
// Regen mode keeps, per sequence, a resident suffix of pages (the kernels
// regenerate a leading run of pages, so the regenerated set is always a
// prefix): pages [first_resident, n_pages) are hot, the rest regenerated.
// The suffix must cover the KeepRecent window; pages in front of the window
// stay as long as the hot pool has room and are the LRU victims when it has
// not.  Tiered mode gives every page a target tier from its position (sink
// and window pages hot; counting back from the window, FP8, then INT8, then
// INT4, INT2 and the 1-bit archive) and moves each page that is hotter than
// its target in one job.
//
// Budgets (CFR-Atlas README, test list: global and per-layer budgets).  A
// runtime serves one layer: hot_blocks is that layer's budget.  Runtimes
// may also share an atlas_residency_budget, a count of hot blocks that all
// of them together may hold (the global budget); a hot block is taken only
// when both the layer's pool and the shared budget have room.
//
// Admission check (CFR-Atlas README, hardening baseline: finite-value
// validation before hot-cache admission).  atlas_regenerate_pages reports
// the non-finite values it stored per job; the caller hands the counts to
// atlas_residency_refuse_admissions, which takes back every flagged page
// (and the pages admitted below it in the same plan, so the resident run
// stays a suffix) before its block can be named by a page table.
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "atlas_residency.h"

namespace atlas {
int32_t report_error(int32_t st, const char *msg);
int32_t report_ok();
}  // namespace atlas

namespace {

constexpr uint32_t kShift = ATLAS_TIER_SHIFT;
constexpr uint32_t kSlotMask = (1u << kShift) - 1u;
// Page classes: the tiers, with the extension tier split into FP8, INT2 and
// the 1-bit archive.
constexpr int kTierHot = 0, kTierI8 = 1, kTierI4 = 2, kTierF8 = 3, kTierI2 = 4, kTierB1 = 5;

int32_t fail(int32_t st, const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    return atlas::report_error(st, buf);
}

// Coldness order of the classes: hot < FP8 < INT8 < INT4 < INT2 < 1-bit.
int coldness(int cls) {
    switch (cls) {
        case kTierHot: return 0;
        case kTierF8: return 1;
        case kTierI8: return 2;
        case kTierI4: return 3;
        case kTierI2: return 4;
        default: return 5;
    }
}

// Page-table entry of a class and slot (FP8, INT2 and 1-bit share tier 3).
uint32_t entry(int cls, int32_t slot) {
    if (cls == kTierI2 || cls == kTierB1)
        return (3u << kShift) |
               ((uint32_t)(cls == kTierI2 ? ATLAS_EXT_INT2 : ATLAS_EXT_1BIT) << ATLAS_EXT_KIND_SHIFT) |
               (uint32_t)slot;
    return ((uint32_t)cls << kShift) | (uint32_t)slot;
}

int class_of(uint32_t e) {
    const uint32_t tier = e >> kShift;
    if (tier < 3) return (int)tier;
    const uint32_t kind = (e >> ATLAS_EXT_KIND_SHIFT) & 3u;
    return kind == ATLAS_EXT_INT2 ? kTierI2 : kind == ATLAS_EXT_1BIT ? kTierB1 : kTierF8;
}

int32_t slot_of(uint32_t e) {
    return (int32_t)(e & ((e >> kShift) == 3u ? (1u << ATLAS_EXT_KIND_SHIFT) - 1u : kSlotMask));
}

}  // namespace

// Hot blocks that several runtimes (layers) may hold together.
struct atlas_residency_budget {
    int64_t limit = 0;
    int64_t used = 0;
};

namespace {

// A pool of numbered slots; freed slots are reused lowest-first so the
// allocation order is deterministic.  The hot pool may also draw on a
// shared budget: a slot is available only while the budget has room.
struct SlotPool {
    std::vector<int32_t> free_;  // kept sorted descending: back() is the lowest
    int32_t capacity = 0;
    atlas_residency_budget *budget = nullptr;
    void init(int32_t n, atlas_residency_budget *b = nullptr) {
        capacity = n;
        budget = b;
        free_.clear();
        for (int32_t i = n - 1; i >= 0; --i) free_.push_back(i);
    }
    // slots that can be taken now
    int64_t available() const {
        int64_t a = (int64_t)free_.size();
        if (budget) a = std::min<int64_t>(a, std::max<int64_t>(0, budget->limit - budget->used));
        return a;
    }
    bool empty() const { return available() == 0; }
    int32_t take() {
        const int32_t s = free_.back();
        free_.pop_back();
        if (budget) ++budget->used;
        return s;
    }
    void give(int32_t s) {
        free_.insert(std::upper_bound(free_.begin(), free_.end(), s, std::greater<int32_t>()), s);
        if (budget) --budget->used;
    }
    int32_t used() const { return capacity - (int32_t)free_.size(); }
};

struct Seq {
    bool active = false;
    int64_t tokens = 0;
    std::vector<uint32_t> pages;  // entry per logical page (regen mode: hot block id)
    int32_t first_resident = 0;   // regen mode: pages before this are regenerated
    uint64_t last_use = 0;
};

}  // namespace

struct atlas_residency {
    atlas_residency_config cfg;
    std::vector<Seq> seqs;
    SlotPool hot, f8, i8, i4, i2, b1;
    uint64_t tick = 0;
    atlas_residency_stats st;

    SlotPool &pool(int tier) {
        switch (tier) {
            case kTierHot: return hot;
            case kTierF8: return f8;
            case kTierI8: return i8;
            case kTierI4: return i4;
            case kTierI2: return i2;
            default: return b1;
        }
    }
    int32_t pages_of(const Seq &s) const {
        return (int32_t)((s.tokens + cfg.page_tokens - 1) / cfg.page_tokens);
    }
    // First page of the KeepRecent window of a sequence with `tokens` keys.
    int32_t window_first(int64_t tokens) const {
        const int64_t t = std::max<int64_t>(0, tokens - cfg.recent_tokens);
        return (int32_t)(t / cfg.page_tokens);
    }
    int32_t sink_pages() const {
        return (int32_t)((cfg.sink_tokens + cfg.page_tokens - 1) / cfg.page_tokens);
    }
    // Tiered mode: the tier page p of a sequence with n pages and window
    // start wf should be in.
    int target_tier(int32_t p, int32_t wf) const {
        if (p < sink_pages() || p >= wf) return kTierHot;
        const int64_t r = wf - 1 - p;  // 0 = the newest cold page
        int64_t edge = cfg.fp8_pages;
        if (r < edge) return kTierF8;
        if (r < (edge += cfg.int8_pages)) return kTierI8;
        const bool i2 = cfg.num_int2 > 0, b1 = cfg.num_1bit > 0;
        if (!i2 && !b1) return kTierI4;
        if (r < (edge += cfg.int4_pages)) return kTierI4;
        if (!b1) return kTierI2;
        if (i2 && r < edge + cfg.int2_pages) return kTierI2;
        return kTierB1;
    }
    // The table entry of pages the runtime does not hand out: regenerated
    // pages and pages past the context.
    int32_t filler() const { return cfg.hot_blocks + cfg.transient_blocks; }
    // Regen mode: resident pages of a sequence that may be dropped back to
    // regeneration (in front of its window).
    int32_t evictable(const Seq &s) const {
        return std::max(0, std::min(window_first(s.tokens), (int32_t)s.pages.size()) -
                               s.first_resident);
    }
};

namespace {

bool valid_seq(const atlas_residency *rt, int32_t seq) {
    return rt && seq >= 0 && seq < rt->cfg.max_seqs;
}

// Regen mode: drop the oldest evictable page of the least recently used
// sequence (ties: lowest id).  Returns false if no page is evictable.
bool evict_one(atlas_residency *rt) {
    int best = -1;
    for (int i = 0; i < (int)rt->seqs.size(); ++i) {
        const Seq &s = rt->seqs[i];
        if (!s.active || rt->evictable(s) == 0) continue;
        if (best < 0 || s.last_use < rt->seqs[best].last_use) best = i;
    }
    if (best < 0) return false;
    Seq &s = rt->seqs[best];
    rt->hot.give((int32_t)s.pages[s.first_resident]);
    s.pages[s.first_resident] = 0;
    ++s.first_resident;
    ++rt->st.evictions;
    return true;
}

}  // namespace

namespace {

atlas_status fill_tables(atlas_residency *rt, const int32_t *seqs, int32_t n, int32_t *page_table,
                         int32_t *context_lens, int32_t *regen_pages,
                         atlas_residency_jobs *jobs) {
    if (!rt) return fail(ATLAS_EINVAL, "runtime is NULL");
    if (n < 0) return fail(ATLAS_EINVAL, "n %d < 0", n);
    if (n > 0 && (!seqs || !page_table || !context_lens))
        return fail(ATLAS_EINVAL, "NULL seqs, page_table or context_lens");
    if (n > 0 && rt->cfg.mode == ATLAS_RESIDENCY_REGEN && !regen_pages)
        return fail(ATLAS_EINVAL, "regen mode needs regen_pages");
    for (int32_t i = 0; i < n; ++i)
        if (!valid_seq(rt, seqs[i]) || !rt->seqs[seqs[i]].active)
            return fail(ATLAS_EINVAL, "sequence %d is not active", seqs[i]);
    for (int32_t i = 0; i < n; ++i)
        if (rt->seqs[seqs[i]].tokens > INT32_MAX) return fail(ATLAS_EINVAL, "context too long");
    if (jobs) {  // archived pages of the listed sequences get transient blocks
        if (jobs->struct_size != sizeof(atlas_residency_jobs))
            return fail(ATLAS_EINVAL, "jobs->struct_size %u != %zu", jobs->struct_size,
                        sizeof(atlas_residency_jobs));
        int64_t archived = 0;
        for (int32_t i = 0; i < n; ++i)
            for (uint32_t e : rt->seqs[seqs[i]].pages)
                if (rt->cfg.mode == ATLAS_RESIDENCY_TIERED && class_of(e) == kTierB1) ++archived;
        if (archived > rt->cfg.transient_blocks) {
            ++rt->st.capacity_failures;
            return fail(ATLAS_ECAPACITY, "%lld archived pages, %d transient blocks",
                        (long long)archived, rt->cfg.transient_blocks);
        }
        if (archived > jobs->capacity)
            return fail(ATLAS_EINVAL, "jobs capacity %d < %lld archived pages", jobs->capacity,
                        (long long)archived);
        if (archived > 0 && (!jobs->promote_src || !jobs->promote_dst))
            return fail(ATLAS_EINVAL, "NULL promote arrays");
        jobs->n_demote = 0;
        jobs->n_admit = 0;
        jobs->n_promote = 0;
    }
    const int32_t M = rt->cfg.max_pages_per_seq;
    int32_t k = 0;  // transient blocks handed out
    for (int32_t i = 0; i < n; ++i) {
        Seq &s = rt->seqs[seqs[i]];
        int32_t *row = page_table + (int64_t)i * M;
        // regenerated pages and pages past the context name a block the
        // runtime never hands out (atlas_write_kv skips such rows when the
        // pool has no block there)
        std::fill(row, row + M, rt->filler());
        for (int32_t p = (rt->cfg.mode == ATLAS_RESIDENCY_REGEN ? s.first_resident : 0);
             p < (int32_t)s.pages.size(); ++p) {
            row[p] = (int32_t)s.pages[p];
            if (jobs && rt->cfg.mode == ATLAS_RESIDENCY_TIERED && class_of(s.pages[p]) == kTierB1) {
                const int32_t blk = rt->cfg.hot_blocks + k;
                jobs->promote_src[k] = (int32_t)s.pages[p];
                jobs->promote_dst[k] = blk;
                row[p] = blk;
                ++k;
            }
        }
        context_lens[i] = (int32_t)s.tokens;
        if (regen_pages) regen_pages[i] = rt->cfg.mode == ATLAS_RESIDENCY_REGEN ? s.first_resident : 0;
        s.last_use = ++rt->tick;
    }
    if (jobs) {
        jobs->n_promote = k;
        rt->st.reconstructions += k;
    }
    return atlas::report_ok();
}

}  // namespace

extern "C" {

atlas_status atlas_residency_create(const atlas_residency_config *c, atlas_residency **out) {
    if (!c || !out) return fail(ATLAS_EINVAL, "config or out is NULL");
    if (c->struct_size != sizeof(atlas_residency_config))
        return fail(ATLAS_EINVAL, "config->struct_size %u != %zu", c->struct_size,
                    sizeof(atlas_residency_config));
    if (c->mode != ATLAS_RESIDENCY_REGEN && c->mode != ATLAS_RESIDENCY_TIERED)
        return fail(ATLAS_EINVAL, "unknown mode %d", c->mode);
    if (c->page_tokens < 1 || c->max_seqs < 1 || c->max_pages_per_seq < 1)
        return fail(ATLAS_EINVAL, "page_tokens, max_seqs and max_pages_per_seq must be >= 1");
    if (c->hot_blocks < 0 || c->hot_blocks > (int32_t)kSlotMask)
        return fail(ATLAS_EINVAL, "hot_blocks %d outside [0, 2^30)", c->hot_blocks);
    if (c->recent_tokens < 0 || c->sink_tokens < 0 || c->admit_per_plan < 0 ||
        c->fp8_pages < 0 || c->int8_pages < 0 || c->int4_pages < 0 || c->num_int2 < 0 ||
        c->num_int2 > (1 << ATLAS_EXT_KIND_SHIFT))
        return fail(ATLAS_EINVAL, "negative policy field");
    if (c->num_fp8 < 0 || c->num_int8 < 0 || c->num_int4 < 0 ||
        c->num_fp8 > (1 << ATLAS_EXT_KIND_SHIFT) || c->num_int8 > (int32_t)kSlotMask ||
        c->num_int4 > (int32_t)kSlotMask)
        return fail(ATLAS_EINVAL, "cold pool size outside [0, 2^30) (FP8: 2^28)");
    if (c->int2_pages < 0 || c->num_1bit < 0 || c->num_1bit > (1 << ATLAS_EXT_KIND_SHIFT) ||
        c->transient_blocks < 0 || (int64_t)c->hot_blocks + c->transient_blocks > (int64_t)kSlotMask)
        return fail(ATLAS_EINVAL, "1-bit archive or transient block field out of range");
    if ((int64_t)c->max_seqs * c->max_pages_per_seq > ((int64_t)1 << 31))
        return fail(ATLAS_EINVAL, "max_seqs * max_pages_per_seq too large");
    atlas_residency *rt = new (std::nothrow) atlas_residency();
    if (!rt) return fail(ATLAS_EINVAL, "out of host memory");
    rt->cfg = *c;
    rt->seqs.resize(c->max_seqs);
    rt->hot.init(c->hot_blocks, c->budget);
    rt->f8.init(c->mode == ATLAS_RESIDENCY_TIERED ? c->num_fp8 : 0);
    rt->i8.init(c->mode == ATLAS_RESIDENCY_TIERED ? c->num_int8 : 0);
    rt->i4.init(c->mode == ATLAS_RESIDENCY_TIERED ? c->num_int4 : 0);
    rt->i2.init(c->mode == ATLAS_RESIDENCY_TIERED ? c->num_int2 : 0);
    rt->b1.init(c->mode == ATLAS_RESIDENCY_TIERED ? c->num_1bit : 0);
    std::memset(&rt->st, 0, sizeof(rt->st));
    rt->st.struct_size = sizeof(atlas_residency_stats);
    *out = rt;
    return atlas::report_ok();
}

atlas_status atlas_residency_destroy(atlas_residency *rt) {
    if (rt && rt->hot.budget) rt->hot.budget->used -= rt->hot.used();  // its blocks go back
    delete rt;
    return atlas::report_ok();
}

atlas_status atlas_residency_budget_create(int64_t blocks, atlas_residency_budget **out) {
    if (!out) return fail(ATLAS_EINVAL, "out is NULL");
    if (blocks < 0) return fail(ATLAS_EINVAL, "blocks %lld < 0", (long long)blocks);
    atlas_residency_budget *b = new (std::nothrow) atlas_residency_budget();
    if (!b) return fail(ATLAS_EINVAL, "out of host memory");
    b->limit = blocks;
    *out = b;
    return atlas::report_ok();
}

atlas_status atlas_residency_budget_destroy(atlas_residency_budget *b) {
    delete b;
    return atlas::report_ok();
}

atlas_status atlas_residency_budget_used(const atlas_residency_budget *b, int64_t *used) {
    if (!b || !used) return fail(ATLAS_EINVAL, "budget or used is NULL");
    *used = b->used;
    return atlas::report_ok();
}

atlas_status atlas_residency_refuse_admissions(atlas_residency *rt,
                                               const atlas_residency_jobs *jobs,
                                               const int32_t *nonfinite) {
    if (!rt || !jobs) return fail(ATLAS_EINVAL, "runtime or jobs is NULL");
    if (jobs->struct_size != sizeof(atlas_residency_jobs))
        return fail(ATLAS_EINVAL, "jobs->struct_size %u != %zu", jobs->struct_size,
                    sizeof(atlas_residency_jobs));
    if (rt->cfg.mode != ATLAS_RESIDENCY_REGEN)
        return fail(ATLAS_EINVAL, "admissions exist in regen mode only");
    const int32_t n = jobs->n_admit;
    if (n < 0 || n > jobs->capacity) return fail(ATLAS_EINVAL, "n_admit %d out of range", n);
    if (n == 0) return atlas::report_ok();
    if (!nonfinite || !jobs->admit_page || !jobs->admit_block)
        return fail(ATLAS_EINVAL, "NULL admission arrays or counts");
    // the owner of every job: the sequence whose page admit_page names the
    // job's block inside its resident suffix (checked before any change)
    std::vector<int> owner(n, -1);
    for (int32_t j = 0; j < n; ++j) {
        const int32_t pg = jobs->admit_page[j], blk = jobs->admit_block[j];
        for (int i = 0; i < (int)rt->seqs.size() && owner[j] < 0; ++i) {
            const Seq &s = rt->seqs[i];
            if (s.active && pg >= s.first_resident && pg < (int32_t)s.pages.size() &&
                s.pages[pg] == (uint32_t)blk)
                owner[j] = i;
        }
        if (owner[j] < 0)
            return fail(ATLAS_EINVAL, "job %d (page %d, block %d) is not a current admission", j,
                        pg, blk);
    }
    // per sequence, the highest flagged page; every page of this plan at or
    // below it goes back to regeneration
    std::vector<int32_t> cut(rt->seqs.size(), -1);
    for (int32_t j = 0; j < n; ++j)
        if (nonfinite[j] != 0) cut[owner[j]] = std::max(cut[owner[j]], jobs->admit_page[j]);
    for (int32_t j = 0; j < n; ++j) {
        Seq &s = rt->seqs[owner[j]];
        const int32_t pg = jobs->admit_page[j];
        if (pg > cut[owner[j]]) continue;
        rt->hot.give(jobs->admit_block[j]);
        s.pages[pg] = 0u;
        ++rt->st.refused_admissions;
        --rt->st.admissions;
    }
    for (int i = 0; i < (int)rt->seqs.size(); ++i)
        if (cut[i] >= 0) rt->seqs[i].first_resident = std::max(rt->seqs[i].first_resident,
                                                               cut[i] + 1);
    return atlas::report_ok();
}

atlas_status atlas_residency_add_seq(atlas_residency *rt, int32_t seq) {
    if (!valid_seq(rt, seq)) return fail(ATLAS_EINVAL, "sequence %d out of range", seq);
    Seq &s = rt->seqs[seq];
    if (s.active) return fail(ATLAS_EINVAL, "sequence %d is already active", seq);
    s = Seq();
    s.active = true;
    s.last_use = ++rt->tick;
    return atlas::report_ok();
}

atlas_status atlas_residency_remove_seq(atlas_residency *rt, int32_t seq) {
    if (!valid_seq(rt, seq) || !rt->seqs[seq].active)
        return fail(ATLAS_EINVAL, "sequence %d is not active", seq);
    Seq &s = rt->seqs[seq];
    const bool tiered = rt->cfg.mode == ATLAS_RESIDENCY_TIERED;
    for (int32_t p = tiered ? 0 : s.first_resident; p < (int32_t)s.pages.size(); ++p) {
        const uint32_t e = s.pages[p];
        const int tier = tiered ? class_of(e) : kTierHot;
        rt->pool(tier).give(tiered ? slot_of(e) : (int32_t)e);
    }
    s = Seq();
    return atlas::report_ok();
}

atlas_status atlas_residency_append(atlas_residency *rt, int32_t seq, int32_t n_tokens) {
    if (!valid_seq(rt, seq) || !rt->seqs[seq].active)
        return fail(ATLAS_EINVAL, "sequence %d is not active", seq);
    if (n_tokens < 0) return fail(ATLAS_EINVAL, "n_tokens %d < 0", n_tokens);
    Seq &s = rt->seqs[seq];
    const int64_t tokens = s.tokens + n_tokens;
    const int64_t pages = (tokens + rt->cfg.page_tokens - 1) / rt->cfg.page_tokens;
    if (pages > rt->cfg.max_pages_per_seq)
        return fail(ATLAS_EINVAL, "sequence %d would need %lld pages > max_pages_per_seq %d", seq,
                    (long long)pages, rt->cfg.max_pages_per_seq);
    const bool regen = rt->cfg.mode == ATLAS_RESIDENCY_REGEN;
    const int32_t old_pages = (int32_t)s.pages.size();
    const int32_t wf = rt->window_first(tokens);
    // Regen mode: while a sequence has no resident page, its new pages in
    // front of the (new) KeepRecent window are regenerated from the start
    // (a long prompt's early pages take no hot block).
    int32_t skip = 0;
    if (regen && s.first_resident == old_pages)
        skip = std::max(0, std::min(wf, (int32_t)pages) - old_pages);
    const int32_t need = (int32_t)pages - old_pages - skip;
    // capacity check before any change (transactional)
    int64_t room = rt->hot.available();
    if (regen && room < need) {
        for (const Seq &o : rt->seqs) {
            if (!o.active) continue;
            // the growing sequence's window moves forward with the new tokens
            room += &o == &s ? std::max(0, std::min(wf, old_pages) - o.first_resident)
                             : rt->evictable(o);
        }
    }
    if (room < need) {
        ++rt->st.capacity_failures;
        return fail(ATLAS_ECAPACITY, "hot pool: %d new pages, room for %lld", need,
                    (long long)room);
    }
    s.tokens = tokens;  // the window of the growing sequence moves first
    for (int32_t i = 0; i < skip; ++i) s.pages.push_back(0u);
    s.first_resident += skip;
    for (int32_t i = 0; i < need; ++i) {
        if (rt->hot.empty()) {
            const bool ok = evict_one(rt);
            (void)ok;  // guaranteed by the room check
        }
        s.pages.push_back((uint32_t)rt->hot.take());
    }
    s.last_use = ++rt->tick;
    rt->st.appended_tokens += n_tokens;
    return atlas::report_ok();
}

atlas_status atlas_residency_plan(atlas_residency *rt, atlas_residency_jobs *jobs) {
    if (!rt || !jobs) return fail(ATLAS_EINVAL, "runtime or jobs is NULL");
    if (jobs->struct_size != sizeof(atlas_residency_jobs))
        return fail(ATLAS_EINVAL, "jobs->struct_size %u != %zu", jobs->struct_size,
                    sizeof(atlas_residency_jobs));
    if (jobs->capacity < 0) return fail(ATLAS_EINVAL, "jobs capacity < 0");
    jobs->n_demote = 0;
    jobs->n_admit = 0;
    jobs->n_promote = 0;

    if (rt->cfg.mode == ATLAS_RESIDENCY_REGEN) {
        if (rt->cfg.admit_per_plan > 0 && jobs->capacity > 0 &&
            (!jobs->admit_page || !jobs->admit_block))
            return fail(ATLAS_EINVAL, "NULL admit arrays");
        // most recently used sequences first (ties: lowest id)
        std::vector<int> order;
        for (int i = 0; i < (int)rt->seqs.size(); ++i)
            if (rt->seqs[i].active && rt->seqs[i].first_resident > 0) order.push_back(i);
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
            return rt->seqs[a].last_use > rt->seqs[b].last_use;
        });
        int32_t n = 0;
        const int32_t limit = std::min(rt->cfg.admit_per_plan, jobs->capacity);
        for (int i : order) {
            Seq &s = rt->seqs[i];
            while (n < limit && s.first_resident > 0 && !rt->hot.empty()) {
                const int32_t blk = rt->hot.take();
                --s.first_resident;
                s.pages[s.first_resident] = (uint32_t)blk;
                jobs->admit_page[n] = s.first_resident;
                jobs->admit_block[n] = blk;
                ++n;
            }
        }
        // admissions of different sequences may name the same logical page:
        // the regenerated values do not depend on the sequence
        jobs->n_admit = n;
        rt->st.admissions += n;
        return atlas::report_ok();
    }

    // tiered: collect the moves, allocate with fallback, commit or roll back
    struct Move {
        int seq;
        int32_t page;
        uint32_t from, to;
    };
    std::vector<Move> moves;
    for (int i = 0; i < (int)rt->seqs.size(); ++i) {
        const Seq &s = rt->seqs[i];
        if (!s.active) continue;
        const int32_t wf = rt->window_first(s.tokens);
        // newest pages first: when a warm pool runs short, the newest pages
        // keep the warmer tiers
        for (int32_t p = (int32_t)s.pages.size() - 1; p >= 0; --p) {
            const int cur = class_of(s.pages[p]);
            const int want = rt->target_tier(p, wf);
            if (coldness(want) > coldness(cur)) moves.push_back({i, p, s.pages[p], (uint32_t)want});
        }
    }
    if ((int64_t)moves.size() > jobs->capacity)
        return fail(ATLAS_EINVAL, "jobs capacity %d < %zu moves", jobs->capacity, moves.size());
    if (!moves.empty() && (!jobs->demote_src || !jobs->demote_dst))
        return fail(ATLAS_EINVAL, "NULL demote arrays");
    std::vector<std::pair<int, int32_t>> taken;  // (tier, slot) taken in this plan
    for (Move &m : moves) {
        int tier = (int)m.to;
        while (tier != -1 && rt->pool(tier).empty()) {  // fall through to colder tiers
            tier = tier == kTierF8   ? kTierI8
                   : tier == kTierI8 ? kTierI4
                   : tier == kTierI4 && rt->cfg.num_int2 > 0 ? kTierI2
                   : (tier == kTierI4 || tier == kTierI2) && rt->cfg.num_1bit > 0 ? kTierB1
                                     : -1;
            // a fallback must still be colder than where the page is now
            if (tier != -1 && coldness(tier) <= coldness(class_of(m.from))) tier = -1;
        }
        if (tier == -1) {
            for (auto &t : taken) rt->pool(t.first).give(t.second);
            ++rt->st.capacity_failures;
            return fail(ATLAS_ECAPACITY, "cold pools full (sequence %d page %d)", m.seq,
                        m.page);
        }
        const int32_t slot = rt->pool(tier).take();
        taken.push_back({tier, slot});
        m.to = entry(tier, slot);
    }
    // commit: entries change now, the old blocks / slots are freed only after
    // every destination was taken, so no job writes what another reads
    int32_t n = 0;
    for (const Move &m : moves) {
        rt->seqs[m.seq].pages[m.page] = m.to;
        jobs->demote_src[n] = (int32_t)m.from;
        jobs->demote_dst[n] = (int32_t)m.to;
        ++n;
        if (class_of(m.from) == kTierHot) ++rt->st.demotions;
        else ++rt->st.transcodes;
    }
    for (const Move &m : moves) rt->pool(class_of(m.from)).give(slot_of(m.from));
    jobs->n_demote = n;
    return atlas::report_ok();
}

atlas_status atlas_residency_tables(atlas_residency *rt, const int32_t *seqs, int32_t n,
                                    int32_t *page_table, int32_t *context_lens,
                                    int32_t *regen_pages) {
    return fill_tables(rt, seqs, n, page_table, context_lens, regen_pages, nullptr);
}

atlas_status atlas_residency_tables_transient(atlas_residency *rt, const int32_t *seqs,
                                              int32_t n, int32_t *page_table,
                                              int32_t *context_lens, int32_t *regen_pages,
                                              atlas_residency_jobs *jobs) {
    if (!jobs) return fail(ATLAS_EINVAL, "jobs is NULL");
    return fill_tables(rt, seqs, n, page_table, context_lens, regen_pages, jobs);
}

atlas_status atlas_residency_get_stats(const atlas_residency *rt, atlas_residency_stats *out) {
    if (!rt || !out) return fail(ATLAS_EINVAL, "runtime or out is NULL");
    if (out->struct_size != sizeof(atlas_residency_stats))
        return fail(ATLAS_EINVAL, "stats->struct_size %u != %zu", out->struct_size,
                    sizeof(atlas_residency_stats));
    *out = rt->st;
    int32_t seqs = 0, regen = 0;
    for (const Seq &s : rt->seqs) {
        if (!s.active) continue;
        ++seqs;
        if (rt->cfg.mode == ATLAS_RESIDENCY_REGEN) regen += s.first_resident;
    }
    out->sequences = seqs;
    out->regenerated_pages = regen;
    out->hot_used = rt->hot.used();
    out->fp8_used = rt->f8.used();
    out->int8_used = rt->i8.used();
    out->int4_used = rt->i4.used();
    out->int2_used = rt->i2.used();
    out->archive_used = rt->b1.used();
    return atlas::report_ok();
}

}  // extern "C"
