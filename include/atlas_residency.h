/*
 * atlas_residency.h - host residency runtime of libatlas.so: the policy layer
 * that decides, per sequence and logical page, whether a page is resident in
 * the hot pool, regenerated, or stored in a cold tier, and hands the
 * attention calls their page tables.
 *
 * Sources.  CFR-Atlas README: a bounded hot-page cache (byte budget, LRU
 * replacement), the KeepRecent { recent_tokens } policy, admission of
 * regenerated pages into the hot cache, runtime counters.  argus-cache,
 * "Visual Architecture" and its configuration (max_active_pages,
 * max_fp8_pages, sink_tokens): an FP16 active pool for recent pages, the
 * compression cascade FP8 -> INT8 -> INT4 -> INT2 -> 1-bit for older ones,
 * attention sinks that stay in FP16, and the transient FP16 reconstruction of
 * archived pages when a query needs them.
 *
 * The runtime is plain host code: it reads and writes no device memory and
 * launches nothing.  It hands out block and slot numbers of pools the caller
 * owns, and describes the device work a step needs as job lists that the
 * caller runs with atlas_demote_pages / atlas_regenerate_pages.  Contract:
 * run the jobs of a plan on the stream before any later write into the pools
 * (atlas_write_kv) or later plan's jobs; then stream order keeps every block
 * a job reads intact until the job has read it.  A handle is not
 * thread-safe: one host thread at a time.
 *
 * A decode step with the runtime:
 *   1. atlas_residency_append(seq, n) for each sequence that grows (new
 *      pages get hot blocks);
 *   2. atlas_residency_tables -> page table, context lengths, regenerated
 *      page counts for the attention call (with a 1-bit archive:
 *      atlas_residency_tables_transient, then atlas_promote_pages on its
 *      jobs); atlas_write_kv the new tokens;
 *   3. the attention call;
 *   4. atlas_residency_plan -> demotions (tiered) or admissions (regen);
 *      run them (atlas_demote_pages, atlas_regenerate_pages with its
 *      non-finite counts), then hand the counts to
 *      atlas_residency_refuse_admissions.
 */
#ifndef ATLAS_RESIDENCY_H
#define ATLAS_RESIDENCY_H

#include "atlas.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Residency modes. */
#define ATLAS_RESIDENCY_REGEN 0  /* CFR: pages outside the hot set are regenerated
                                    (atlas_paged_attention_regen) */
#define ATLAS_RESIDENCY_TIERED 1 /* ARGUS: pages outside the hot set move down the
                                    cascade (atlas_paged_attention_tiered) */

typedef struct atlas_residency_config {
    uint32_t struct_size;      /* = sizeof(atlas_residency_config) */
    int32_t mode;              /* ATLAS_RESIDENCY_REGEN or _TIERED */
    int32_t page_tokens;       /* tokens per page, >= 1 (the attention calls' page_tokens) */
    int32_t max_seqs;          /* sequence ids are 0 .. max_seqs - 1 */
    int32_t max_pages_per_seq; /* row length of the page tables it fills */
    int32_t hot_blocks;        /* hot pool blocks it may hand out: blocks 0 .. hot_blocks - 1
                                  (the CFR hot-cache byte budget divided by the bytes of
                                  one block) */
    int32_t recent_tokens;     /* KeepRecent: pages holding any of the newest
                                  recent_tokens keys stay hot, >= 0 */
    int32_t sink_tokens;       /* tiered: pages holding any of the first sink_tokens keys
                                  stay hot, >= 0 */
    int32_t admit_per_plan;    /* regen: regenerated pages admitted into free hot blocks
                                  per plan (0 = no admission), >= 0 */
    int32_t fp8_pages;         /* tiered: per sequence, the newest cold pages kept in FP8 */
    int32_t int8_pages;        /* tiered: the next this many cold pages in INT8; older
                                  pages INT4 */
    int32_t num_fp8;           /* tiered: cold pool capacities in slots (slots 0 .. n-1) */
    int32_t num_int8;
    int32_t num_int4;
    int32_t int4_pages;        /* tiered, with num_int2 > 0: the next this many cold pages
                                  in INT4, older pages INT2 */
    int32_t num_int2;          /* tiered: INT2 pool capacity (0: INT4 is the last tier) */
    int32_t int2_pages;        /* tiered, with num_1bit > 0: the next this many cold pages
                                  in INT2 (or INT4 without an INT2 pool); older pages go to
                                  the 1-bit archive */
    int32_t num_1bit;          /* tiered: 1-bit archive capacity in slots (0: no archive) */
    int32_t transient_blocks;  /* tiered: hot blocks hot_blocks .. hot_blocks +
                                  transient_blocks - 1, reserved for archived pages rebuilt
                                  for one attention call (atlas_residency_tables_transient) */
    struct atlas_residency_budget *budget; /* optional shared (global) budget: hot blocks
                                  that all runtimes naming it may hold together, or NULL.
                                  A runtime serves one layer, so hot_blocks is that
                                  layer's budget (CFR-Atlas README, test list: global and
                                  per-layer budgets) */
} atlas_residency_config;

typedef struct atlas_residency_stats {
    uint32_t struct_size;      /* = sizeof(atlas_residency_stats) */
    int32_t sequences;         /* active sequences */
    int32_t hot_used;          /* hot blocks in use */
    int32_t fp8_used;          /* cold slots in use, per tier */
    int32_t int8_used;
    int32_t int4_used;
    int32_t int2_used;
    int32_t regenerated_pages; /* regen: pages now served by regeneration */
    int64_t appended_tokens;   /* counters since creation */
    int64_t demotions;         /* jobs whose source was a hot block */
    int64_t transcodes;        /* jobs whose source was a cold slot */
    int64_t admissions;        /* regenerated pages admitted into the hot pool */
    int64_t evictions;         /* resident pages dropped back to regeneration (LRU) */
    int64_t capacity_failures; /* calls refused with ATLAS_ECAPACITY */
    int64_t archive_used;      /* 1-bit archive slots in use */
    int64_t reconstructions;   /* promotion jobs handed out by tables_transient */
    int64_t refused_admissions; /* admitted pages taken back by
                                   atlas_residency_refuse_admissions */
} atlas_residency_stats;

/* Job lists filled by atlas_residency_plan.  The caller provides the arrays
 * (host memory, `capacity` entries each). */
typedef struct atlas_residency_jobs {
    uint32_t struct_size;      /* = sizeof(atlas_residency_jobs) */
    int32_t capacity;          /* entries each array can hold */
    int32_t n_demote;          /* out: jobs for atlas_demote_pages */
    int32_t n_admit;           /* out: jobs for atlas_regenerate_pages */
    int32_t *demote_src;       /* source entries (tier << 30) | slot */
    int32_t *demote_dst;       /* destination entries */
    int32_t *admit_page;       /* logical page to regenerate ... */
    int32_t *admit_block;      /* ... into this hot block */
    int32_t n_promote;         /* out: jobs for atlas_promote_pages (tables_transient) */
    int32_t reserved;          /* 0 */
    int32_t *promote_src;      /* archived entries ... */
    int32_t *promote_dst;      /* ... rebuilt into these transient hot blocks */
} atlas_residency_jobs;

typedef struct atlas_residency atlas_residency; /* opaque */
typedef struct atlas_residency_budget atlas_residency_budget; /* opaque */

/* A shared budget of `blocks` hot blocks (host memory only).  Runtimes that
 * name it in their config take a hot block only while it has room; blocks
 * return to it when freed or when their runtime is destroyed.  Destroy the
 * runtimes before their budget.  Runtimes sharing a budget are used from one
 * host thread at a time. */
atlas_status atlas_residency_budget_create(int64_t blocks, atlas_residency_budget **out);
atlas_status atlas_residency_budget_destroy(atlas_residency_budget *budget);
/* Hot blocks currently held by the runtimes that share the budget. */
atlas_status atlas_residency_budget_used(const atlas_residency_budget *budget, int64_t *used);

/* Creates a runtime (host memory only).  Checks every field; *out is set on
 * success only. */
atlas_status atlas_residency_create(const atlas_residency_config *config,
                                    atlas_residency **out);

/* Frees the runtime (NULL is allowed). */
atlas_status atlas_residency_destroy(atlas_residency *rt);

/* Starts sequence `seq` (0 <= seq < max_seqs, not active) with no tokens. */
atlas_status atlas_residency_add_seq(atlas_residency *rt, int32_t seq);

/* Ends sequence `seq`: its blocks and slots return to the pools (their
 * contents are not touched). */
atlas_status atlas_residency_remove_seq(atlas_residency *rt, int32_t seq);

/* Grows `seq` by n_tokens >= 0 keys; every new page gets a hot block.  Regen
 * mode: while the sequence has no resident page, its new pages in front of
 * its KeepRecent window start out regenerated (a long prompt's early pages
 * take no block); when no block is free, the least recently used sequence's
 * oldest resident page outside its KeepRecent window goes back to
 * regeneration (LRU).  Fails with ATLAS_ECAPACITY, changing nothing, when the pool cannot
 * hold the new pages, or with ATLAS_EINVAL past max_pages_per_seq pages. */
atlas_status atlas_residency_append(atlas_residency *rt, int32_t seq, int32_t n_tokens);

/* Applies the policy to every active sequence and fills `jobs`.  Tiered mode:
 * each page's target is hot for sink and KeepRecent pages; counting back
 * from the window, fp8_pages FP8 pages, then int8_pages INT8 pages, then
 * INT4 (with an INT2 pool: int4_pages INT4 pages, then INT2; with a 1-bit
 * archive the last of these bands is int4_pages or int2_pages long and the
 * rest is archived); a full pool falls through to the next colder tier.
 * Archiving jobs have 1-bit destinations (atlas_demote_pages).  Each page that
 * is hotter than its target gets one job (its current entry -> a new slot of
 * the target tier); its old block or slot is freed after the plan, so no
 * job of a plan writes where another reads (give each cold pool headroom of
 * one plan's moves, or moved pages fall through to a colder tier).  Regen mode: up to
 * admit_per_plan regenerated pages just before a resident run (most recently
 * used sequences first) get free hot blocks as admission jobs.  Fails with
 * ATLAS_ECAPACITY (every cold pool full) or ATLAS_EINVAL (jobs capacity too
 * small), changing nothing.  n_promote is set to 0. */
atlas_status atlas_residency_plan(atlas_residency *rt, atlas_residency_jobs *jobs);

/* Host arrays for an attention call over the sequences seqs[0..n-1]:
 * page_table [n][max_pages_per_seq] (hot block ids, or tiered entries in
 * tiered mode; entries of regenerated pages and past the context name block
 * hot_blocks + transient_blocks, which the runtime never hands out: with a
 * pool of exactly that many blocks atlas_write_kv skips rows of such pages;
 * archived pages keep their 1-bit entries, which attention refuses),
 * context_lens [n], regen_pages [n] (regen mode; may be NULL otherwise).
 * Marks the sequences as used (LRU). */
atlas_status atlas_residency_tables(atlas_residency *rt, const int32_t *seqs, int32_t n,
                                    int32_t *page_table, int32_t *context_lens,
                                    int32_t *regen_pages);

/* atlas_residency_tables plus the transient reconstruction of archived
 * pages: the k-th 1-bit page of the listed sequences (in sequence, then page
 * order) is given transient block hot_blocks + k in page_table, and jobs gets
 * the promotion (promote_src = its 1-bit entry, promote_dst = that block) for
 * atlas_promote_pages, to run before the attention call.  The transient
 * blocks hold these pages until the next tables_transient call.  jobs
 * (capacity >= the archived pages) is required; its n_demote and n_admit are
 * set to 0.  Fails with ATLAS_ECAPACITY when the archived pages outnumber
 * transient_blocks, or ATLAS_EINVAL for a small jobs capacity; the runtime
 * is then unchanged and the outputs are unspecified. */
atlas_status atlas_residency_tables_transient(atlas_residency *rt, const int32_t *seqs,
                                              int32_t n, int32_t *page_table,
                                              int32_t *context_lens, int32_t *regen_pages,
                                              atlas_residency_jobs *jobs);

/* Finite-value validation before admission (CFR-Atlas README, hardening
 * baseline).  Regen mode, right after the admission jobs of the last
 * atlas_residency_plan ran through atlas_regenerate_pages with its
 * `nonfinite` output copied back to the host: every job j with
 * nonfinite[j] != 0 (non-finite values stored, or -1: the job was rejected)
 * is taken back -- its page is regenerated again and its block freed -- and
 * so are the pages the same plan admitted below it in that sequence (the
 * resident pages stay a suffix).  Call it before the next tables call.
 * Fails with ATLAS_EINVAL, changing nothing, when a job is not a current
 * admission. */
atlas_status atlas_residency_refuse_admissions(atlas_residency *rt,
                                               const atlas_residency_jobs *jobs,
                                               const int32_t *nonfinite);

/* Current counters. */
atlas_status atlas_residency_get_stats(const atlas_residency *rt, atlas_residency_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* ATLAS_RESIDENCY_H */
