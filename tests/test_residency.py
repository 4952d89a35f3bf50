"""CPU tests of the host residency runtime (include/atlas_residency.h): the
CFR KeepRecent / hot-cache / admission policy and the ARGUS sink / window /
cascade policy, through the C ABI.  No GPU: the runtime is host code."""

import numpy as np
import pytest

import oracle
from kv_cache_runtime_amd import atlas
from kv_cache_runtime_amd.residency import REGEN, TIERED, Residency

TIER = lambda e: (int(e) & 0xFFFFFFFF) >> 30  # noqa: E731
SLOT = lambda e: int(e) & ((1 << 30) - 1)  # noqa: E731


def _regen(**kw):
    cfg = dict(mode=REGEN, page_tokens=16, max_seqs=4, max_pages_per_seq=64, hot_blocks=8,
               recent_tokens=64)
    cfg.update(kw)
    return Residency(**cfg)


def _tiered(**kw):
    cfg = dict(mode=TIERED, page_tokens=16, max_seqs=4, max_pages_per_seq=64, hot_blocks=32,
               recent_tokens=64, sink_tokens=16, fp8_pages=2, int8_pages=3, num_fp8=16,
               num_int8=16, num_int4=64)
    cfg.update(kw)
    return Residency(**cfg)


def test_config_is_checked():
    for bad in (dict(mode=7), dict(page_tokens=0), dict(hot_blocks=-1), dict(recent_tokens=-1),
                dict(max_seqs=0), dict(num_int4=-3)):
        with pytest.raises(atlas.AtlasError) as e:
            _tiered(**bad)
        assert e.value.status == atlas.EINVAL


def test_regen_keep_recent_and_long_prompt():
    r = _regen()
    r.add_seq(0)
    r.append(0, 200)  # 13 pages; window = newest 64 tokens = pages 8..12
    table, ctx, regen = r.tables([0])
    assert ctx[0] == 200 and regen[0] == 8
    blocks = table[0, 8:13]
    assert len(set(blocks.tolist())) == 5 and blocks.max() < 8
    assert (table[0, :8] == 8).all() and (table[0, 13:] == 8).all()  # no block there
    assert r.stats()["hot_used"] == 5 and r.stats()["regenerated_pages"] == 8


def test_regen_window_slides_and_lru_evicts_oldest_cached_page():
    r = _regen()
    r.add_seq(0)
    r.append(0, 200)
    r.append(0, 64)   # 17 pages, window 12..16: needs 4 blocks, 3 free -> one eviction
    table, ctx, regen = r.tables([0])
    assert regen[0] == 9 and r.stats()["evictions"] == 1 and r.stats()["hot_used"] == 8
    assert len(set(table[0, 9:17].tolist())) == 8


def test_regen_lru_picks_least_recently_used_sequence():
    r = _regen(hot_blocks=12)
    for s in (0, 1):
        r.add_seq(s)
        r.append(s, 64)          # 4 pages each, all in the window
        r.append(s, 32)          # window moves: pages 0, 1 now cached outside it
    r.tables([0])                # sequence 0 used last
    r.add_seq(2)
    r.append(2, 32)              # 2 pages: 12 blocks all in use -> evict 2
    # the victims are sequence 1's cached pages (least recently used), oldest first
    _, _, regen = r.tables([0, 1, 2])
    assert regen.tolist() == [0, 2, 0] and r.stats()["evictions"] == 2
    r.append(2, 64)              # 4 more pages: sequence 0 (now least recent) gives its 2
    _, _, regen = r.tables([0, 1, 2])  # cached pages, then sequence 2 its own 2
    assert regen.tolist() == [2, 2, 2] and r.stats()["evictions"] == 6
    with pytest.raises(atlas.AtlasError):
        r.append(2, 200)         # nothing evictable is left for this much


def test_regen_capacity_failure_changes_nothing():
    r = _regen(hot_blocks=4)
    r.add_seq(0)
    r.append(0, 64)
    before = r.tables([0])
    with pytest.raises(atlas.AtlasError) as e:
        r.append(0, 8)           # 72 keys: the newest 64 span 5 pages, 4 blocks
    assert e.value.status == atlas.ECAPACITY
    after = r.tables([0])
    assert all(np.array_equal(a, b) for a, b in zip(before, after))
    assert r.stats()["capacity_failures"] == 1


def test_regen_admission_fills_free_blocks_most_recent_first():
    r = _regen(hot_blocks=16, admit_per_plan=3)
    for s in (0, 1):
        r.add_seq(s)
        r.append(s, 160)         # 10 pages, 4 resident, 6 regenerated
    r.tables([1])                # sequence 1 most recent
    src, dst, pages, blocks = r.plan()
    assert len(src) == 0 and pages.tolist() == [5, 4, 3]
    _, _, regen = r.tables([0, 1])
    assert regen.tolist() == [6, 3]
    assert len(set(blocks.tolist())) == 3 and r.stats()["admissions"] == 3


def _tiers(r, seq=0):
    table, ctx, _ = r.tables([seq])
    n = -(-int(ctx[0]) // 16)
    return [TIER(e) for e in table[0, :n]], table[0, :n]


def test_tiered_targets_by_position():
    r = _tiered()
    r.add_seq(0)
    r.append(0, 400)             # 25 pages, window 21..24, sink page 0
    src, dst, _, _ = r.plan()
    tiers, _ = _tiers(r)
    want = [0] + [2] * 15 + [1] * 3 + [3] * 2 + [0] * 4
    assert tiers == want
    assert all(TIER(e) == 0 for e in src) and len(src) == 20
    assert len(set(dst.tolist())) == 20
    st = r.stats()
    assert st["hot_used"] == 5 and st["fp8_used"] == 2 and st["int8_used"] == 3
    assert st["int4_used"] == 15 and st["demotions"] == 20


def test_tiered_cascade_step_transcodes_and_never_reuses_within_a_plan():
    # one slot of headroom per tier: a slot freed by a plan returns to its
    # pool only after the plan
    r = _tiered(num_fp8=3, num_int8=4)
    r.add_seq(0)
    r.append(0, 400)
    r.plan()
    r.append(0, 16)              # window 22..25: page 21 -> FP8, 19 -> INT8, 16 -> INT4
    src, dst, _, _ = r.plan()
    assert sorted((TIER(s), TIER(d)) for s, d in zip(src, dst)) == [(0, 3), (1, 2), (3, 1)]
    # a slot freed by one job is not the destination of another in the same plan
    assert not {(TIER(e), SLOT(e)) for e in src} & {(TIER(e), SLOT(e)) for e in dst}
    tiers, _ = _tiers(r)
    assert tiers == [0] + [2] * 16 + [1] * 3 + [3] * 2 + [0] * 4
    assert r.stats()["transcodes"] == 2


def test_tiered_full_pools_fall_through_then_fail_unchanged():
    r = _tiered(num_fp8=1, num_int8=1, num_int4=64)
    r.add_seq(0)
    r.append(0, 400)
    r.plan()
    tiers, _ = _tiers(r)
    assert tiers == [0] + [2] * 18 + [1] + [3] + [0] * 4   # FP8 and INT8 hold one page each
    r2 = _tiered(num_fp8=0, num_int8=0, num_int4=3)
    r2.add_seq(0)
    r2.append(0, 400)
    before = r2.tables([0])
    with pytest.raises(atlas.AtlasError) as e:
        r2.plan()
    assert e.value.status == atlas.ECAPACITY
    assert all(np.array_equal(a, b) for a, b in zip(before, r2.tables([0])))
    assert r2.stats()["int4_used"] == 0


def test_tiered_hot_pool_exhaustion_and_remove_frees_everything():
    r = _tiered(hot_blocks=6)
    r.add_seq(0)
    with pytest.raises(atlas.AtlasError) as e:
        r.append(0, 7 * 16)      # 7 pages before any plan
    assert e.value.status == atlas.ECAPACITY
    r.append(0, 6 * 16)          # window 2..5 and sink page 0 hot; page 1 -> FP8
    r.plan()
    r.add_seq(1)
    r.append(1, 16)              # the block page 1 left
    assert r.stats()["hot_used"] == 6 and r.stats()["fp8_used"] == 1
    r.remove_seq(0)
    st = r.stats()
    assert st["sequences"] == 1 and st["hot_used"] == 1 and st["fp8_used"] == 0
    with pytest.raises(atlas.AtlasError):
        r.tables([0])


def test_bad_calls_are_rejected():
    r = _tiered()
    with pytest.raises(atlas.AtlasError):
        r.append(0, 5)           # not active
    r.add_seq(0)
    with pytest.raises(atlas.AtlasError):
        r.add_seq(0)             # already active
    with pytest.raises(atlas.AtlasError):
        r.add_seq(9)             # out of range
    with pytest.raises(atlas.AtlasError):
        r.append(0, 64 * 16 + 1)  # past max_pages_per_seq


def test_tiered_without_headroom_falls_through_to_colder_tiers():
    # exactly full FP8 / INT8 pools: the slots freed by this plan's moves are
    # not reused within it, so the moved pages go one tier colder
    r = _tiered(num_fp8=2, num_int8=3)
    r.add_seq(0)
    r.append(0, 400)
    r.plan()
    r.append(0, 16)
    src, dst, _, _ = r.plan()
    assert sorted((TIER(s), TIER(d)) for s, d in zip(src, dst)) == [(0, 2), (1, 2), (3, 2)]


def test_tiered_cascade_ends_in_int2_when_it_has_a_pool():
    r = _tiered(int4_pages=4, num_int2=32)
    r.add_seq(0)
    r.append(0, 400)             # 25 pages, window 21..24, sink page 0
    r.plan()
    table, ctx, _ = r.tables([0])
    cls = [oracle.entry_class(e)[0] for e in table[0, :25]]
    # newest cold first: 2 FP8, 3 INT8, 4 INT4, the rest (pages 1..11) INT2
    assert cls == [0] + [4] * 11 + [2] * 4 + [1] * 3 + [3] * 2 + [0] * 4
    st = r.stats()
    assert st["int2_used"] == 11 and st["int4_used"] == 4
    r.append(0, 16)
    src, dst, _, _ = r.plan()
    moves = sorted((oracle.entry_class(s)[0], oracle.entry_class(d)[0]) for s, d in zip(src, dst))
    assert moves == [(0, 3), (1, 2), (2, 4), (3, 1)]


def test_tiered_cascade_ends_in_the_1bit_archive():
    r = _tiered(int4_pages=4, num_int2=32, int2_pages=3, num_1bit=16, transient_blocks=16)
    r.add_seq(0)
    r.append(0, 400)             # 25 pages, window 21..24, sink page 0
    src, dst, _, _ = r.plan()
    assert sum(oracle.entry_class(d)[0] == 5 for d in dst) == 8
    table, ctx, _ = r.tables([0])
    cls = [oracle.entry_class(e)[0] for e in table[0, :25]]
    # newest cold first: 2 FP8, 3 INT8, 4 INT4, 3 INT2, the rest (pages 1..8) archived
    assert cls == [0] + [5] * 8 + [4] * 3 + [2] * 4 + [1] * 3 + [3] * 2 + [0] * 4
    assert r.stats()["archive_used"] == 8
    # without an INT2 pool the INT4 band comes last before the archive
    r2 = _tiered(int4_pages=4, int2_pages=3, num_1bit=16)
    r2.add_seq(0)
    r2.append(0, 400)
    r2.plan()
    t2, _, _ = r2.tables([0])
    assert [oracle.entry_class(e)[0] for e in t2[0, :25]] == (
        [0] + [5] * 11 + [2] * 4 + [1] * 3 + [3] * 2 + [0] * 4)


def test_transient_tables_rebuild_archived_pages():
    r = _tiered(int4_pages=4, num_int2=32, int2_pages=3, num_1bit=16, transient_blocks=16)
    for s in (0, 1):
        r.add_seq(s)
    r.append(0, 400)
    r.append(1, 60)              # no archived page
    r.plan()
    plain, _, _ = r.tables([1, 0])
    table, ctx, _, psrc, pdst = r.tables_transient([1, 0])
    assert list(ctx) == [60, 400]
    np.testing.assert_array_equal(table[0], plain[0])
    archived = [p for p in range(25) if oracle.entry_class(plain[1, p])[0] == 5]
    assert archived == list(range(1, 9))
    # the k-th archived page (sequence, then page order) gets block hot_blocks + k
    assert list(pdst) == list(range(32, 40))
    assert list(psrc) == [int(plain[1, p]) for p in archived]
    assert [int(table[1, p]) for p in archived] == list(range(32, 40))
    others = [p for p in range(25) if p not in archived]
    np.testing.assert_array_equal(table[1, others], plain[1, others])
    # past the context: the block the runtime never hands out
    assert set(table[1, 25:].tolist()) == {32 + 16} and set(table[0, 4:].tolist()) == {48}
    assert r.stats()["reconstructions"] == 8


def test_transient_capacity_failure_and_archive_fall_through():
    r = _tiered(int4_pages=4, num_int2=32, int2_pages=3, num_1bit=16, transient_blocks=5)
    r.add_seq(0)
    r.append(0, 400)
    r.plan()
    with pytest.raises(atlas.AtlasError) as e:
        r.tables_transient([0])
    assert e.value.status == atlas.ECAPACITY
    assert r.stats()["reconstructions"] == 0 and r.stats()["capacity_failures"] == 1
    table, _, _ = r.tables([0])           # the plain tables still work
    assert sum(oracle.entry_class(x)[0] == 5 for x in table[0, :25]) == 8
    # a full INT2 pool sends its band to the archive
    r3 = _tiered(int4_pages=4, num_int2=1, int2_pages=3, num_1bit=16)
    r3.add_seq(0)
    r3.append(0, 400)
    r3.plan()
    t3, _, _ = r3.tables([0])
    assert [oracle.entry_class(x)[0] for x in t3[0, 1:12]].count(4) == 1
    assert r3.stats()["archive_used"] == 10


def test_archive_config_is_checked():
    for bad in (dict(num_1bit=-1), dict(int2_pages=-2), dict(transient_blocks=-1),
                dict(num_1bit=(1 << 28) + 1)):
        with pytest.raises(atlas.AtlasError) as e:
            _tiered(**bad)
        assert e.value.status == atlas.EINVAL


# ---------------------------------------------------------------------------
# Hardening: finite-value validation before admission, global and per-layer
# budgets (CFR-Atlas README, hardening baseline and test list)
# ---------------------------------------------------------------------------

def test_refused_admission_goes_back_to_regeneration():
    r = _regen(hot_blocks=16, admit_per_plan=3)
    for s in (0, 1):
        r.add_seq(s)
        r.append(s, 160)         # 10 pages, 4 resident, 6 regenerated
    r.tables([1])
    _, _, pages, blocks = r.plan()
    assert pages.tolist() == [5, 4, 3]          # all for sequence 1
    used = r.stats()["hot_used"]
    # the regenerator found non-finite values in page 4's block: pages 4 and
    # 3 (admitted below it) go back; page 5 stays resident
    r.refuse_admissions(pages, blocks, [0, 7, 0])
    st = r.stats()
    assert st["refused_admissions"] == 2 and st["admissions"] == 1
    assert st["hot_used"] == used - 2
    table, _, regen = r.tables([0, 1])
    assert regen.tolist() == [6, 5]
    assert table[1, 5] == blocks[0]
    # a rejected job (-1) is refused too, and refusing nothing changes nothing
    _, _, pages, blocks = r.plan()
    assert pages.tolist() == [4, 3, 2]
    r.refuse_admissions(pages, blocks, [0, 0, 0])
    assert r.tables([1])[2].tolist() == [2]
    _, _, pages, blocks = r.plan()
    r.refuse_admissions(pages, blocks, [-1] * len(pages))
    assert r.tables([1])[2].tolist() == [2]


def test_refuse_checks_its_jobs_before_changing_anything():
    r = _regen(hot_blocks=16, admit_per_plan=2)
    r.add_seq(0)
    r.append(0, 160)
    _, _, pages, blocks = r.plan()
    before = r.stats()
    with pytest.raises(atlas.AtlasError) as e:
        r.refuse_admissions(pages, blocks[::-1].copy(), [1, 1])  # blocks do not match
    assert e.value.status == atlas.EINVAL
    assert r.stats() == before
    t = _tiered()
    t.add_seq(0)
    t.append(0, 10)
    with pytest.raises(atlas.AtlasError):
        t.refuse_admissions([0], [0], [1])  # no admissions in tiered mode


def test_shared_budget_caps_layers_together():
    from kv_cache_runtime_amd.residency import Budget
    b = Budget(10)
    layers = [_regen(hot_blocks=8, recent_tokens=64, budget=b) for _ in range(2)]
    for r in layers:
        r.add_seq(0)
    layers[0].append(0, 100)             # 7 pages: window 64 tokens -> 5 resident
    assert b.used == layers[0].stats()["hot_used"] == 7 - 2
    layers[1].append(0, 64)              # 4 pages, all in the window
    assert b.used == 9
    # layer 1 has 4 free blocks of its own, the shared budget only 1: the
    # layer evicts its own least recently used page outside its window
    layers[1].append(0, 32)              # 6 pages, window 64 tokens: pages 2..5
    assert b.used == 10 and layers[1].stats()["hot_used"] == 5
    with pytest.raises(atlas.AtlasError) as e:   # a sequence with no evictable page
        layers[1].add_seq(1)
        layers[1].append(1, 64)
    assert e.value.status == atlas.ECAPACITY
    assert b.used == 10
    # freeing a layer's pages returns them to the budget
    layers[0].remove_seq(0)
    assert b.used == 5
    layers[1].append(1, 64)  # 3 free blocks of its own, then its oldest evictable page
    assert b.used == 8 and layers[1].stats()["evictions"] == 2
    for r in layers:
        r.close()
    assert b.used == 0
    b.close()


def test_per_layer_budget_is_the_runtime_pool():
    from kv_cache_runtime_amd.residency import Budget
    b = Budget(1000)  # a global budget far above the layer's
    r = _regen(hot_blocks=4, recent_tokens=128, budget=b)
    r.add_seq(0)
    with pytest.raises(atlas.AtlasError) as e:
        r.append(0, 80)  # 5 pages in the window > 4 blocks
    assert e.value.status == atlas.ECAPACITY and b.used == 0
    r.append(0, 64)
    assert b.used == 4
    r.close()
    b.close()
