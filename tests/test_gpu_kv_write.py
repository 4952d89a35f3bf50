"""GPU checks of the KV write path through the C ABI: writing new tokens'
K/V into their pages (bit-exact placement, then attention on the updated
cache against the oracle) and demoting hot pages into the int8 / int4 tiers
(codes and scales bit-exact against the oracle's encoder, then tiered
attention on the demoted pages against the oracle)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from tests.test_gpu_parity import check, run

pytestmark = pytest.mark.gpu


def _row_positions(w):
    """(seq, own key position) of every query row."""
    out = []
    for s in range(w.num_seqs):
        n_q, c = int(w.query_lens[s]), int(w.context_lens[s])
        out += [(s, c - n_q + t) for t in range(n_q)]
    return out


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("kv,prefill", [("bf16", False), ("f16", False), ("f32", False),
                                        ("bf16", True)])
def test_write_kv_places_rows_and_attention_sees_them(gpu, kv, prefill):
    spec = dict(num_seqs=3, context_lens=[40, 300, 1025], num_heads=8, num_kv_heads=2,
                head_dim=128 if kv != "f32" else 64, page_tokens=16, kv_dtype=kv,
                placement="permuted")
    if prefill:
        spec["query_lens"] = [7, 16, 33]
    w = synth.build(spec, device=gpu, seed=77, name=f"write-{kv}-{prefill}")
    gen = torch.Generator(device=gpu).manual_seed(5)
    shape = (w.total_q, w.num_kv_heads, w.head_dim)
    k_new = torch.randn(shape, generator=gen, device=gpu).to(w.k_pool.dtype)
    v_new = torch.randn(shape, generator=gen, device=gpu).to(w.v_pool.dtype)
    k_before, v_before = w.k_pool.clone(), w.v_pool.clone()
    prob = atlas.Problem(w)
    atlas.atlas_write_kv(prob.args, k_new, v_new)
    torch.cuda.synchronize()

    # placement: every row's own key holds its new K/V; nothing else changed
    touched = torch.zeros(w.k_pool.shape[:3], dtype=torch.bool, device=gpu)
    for row, (s, pos) in enumerate(_row_positions(w)):
        blk, r = int(w.page_table[s, pos // w.page_tokens]), pos % w.page_tokens
        assert torch.equal(_bits(w.k_pool[blk, :, r]), _bits(k_new[row]))
        assert torch.equal(_bits(w.v_pool[blk, :, r]), _bits(v_new[row]))
        touched[blk, :, r] = True
    keep = ~touched
    for after, before in ((w.k_pool, k_before), (w.v_pool, v_before)):
        a, b = _bits(after)[keep], _bits(before)[keep]
        assert torch.equal(a, b)
    out, lse = run(w)
    check(w, out, lse)


def test_write_kv_skips_invalid_blocks(gpu):
    w = synth.build(dict(num_seqs=2, context_lens=[20, 50], num_heads=4, num_kv_heads=2,
                         head_dim=64, page_tokens=16, kv_dtype="bf16"), device=gpu, seed=3)
    prob = atlas.Problem(w)
    prob.table[1, 50 // 16] = w.num_blocks + 5   # the last page of seq 1 names no block
    before = w.k_pool.clone()
    k_new = torch.ones((2, 2, 64), dtype=torch.bfloat16, device=gpu)
    atlas.atlas_write_kv(prob.args, k_new, k_new)
    torch.cuda.synchronize()
    blk0 = int(w.page_table[0, 19 // 16])
    assert torch.equal(w.k_pool[blk0, :, 19 % 16], k_new[0])
    changed = (_bits(w.k_pool) != _bits(before)).any(dim=-1)
    assert int(changed.sum()) == 2   # seq 0's row only, both kv heads


def _demote_case(gpu, hot_dtype, seed):
    w = synth.build(dict(num_seqs=3, context_lens=[700, 1300, 2100], num_heads=8,
                         num_kv_heads=2, head_dim=128, page_tokens=16, q_dtype="bf16",
                         kv_dtype=hot_dtype, placement="permuted",
                         tiers=dict(hot_tokens=600, p_int8=0.5)),
                    device=gpu, seed=seed, name=f"demote-{hot_dtype}")
    return w


@pytest.mark.parametrize("hot_dtype", ["f16", "bf16"])
def test_demote_pages_bit_exact_and_attention(gpu, hot_dtype):
    w = _demote_case(gpu, hot_dtype, seed=11)
    Hkv, P, D = w.num_kv_heads, w.page_tokens, w.head_dim
    # full hot pages of sequence 2 (not its last page): demote half to int8,
    # half to int4, into fresh slots appended to the cold pools
    s = 2
    ctx = int(w.context_lens[s])
    ent = w.page_table[s].view(np.uint32)
    pages = [p for p in range(ctx // P) if (int(ent[p]) >> 30) == 0][:6]
    assert len(pages) == 6
    counts = w.tiers["counts"]
    n8, n4 = w.tiers["i8_k"].shape[0], w.tiers["i4_k"].shape[0]
    for key, extra in (("i8", 3), ("i4", 3)):
        for kv in ("k", "v"):
            t = w.tiers[f"{key}_{kv}"]
            w.tiers[f"{key}_{kv}"] = torch.cat([t, torch.zeros((extra,) + t.shape[1:],
                                                               dtype=t.dtype, device=gpu)])
            sc = w.tiers[f"{key}_{kv}_scale"]
            w.tiers[f"{key}_{kv}_scale"] = torch.cat(
                [sc, torch.full((extra, Hkv), -1.0, device=gpu)])
    src = [int(ent[p]) & ((1 << 30) - 1) for p in pages]
    dst = [(1 << 30) | (n8 + i) for i in range(3)] + [(2 << 30) | (n4 + i) for i in range(3)]
    prob = atlas.Problem(w)
    src_t = torch.tensor(src, dtype=torch.int32, device=gpu)
    dst_t = torch.tensor(np.array(dst, dtype=np.uint32).view(np.int32), device=gpu)
    rejected = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_demote_pages(prob.args, prob.tiers, src_t, dst_t, rejected)
    torch.cuda.synchronize()
    assert int(rejected) == 0

    host = oracle.HostView(w)
    (ka, kind), (va, _) = host.pools()
    ta = host.tier_arrays()
    for i, (b, e) in enumerate(zip(src, dst)):
        tier, slot = e >> 30, e & ((1 << 30) - 1)
        key, qmax = ("i8", 127) if tier == 1 else ("i4", 7)
        for arr, kv in ((ka, "k"), (va, "v")):
            for g in range(Hkv):
                x = oracle.widen_bits(arr[b, g], kind).astype(np.float32)
                codes, scale = oracle.quantize_block(x, qmax)
                got_scale = np.float32(ta[f"{key}_{kv}_scale"][slot, g])
                assert got_scale.tobytes() == scale.tobytes(), (i, kv, g)
                want = codes.astype(np.int8) if tier == 1 else oracle.pack_int4(codes)
                got = ta[f"{key}_{kv}"][slot, g]
                assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (i, kv, g)

    # point the pages at their cold copies and attend
    new_ent = ent.copy()
    for p, e in zip(pages, dst):
        new_ent[p] = e
    w.page_table[s] = new_ent.view(np.int32)
    prob.table[s] = torch.from_numpy(w.page_table[s].copy()).to(gpu)
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("hot_dtype", ["f16", "bf16"])
def test_demote_block_with_non_finite_value_gets_nan_scale(gpu, hot_dtype):
    """A hot block holding a NaN (or an infinity) is demoted to a NaN scale
    with codes 0 -- every value read back is NaN -- while the other blocks of
    the same pages encode as usual; codes and scales match the oracle's
    encoder, NaN for NaN."""
    w = _demote_case(gpu, hot_dtype, seed=13)
    Hkv, P = w.num_kv_heads, w.page_tokens
    s = 2
    ctx = int(w.context_lens[s])
    ent = w.page_table[s].view(np.uint32)
    pages = [p for p in range(ctx // P) if (int(ent[p]) >> 30) == 0][:2]
    assert len(pages) == 2
    src = [int(ent[p]) & ((1 << 30) - 1) for p in pages]
    w.k_pool[src[0], 0, 3, 17] = float("nan")
    w.v_pool[src[1], Hkv - 1, 5, 2] = float("inf")
    n8, n4 = w.tiers["i8_k"].shape[0], w.tiers["i4_k"].shape[0]
    for key in ("i8", "i4"):
        for kv in ("k", "v"):
            t = w.tiers[f"{key}_{kv}"]
            w.tiers[f"{key}_{kv}"] = torch.cat([t, torch.zeros((1,) + t.shape[1:],
                                                               dtype=t.dtype, device=gpu)])
            sc = w.tiers[f"{key}_{kv}_scale"]
            w.tiers[f"{key}_{kv}_scale"] = torch.cat([sc, torch.full((1, Hkv), -1.0, device=gpu)])
    dst = [(1 << 30) | n8, (2 << 30) | n4]
    prob = atlas.Problem(w)
    atlas.atlas_demote_pages(prob.args, prob.tiers, torch.tensor(src, dtype=torch.int32,
                                                                 device=gpu),
                             torch.tensor(np.array(dst, dtype=np.uint32).view(np.int32),
                                          device=gpu))
    torch.cuda.synchronize()
    host = oracle.HostView(w)
    (ka, kind), (va, _) = host.pools()
    ta = host.tier_arrays()
    nan_blocks = 0
    for b, e in zip(src, dst):
        tier, slot = e >> 30, e & ((1 << 30) - 1)
        key, qmax = ("i8", 127) if tier == 1 else ("i4", 7)
        for arr, kv in ((ka, "k"), (va, "v")):
            for g in range(Hkv):
                x = oracle.widen_bits(arr[b, g], kind).astype(np.float32)
                codes, scale = oracle.quantize_block(x, qmax)
                got_scale = np.float32(ta[f"{key}_{kv}_scale"][slot, g])
                if np.isnan(scale):
                    nan_blocks += 1
                    assert np.isnan(got_scale), (b, kv, g)
                else:
                    assert got_scale.tobytes() == scale.tobytes(), (b, kv, g)
                want = codes.astype(np.int8) if tier == 1 else oracle.pack_int4(codes)
                got = ta[f"{key}_{kv}"][slot, g]
                assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (b, kv, g)
    assert nan_blocks == 2


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_demote_cold_source_with_non_finite_scale(gpu, bad):
    """A cold source block whose scale is NaN or infinite reads back as
    non-finite values, so moving it down the cascade (int8 -> int4) gives a
    NaN scale and codes 0, like a hot block holding them; the block's other
    (kv, kv head) blocks encode as usual.  Expected values: the oracle's
    encoder on the oracle's reading of the source."""
    w = _demote_case(gpu, "bf16", seed=14)
    Hkv = w.num_kv_heads
    s = 2
    ent = w.page_table[s].view(np.uint32)
    n_full = int(w.context_lens[s]) // w.page_tokens
    src = [int(e) for e in ent[:n_full] if (int(e) >> 30) == 1][0]
    w.tiers["i8_k_scale"][src & ((1 << 30) - 1), 1] = bad
    n4 = w.tiers["i4_k"].shape[0]
    for kv in ("k", "v"):
        t = w.tiers[f"i4_{kv}"]
        w.tiers[f"i4_{kv}"] = torch.cat([t, torch.zeros((1,) + t.shape[1:], dtype=t.dtype,
                                                        device=gpu)])
        sc = w.tiers[f"i4_{kv}_scale"]
        w.tiers[f"i4_{kv}_scale"] = torch.cat([sc, torch.full((1, Hkv), -1.0, device=gpu)])
    dst = (2 << 30) | n4
    host = oracle.HostView(w)
    want = {(kv, g): oracle.quantize_block(oracle.block_f32(w, src, g, kv, host=host), 7)
            for kv in ("k", "v") for g in range(Hkv)}
    prob = atlas.Problem(w)
    rejected = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_demote_pages(
        prob.args, prob.tiers,
        torch.tensor(np.array([src], np.uint32).view(np.int32), device=gpu),
        torch.tensor(np.array([dst], np.uint32).view(np.int32), device=gpu), rejected)
    torch.cuda.synchronize()
    assert int(rejected) == 0
    ta = oracle.HostView(w).tier_arrays()
    nan_blocks = 0
    for (kv, g), (codes, scale) in want.items():
        got_scale = np.float32(ta[f"i4_{kv}_scale"][n4, g])
        if np.isnan(scale):
            nan_blocks += 1
            assert np.isnan(got_scale), (kv, g)
        else:
            assert got_scale.tobytes() == scale.tobytes(), (kv, g)
        got = ta[f"i4_{kv}"][n4, g]
        assert np.array_equal(got.view(np.uint8), oracle.pack_int4(codes).view(np.uint8)), (kv, g)
    assert nan_blocks == 1


def test_demote_rejects_bad_destinations_and_poisons_bad_sources(gpu):
    w = _demote_case(gpu, "f16", seed=12)
    Hkv = w.num_kv_heads
    prob = atlas.Problem(w)
    n8 = w.tiers["i8_k"].shape[0]
    before = w.tiers["i8_k"].clone()
    src_t = torch.tensor([0, w.num_blocks + 9], dtype=torch.int32, device=gpu)
    dst = np.array([(1 << 30) | (n8 + 40), (1 << 30) | 0], dtype=np.uint32)
    dst_t = torch.tensor(dst.view(np.int32), device=gpu)
    rejected = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_demote_pages(prob.args, prob.tiers, src_t, dst_t, rejected)
    torch.cuda.synchronize()
    assert int(rejected) == 2
    assert torch.equal(w.tiers["i8_k"], before)                 # codes untouched
    assert torch.isnan(w.tiers["i8_k_scale"][0]).all()          # bad source: NaN scales
    assert torch.isnan(w.tiers["i8_v_scale"][0]).all()
    assert w.tiers["i8_k_scale"].shape[1] == Hkv


def test_demote_full_size_sampled(gpu):
    """The benchmarked demotion (every full page of the 64-sequence bf16 GQA
    decode workload, split int8 / int4 by a seeded coin), checked bit-exact on
    sampled (page, kv head) blocks, including the first and the last."""
    import bench
    w = synth.config(3, device=gpu, seed=42)
    Hkv, P, D = w.num_kv_heads, w.page_tokens, w.head_dim
    src, dst, n8, n4 = bench.demote_plan(w)
    tiers = {}
    for kv in ("k", "v"):
        tiers[f"i8_{kv}"] = torch.zeros((n8, Hkv, P, D), dtype=torch.int8, device=gpu)
        tiers[f"i4_{kv}"] = torch.zeros((n4, Hkv, P, D // 2), dtype=torch.uint8, device=gpu)
        tiers[f"i8_{kv}_scale"] = torch.full((n8, Hkv), -1.0, device=gpu)
        tiers[f"i4_{kv}_scale"] = torch.full((n4, Hkv), -1.0, device=gpu)
    prob = atlas.Problem(w)
    rejected = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_demote_pages(prob.args, atlas.make_tiers(tiers), torch.from_numpy(src).to(gpu),
                             torch.from_numpy(dst).to(gpu), rejected)
    torch.cuda.synchronize()
    assert int(rejected) == 0
    # every destination scale was written (no -1 left)
    for key in ("i8_k_scale", "i8_v_scale", "i4_k_scale", "i4_v_scale"):
        assert bool((tiers[key] >= 0).all()), key

    rng = np.random.default_rng(3)
    pick = np.unique(np.concatenate([[0, len(src) - 1], rng.integers(0, len(src), 48)]))
    host = oracle.HostView(w)
    (ka, kind), (va, _) = host.pools()
    for i in pick:
        e = int(np.uint32(dst[i]))
        tier, slot = e >> 30, e & ((1 << 30) - 1)
        key, qmax = ("i8", 127) if tier == 1 else ("i4", 7)
        for arr, kv in ((ka, "k"), (va, "v")):
            got_codes = tiers[f"{key}_{kv}"][slot].cpu().numpy()
            got_scale = tiers[f"{key}_{kv}_scale"][slot].cpu().numpy()
            for g in range(Hkv):
                x = oracle.widen_bits(arr[int(src[i]), g], kind).astype(np.float32)
                codes, scale = oracle.quantize_block(x, qmax)
                assert got_scale[g].tobytes() == scale.tobytes(), (i, kv, g)
                want = codes.astype(np.int8) if tier == 1 else oracle.pack_int4(codes)
                assert np.array_equal(got_codes[g].view(np.uint8), want.view(np.uint8)), (i, kv, g)


@pytest.mark.parametrize("hot_dtype", ["f16", "bf16"])
def test_demote_cascade_transcodes_cold_slots(gpu, hot_dtype):
    """The compression cascade: hot -> FP8 -> INT8 -> INT4, and hot -> INT8 ->
    INT4, each step bit-exact against the oracle's encoder applied to the
    oracle's f32 reading of the source block."""
    w = _demote_case(gpu, hot_dtype, seed=13)
    Hkv, P, D = w.num_kv_heads, w.page_tokens, w.head_dim
    ent = w.page_table[2].view(np.uint32)
    pages = [p for p in range(int(w.context_lens[2]) // P) if (int(ent[p]) >> 30) == 0][:2]
    src0 = [int(ent[p]) for p in pages]
    n8, n4 = w.tiers["i8_k"].shape[0], w.tiers["i4_k"].shape[0]
    for key, extra in (("i8", 2), ("i4", 2)):
        for kv in ("k", "v"):
            t = w.tiers[f"{key}_{kv}"]
            w.tiers[f"{key}_{kv}"] = torch.cat([t, torch.zeros((extra,) + t.shape[1:],
                                                               dtype=t.dtype, device=gpu)])
            sc = w.tiers[f"{key}_{kv}_scale"]
            w.tiers[f"{key}_{kv}_scale"] = torch.cat([sc, torch.full((extra, Hkv), -1.0,
                                                                     device=gpu)])
    for kv in ("k", "v"):
        w.tiers[f"f8_{kv}"] = torch.zeros((1, Hkv, P, D), dtype=torch.uint8, device=gpu)
        w.tiers[f"f8_{kv}_scale"] = torch.full((1, Hkv), -1.0, device=gpu)
    chains = [[src0[0], (3 << 30) | 0, (1 << 30) | n8, (2 << 30) | n4],
              [src0[1], (1 << 30) | (n8 + 1), (2 << 30) | (n4 + 1)]]
    qfun = {1: lambda x: oracle.quantize_block(x, 127), 2: lambda x: oracle.quantize_block(x, 7),
            3: oracle.quantize_block_fp8}
    for step in range(3):
        jobs = [(c[step], c[step + 1]) for c in chains if step + 1 < len(c)]
        prob = atlas.Problem(w)
        src = torch.tensor(np.array([j[0] for j in jobs], np.uint32).view(np.int32), device=gpu)
        dst = torch.tensor(np.array([j[1] for j in jobs], np.uint32).view(np.int32), device=gpu)
        rejected = torch.zeros(1, dtype=torch.int32, device=gpu)
        # expected from the source as it stands before the step
        host = oracle.HostView(w)
        want = {}
        for s_e, d_e in jobs:
            for kv in ("k", "v"):
                for g in range(Hkv):
                    x = oracle.block_f32(w, s_e, g, kv, host=host)
                    want[(d_e, kv, g)] = qfun[d_e >> 30](x)
        atlas.atlas_demote_pages(prob.args, prob.tiers, src, dst, rejected)
        torch.cuda.synchronize()
        assert int(rejected) == 0
        ta = oracle.HostView(w).tier_arrays()
        for (d_e, kv, g), (codes, scale) in want.items():
            tier, slot = d_e >> 30, d_e & ((1 << 30) - 1)
            key = {1: "i8", 2: "i4", 3: "f8"}[tier]
            assert np.float32(ta[f"{key}_{kv}_scale"][slot, g]).tobytes() == scale.tobytes()
            got = ta[f"{key}_{kv}"][slot, g]
            exp = oracle.pack_int4(codes) if tier == 2 else codes.astype(
                np.int8 if tier == 1 else np.uint8)
            assert np.array_equal(got.view(np.uint8), exp.view(np.uint8)), (step, d_e, kv, g)
    # point the pages at the ends of their chains and attend
    new = ent.copy()
    for p, c in zip(pages, chains):
        new[p] = c[-1]
    w.page_table[2] = new.view(np.int32)
    out, lse = run(w)
    check(w, out, lse)
