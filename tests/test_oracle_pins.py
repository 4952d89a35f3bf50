"""Pins of the f64 oracle against facts that do not come from the oracle.

Each test ties one part of the oracle to a library routine, a closed form, an
invariant stated on the source pages, a printed value, or a published
reference stream, chosen so that a dropped term, a wrong sign or index, a
transposed operand or an off-by-one in the causal limit fails at least one.
"""

import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bottom_right_mask(n_q, n_keys, ctx):
    # Row t of a chunk of n_q new queries sits at position ctx - n_q + t.
    pos = ctx - n_q + np.arange(n_q)
    return np.arange(n_keys)[None, :] <= pos[:, None]


# ---------------------------------------------------------------------------
# 1. Attention definition vs torch's SDPA (float64, explicit mask)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ctx,n_q,d", [(1, 1, 1), (2, 2, 3), (5, 3, 4),
                                       (8, 8, 2), (8, 1, 4), (7, 4, 16)])
def test_attend_matches_torch_sdpa(ctx, n_q, d):
    rng = np.random.default_rng(ctx * 100 + n_q * 10 + d)
    q = rng.standard_normal((n_q, d))
    k = rng.standard_normal((ctx, d))
    v = rng.standard_normal((ctx, d))
    scale = 0.37
    vis = ctx - n_q + np.arange(n_q) + 1
    out, lse = oracle.attend(q, k, v, vis, scale)
    mask = torch.from_numpy(_bottom_right_mask(n_q, ctx, ctx))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], attn_mask=mask[None], scale=scale)[0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    scores = (torch.from_numpy(q) @ torch.from_numpy(k).T) * scale
    scores = scores.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(scores, dim=-1).numpy(),
                               rtol=0, atol=1e-12)


def test_folded_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    ctx, n_q, d = 37, 5, 8
    q, k, v = (rng.standard_normal(s) for s in ((n_q, d), (ctx, d), (ctx, d)))
    vis = ctx - n_q + np.arange(n_q) + 1
    mask = torch.from_numpy(_bottom_right_mask(n_q, ctx, ctx))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], attn_mask=mask[None], scale=0.5)[0]
    for P in (1, 3, 4, 16, 64):
        out, _ = oracle.attend(q, k, v, vis, 0.5, page_tokens=P)
        np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 2. Closed forms
# ---------------------------------------------------------------------------

def test_one_token_context_returns_v0():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((1, 6)), rng.standard_normal((1, 6)), rng.standard_normal((1, 6))
    out, lse = oracle.attend(q, k, v, [1], 0.25)
    np.testing.assert_array_equal(out[0], v[0])
    assert lse[0] == pytest.approx(0.25 * float(q[0] @ k[0]), abs=1e-15)


def test_identical_v_rows_return_that_row():
    rng = np.random.default_rng(2)
    ctx, d = 50, 8
    q = rng.standard_normal((3, d))
    k = rng.standard_normal((ctx, d))
    v = np.tile(rng.standard_normal(d), (ctx, 1))
    out, _ = oracle.attend(q, k, v, [50, 17, 1], 1.3)
    np.testing.assert_allclose(out, np.tile(v[0], (3, 1)), rtol=0, atol=1e-14)


def test_identical_k_rows_give_mean_of_visible_v():
    rng = np.random.default_rng(3)
    ctx, d = 40, 4
    q = rng.standard_normal((2, d))
    k = np.tile(rng.standard_normal(d), (ctx, 1))
    v = rng.standard_normal((ctx, d))
    vis = [40, 9]
    out, lse = oracle.attend(q, k, v, vis, 0.7)
    for r, n in enumerate(vis):
        np.testing.assert_allclose(out[r], v[:n].mean(axis=0), rtol=0, atol=1e-13)
        s = 0.7 * float(q[r] @ k[0])
        assert lse[r] == pytest.approx(s + math.log(n), abs=1e-12)


def test_zero_query_gives_mean_and_log_count():
    rng = np.random.default_rng(4)
    ctx, d = 33, 5
    k, v = rng.standard_normal((ctx, d)), rng.standard_normal((ctx, d))
    out, lse = oracle.attend(np.zeros((3, d)), k, v, [33, 2, 1], 0.9)
    for r, n in enumerate([33, 2, 1]):
        np.testing.assert_allclose(out[r], v[:n].mean(axis=0), rtol=0, atol=1e-13)
        assert lse[r] == pytest.approx(math.log(n), abs=1e-13)


def test_one_hot_values_expose_softmax_weights():
    # V_j = e_j: out is the softmax row itself; keys past the causal limit
    # must get exactly zero weight.
    rng = np.random.default_rng(5)
    ctx = 12
    q = rng.standard_normal((4, 3))
    k = rng.standard_normal((ctx, 3))
    v = np.eye(ctx)
    vis = np.array([12, 11, 5, 1])
    qd = np.concatenate([q, np.zeros((4, ctx - 3))], axis=1)
    kd = np.concatenate([k, np.zeros((ctx, ctx - 3))], axis=1)
    out, _ = oracle.attend(qd, kd, v, vis, 0.8)
    for r, n in enumerate(vis):
        w = scipy.special.softmax(0.8 * (k[:n] @ q[r]))
        np.testing.assert_allclose(out[r, :n], w, rtol=0, atol=1e-14)
        assert np.all(out[r, n:] == 0.0)


def test_two_key_closed_form_has_the_scale_and_sign():
    q = np.array([[1.0, 2.0]])
    k = np.array([[0.5, -1.0], [2.0, 0.25]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    scale = 0.3
    s0, s1 = scale * (0.5 - 2.0), scale * (2.0 + 0.5)
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    out, lse = oracle.attend(q, k, v, [2], scale)
    np.testing.assert_allclose(out[0], [1 - w1, w1], rtol=0, atol=1e-15)
    assert lse[0] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), abs=1e-14)


def test_empty_context_gives_zero_and_minus_inf():
    out, lse = oracle.attend(np.ones((1, 2)), np.ones((3, 2)), np.ones((3, 2)), [0], 1.0)
    assert np.all(out == 0) and lse[0] == -np.inf


def test_large_scores_do_not_overflow():
    # Max subtraction (RustAttention "Numerically Stable Softmax"): scores of
    # 1e4 would overflow exp() without it.
    q = np.array([[100.0]])
    k = np.array([[100.0], [99.0]])
    v = np.array([[1.0], [3.0]])
    out, lse = oracle.attend(q, k, v, [2], 1.0)
    w = 1.0 / (1.0 + math.exp(100.0))
    assert out[0, 0] == pytest.approx(1.0 + 2.0 * w, abs=1e-15)
    assert lse[0] == pytest.approx(10000.0 + math.log1p(math.exp(-100.0)), abs=1e-9)


# ---------------------------------------------------------------------------
# 3. CFR-Atlas contract: folded == full-KV; page-size invariance
# ---------------------------------------------------------------------------

def test_folded_equals_full_and_is_page_size_invariant():
    rng = np.random.default_rng(6)
    ctx, d, n_q = 1000, 16, 9
    q, k, v = (rng.standard_normal(s) for s in ((n_q, d), (ctx, d), (ctx, d)))
    vis = ctx - n_q + np.arange(n_q) + 1
    full, lse_full = oracle.attend(q, k, v, vis, 0.25)
    for P in (1, 7, 16, 64, 256, 512, 4096):
        fo, fl = oracle.attend(q, k, v, vis, 0.25, page_tokens=P)
        assert np.max(np.abs(fo - full)) <= 1e-12
        assert np.max(np.abs(fl - lse_full)) <= 1e-12


# ---------------------------------------------------------------------------
# 4. Split merge (log-sum-exp) vs unsplit attention
# ---------------------------------------------------------------------------

def test_merge_of_any_key_partition_equals_unsplit():
    rng = np.random.default_rng(8)
    ctx, d = 300, 8
    q = rng.standard_normal((1, d))
    k, v = rng.standard_normal((ctx, d)), rng.standard_normal((ctx, d))
    full, lse_full = oracle.attend(q, k, v, [ctx], 0.4)
    for cuts in ([0, 300], [0, 1, 300], [0, 100, 200, 300], [0, 0, 150, 150, 300],
                 [0, 17, 18, 250, 300]):
        po, pl = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, l = oracle.attend(q, k[a:b], v[a:b], [b - a], 0.4)
            po.append(o)
            pl.append(l)
        mo, ml = oracle.merge_splits(np.stack(po), np.stack(pl))
        np.testing.assert_allclose(mo, full, rtol=0, atol=1e-13)
        np.testing.assert_allclose(ml, lse_full, rtol=0, atol=1e-12)


def test_merge_single_split_is_identity_and_all_empty_is_zero():
    o = np.array([[[1.5, -2.0]]])
    l = np.array([[0.75]])
    mo, ml = oracle.merge_splits(o, l)
    np.testing.assert_array_equal(mo, o[0])
    np.testing.assert_array_equal(ml, l[0])
    mo, ml = oracle.merge_splits(np.zeros((3, 1, 2)), np.full((3, 1), -np.inf))
    assert np.all(mo == 0) and ml[0] == -np.inf


# ---------------------------------------------------------------------------
# 5. Paging, GQA head mapping and tiers, through synth problems
# ---------------------------------------------------------------------------

def _repaged(w, P_new, placement_seed):
    """Same logical K/V, re-laid into a pool with page size P_new and a
    different physical permutation."""
    S, Hkv, D = w.num_seqs, w.num_kv_heads, w.head_dim
    rng = np.random.default_rng(placement_seed)
    host = oracle.HostView(w)
    logical = [[oracle.logical_kv(w, s, g, host=host) for g in range(Hkv)]
               for s in range(S)]
    n_pages = [-(-int(c) // P_new) for c in w.context_lens]
    total = sum(n_pages)
    ids = rng.permutation(total)
    kp = np.full((total + 1, Hkv, P_new, D), np.nan)
    vp = np.full((total + 1, Hkv, P_new, D), np.nan)
    table = np.full((S, max(n_pages)), total, dtype=np.int32)
    i = 0
    for s in range(S):
        ctx = int(w.context_lens[s])
        for p in range(n_pages[s]):
            blk = int(ids[i])
            i += 1
            table[s, p] = blk
            t0, t1 = p * P_new, min(ctx, (p + 1) * P_new)
            for g in range(Hkv):
                kp[blk, g, :t1 - t0] = logical[s][g][0][t0:t1]
                vp[blk, g, :t1 - t0] = logical[s][g][1][t0:t1]
    w2 = synth.Paged(S, w.num_heads, Hkv, D, P_new, w.q_dtype, "f32",
                     w.context_lens, w.query_lens, w.scale, w.q,
                     torch.from_numpy(kp.astype(np.float32)),
                     torch.from_numpy(vp.astype(np.float32)), table)
    return w2


def test_reference_is_invariant_to_page_size_and_placement():
    w = synth.build(dict(num_seqs=3, context_lens=[37, 64, 5], query_lens=[1, 3, 2],
                         num_heads=4, num_kv_heads=2, head_dim=8, page_tokens=16,
                         kv_dtype="f32"), seed=11)
    out, lse = oracle.reference(w)
    assert np.all(np.isfinite(out))
    for P_new, seed in ((1, 1), (5, 2), (64, 3), (16, 4)):
        o2, l2 = oracle.reference(_repaged(w, P_new, seed))
        np.testing.assert_allclose(o2, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)


def test_reference_matches_unpaged_sdpa_per_head():
    # Logical K/V read straight from the pool through the table, attended by
    # torch SDPA (float64) with the bottom-right causal mask.
    w = synth.build(dict(num_seqs=2, context_lens=[40, 23], query_lens=[4, 1],
                         num_heads=6, num_kv_heads=2, head_dim=4, page_tokens=16,
                         kv_dtype="bf16"), seed=12)
    out, lse = oracle.reference(w)
    qs = w.query_start
    kb = w.k_pool.view(torch.int16).numpy().view(np.uint16)
    vb = w.v_pool.view(torch.int16).numpy().view(np.uint16)

    def bf(a):
        return torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32)).double()

    for s in range(2):
        ctx, n_q = int(w.context_lens[s]), int(w.query_lens[s])
        blocks = [int(w.page_table[s, j // 16]) for j in range(ctx)]
        for h in range(6):
            g = h // 3
            K = bf(np.stack([kb[blocks[j], g, j % 16] for j in range(ctx)]))
            V = bf(np.stack([vb[blocks[j], g, j % 16] for j in range(ctx)]))
            Q = w.q[qs[s]:qs[s] + n_q, h].double()
            mask = torch.from_numpy(_bottom_right_mask(n_q, ctx, ctx))
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], attn_mask=mask[None], scale=w.scale)[0]
            np.testing.assert_allclose(out[qs[s]:qs[s] + n_q, h], ref.numpy(),
                                       rtol=0, atol=1e-12)
            sc = (Q @ K.T * w.scale).masked_fill(~mask, float("-inf"))
            np.testing.assert_allclose(lse[qs[s]:qs[s] + n_q, h],
                                       torch.logsumexp(sc, -1).numpy(), rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_replicated_kv():
    w = synth.build(dict(num_seqs=2, context_lens=[50, 31], num_heads=8,
                         num_kv_heads=2, head_dim=8, page_tokens=16,
                         kv_dtype="f32"), seed=13)
    out, lse = oracle.reference(w)
    G = 4
    idx = torch.arange(8) // G
    w_mha = synth.Paged(w.num_seqs, 8, 8, 8, 16, "f32", "f32", w.context_lens,
                        w.query_lens, w.scale, w.q,
                        w.k_pool[:, idx].contiguous(), w.v_pool[:, idx].contiguous(),
                        w.page_table)
    o2, l2 = oracle.reference(w_mha)
    np.testing.assert_array_equal(o2, out)
    np.testing.assert_array_equal(l2, lse)
    # and a different kv head really gives a different answer
    w_swap = synth.Paged(w.num_seqs, 8, 2, 8, 16, "f32", "f32", w.context_lens,
                         w.query_lens, w.scale, w.q, w.k_pool.flip(1).contiguous(),
                         w.v_pool.flip(1).contiguous(), w.page_table)
    o3, _ = oracle.reference(w_swap)
    assert np.max(np.abs(o3 - out)) > 1e-3


def test_poisoned_tails_and_unused_blocks_never_reach_the_reference():
    w = synth.build(dict(num_seqs=3, context_lens=[17, 1, 48], num_heads=2,
                         num_kv_heads=1, head_dim=4, page_tokens=16, kv_dtype="f32"),
                    seed=14)
    assert torch.isnan(w.k_pool).any()  # the poison is there ...
    out, lse = oracle.reference(w)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))  # ... and unread


# ---------------------------------------------------------------------------
# 6. Cold-tier decoding
# ---------------------------------------------------------------------------

def test_int4_nibble_decoding_by_hand():
    packed = np.array([[0x7F, 0x80, 0x08, 0x00, 0xF1, 0x9E]], dtype=np.uint8)
    np.testing.assert_array_equal(
        oracle.int4_codes(packed),
        [[-1, 7, 0, -8, -8, 0, 0, 0, 1, -1, -2, -7]])


def test_dequant_is_code_times_scale():
    codes = np.array([[[[127, -127, 0, 1]]]], dtype=np.int8)
    scale = np.array([[0.5]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.dequant_f32(codes, scale),
                                  [[[[63.5, -63.5, 0.0, 0.5]]]])


def test_tiered_reference_reads_each_tier():
    w = synth.build(dict(num_seqs=2, context_lens=[100, 70], num_heads=4,
                         num_kv_heads=2, head_dim=8, page_tokens=16, q_dtype="bf16",
                         kv_dtype="f16", tiers=dict(hot_tokens=20, p_int8=0.5)),
                    seed=15)
    tiers = w.page_table.view(np.uint32) >> synth.TIER_SHIFT
    assert set(np.unique(tiers)) >= {0, 1, 2}
    host = oracle.HostView(w)
    ta = host.tier_arrays()
    # K of sequence 0, kv head 1, compared page by page with direct decoding
    K, V = oracle.logical_kv(w, 0, 1, host=host)
    for p in range(w.pages_of(0)):
        e = int(w.page_table[0, p]) & 0xFFFFFFFF
        t, slot = e >> 30, e & ((1 << 30) - 1)
        rows = slice(p * 16, min(100, p * 16 + 16))
        n = rows.stop - rows.start
        if t == 1:
            ref = ta["i8_k"][slot, 1, :n].astype(np.float64) * float(ta["i8_k_scale"][slot, 1])
        elif t == 2:
            ref = oracle.int4_codes(ta["i4_k"][slot, 1, :n]).astype(np.float64) * \
                float(ta["i4_k_scale"][slot, 1])
        else:
            ref = w.k_pool[slot, 1, :n].double().numpy()
        np.testing.assert_array_equal(K[rows], ref)
    # quantisation error of the cold tiers stays within half a step
    assert np.all(np.isfinite(oracle.reference(w)[0]))


# ---------------------------------------------------------------------------
# 7. SplitMix64 regenerator
# ---------------------------------------------------------------------------

def test_splitmix64_matches_published_stream():
    with open(os.path.join(GOLDEN, "splitmix64_reference_stream.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for seed, n, val in rows:
        assert oracle.splitmix64(int(seed), int(n)) == int(val)


def test_regen_first_counter_from_published_output():
    # counter 0 (layer 0, head 0, token 0, dim 0, K) is output 1 of the
    # stream; seed 0's first output is 0xE220A8397B1DCDAF (golden file).
    z = 0xE220A8397B1DCDAF
    x = np.float32(((z >> 40) - 2**23) / 2**23)
    bits = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    expect = np.array([rounded], dtype=np.uint32).view(np.float32)[0]
    got = oracle.regen_values(0, 0, 0, 0, 1, 1, 0)[0, 0]
    assert got == expect


def test_regen_values_are_bf16_in_range_and_distinct_per_coordinate():
    vals = {}
    for layer in (0, 3):
        for g in (0, 7):
            for kv in (0, 1):
                a = oracle.regen_values(42, layer, g, 1000, 64, 128, kv)
                assert np.all(np.abs(a) <= 1.0)
                bits = a.view(np.uint32)
                assert np.all((bits & 0xFFFF) == 0)
                vals[(layer, g, kv)] = a
    keys = list(vals)
    for i in range(len(keys)):
        for j in range(i + 1, len(keys)):
            assert np.mean(vals[keys[i]] == vals[keys[j]]) < 0.02
    a = vals[(0, 0, 0)]
    assert abs(float(a.mean())) < 0.02 and abs(float(a.var()) - 1 / 3) < 0.02
    # token ranges compose: [1000, 1064) == [1000, 1032) ++ [1032, 1064)
    b = np.concatenate([oracle.regen_values(42, 0, 0, 1000, 32, 128, 0),
                        oracle.regen_values(42, 0, 0, 1032, 32, 128, 0)])
    np.testing.assert_array_equal(a, b)


def test_regenerated_problem_uses_generator_for_every_page():
    w = synth.build(dict(num_seqs=1, context_lens=300, query_lens=20, num_heads=4,
                         num_kv_heads=2, head_dim=8, page_tokens=32, kv_dtype="bf16",
                         regen=dict(seed=9, layer=2, fraction=0.5)), seed=16)
    assert int(w.regen["regen_pages"][0]) == 5
    # resident pages are not materialised on the host side (NaN until the
    # library writes them), so the oracle regenerates every page
    assert torch.isnan(w.k_pool).all()
    K, V = oracle.logical_kv(w, 0, 1)
    np.testing.assert_array_equal(K, oracle.regen_values(9, 2, 1, 0, 300, 8, 0))
    np.testing.assert_array_equal(V, oracle.regen_values(9, 2, 1, 0, 300, 8, 1))


# ---------------------------------------------------------------------------
# 8. Byte accounting of the CFR-Atlas benchmark run
# ---------------------------------------------------------------------------

def test_cfr_bench_byte_accounting():
    with open(os.path.join(GOLDEN, "cfr_atlas_bench_65536_64_512.txt")) as f:
        g = dict(l.strip().split("=") for l in f if "=" in l and not l.startswith("#"))
    spec = synth.CONFIG_SPECS[2]
    ctx, D, P = spec["context_lens"], spec["head_dim"], spec["page_tokens"]
    assert (ctx, D, P) == (int(g["context_tokens"]), int(g["head_dim"]), int(g["page_tokens"]))
    per_head_kv = ctx * D * 4 * 2
    scratch = P * D * 4 * 2
    assert per_head_kv == int(g["baseline_kv_bytes"])
    assert scratch == int(g["cfr_scratch_bytes"])
    assert per_head_kv / scratch == float(g["estimated_memory_reduction"]) == ctx / P


# ---------------------------------------------------------------------------
# Cold-tier encoding (page demotion)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("qmax", [127, 7, 1])
def test_quantize_block_is_the_nearest_code(qmax):
    """Brute force: each code is the integer in [-qmax, qmax] nearest to
    x / scale (ties to even), found by exhaustive search."""
    rng = np.random.default_rng(qmax)
    x = (rng.standard_normal(96) * 1.7).astype(np.float32)
    codes, scale = oracle.quantize_block(x, qmax)
    assert scale == np.float32(np.max(np.abs(x)) / np.float32(qmax))
    cand = np.arange(-qmax, qmax + 1, dtype=np.float64)
    for xi, ci in zip(x, codes):
        t = np.float64(np.float32(xi / scale))
        d = np.abs(cand - t)
        best = cand[d == d.min()]
        want = best[0] if best.size == 1 else best[np.argmin(np.abs(best) % 2)]
        assert ci == want


@pytest.mark.parametrize("qmax", [127, 7, 1])
def test_quantize_block_extremes_symmetry_and_round_trip(qmax):
    rng = np.random.default_rng(3 + qmax)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    codes, scale = oracle.quantize_block(x, qmax)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert abs(int(codes[i])) == qmax and np.sign(codes[i]) == np.sign(x[i])
    assert np.all(np.abs(codes) <= qmax)
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * float(scale))
    assert np.all(err <= 0.5 * float(scale) * (1 + 1e-5))
    nc, ns = oracle.quantize_block(-x, qmax)
    assert ns == scale and np.array_equal(nc, -codes)
    pc, ps = oracle.quantize_block(x * np.float32(8.0), qmax)   # power-of-two scaling
    assert ps == scale * np.float32(8.0) and np.array_equal(pc, codes)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_quantize_block_with_a_non_finite_value_gives_nan(bad):
    """A block holding a NaN or an infinity encodes to a NaN scale with codes
    0, integer tiers and FP8 alike, so every value decoded from it is NaN:
    f32(code * NaN) is NaN for every code, the E4M3 values included."""
    x = np.linspace(-3, 3, 64, dtype=np.float32).reshape(8, 8)
    x[5, 3] = bad
    for qmax in (127, 7, 1):
        codes, scale = oracle.quantize_block(x, qmax)
        assert np.isnan(scale) and not codes.any()
        assert np.isnan(codes.astype(np.float32) * scale).all()
    codes, scale = oracle.quantize_block_fp8(x)
    assert np.isnan(scale) and not codes.any()
    assert np.isnan(oracle.fp8_e4m3_value(codes) * np.float64(scale)).all()


def test_quantize_block_zero_and_int4_packing():
    codes, scale = oracle.quantize_block(np.zeros((4, 8), np.float32), 7)
    assert scale == 0 and not codes.any()
    c = np.array([[-7, 7, 0, -1, 3, -8, 5, 2]], dtype=np.int16)
    packed = oracle.pack_int4(c)
    assert packed.tolist() == [[0x79, 0xF0, 0x83, 0x25]]
    assert np.array_equal(oracle.int4_codes(packed), c)


# ---------------------------------------------------------------------------
# 10. Positional policy: RoPE and ALiBi (CFR-Atlas README module list and
#     test list name both; the definitions are those of their papers)
# ---------------------------------------------------------------------------

def test_rope_known_rotations():
    # d = 4, theta = 10000: pair 0 turns by pos radians, pair 1 by pos / 100
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    e2 = np.array([0.0, 0.0, 1.0, 0.0])
    np.testing.assert_allclose(oracle.rope(e0, 1, 10000.0),
                               [0.5403023058681398, 0.8414709848078965, 0, 0], atol=1e-15)
    np.testing.assert_allclose(oracle.rope(e2, 1, 10000.0),
                               [0, 0, 0.9999500004166653, 0.009999833334166664], atol=1e-15)
    # pos = 3: pair 1 turns by 0.03 (the sign fixes the rotation direction)
    e3 = np.array([0.0, 0.0, 0.0, 1.0])
    np.testing.assert_allclose(oracle.rope(e3, 3, 10000.0),
                               [0, 0, -math.sin(0.03), math.cos(0.03)], atol=1e-15)
    # position 0 is the identity
    x = np.random.default_rng(0).standard_normal((5, 8))
    np.testing.assert_array_equal(oracle.rope(x, 0, 10000.0), x)


def test_rope_equals_complex_multiplication():
    # RoFormer's complex form: z_i = x_2i + i x_2i+1 times exp(i pos theta^(-2i/d))
    rng = np.random.default_rng(1)
    d, theta = 16, 500.0
    x = rng.standard_normal((7, d))
    pos = np.array([0, 1, 5, 77, 1000, 65535, 131071])
    z = x[:, 0::2] + 1j * x[:, 1::2]
    freq = np.array([theta ** (-(2.0 * i) / d) for i in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = zr.real, zr.imag
    np.testing.assert_allclose(oracle.rope(x, pos, theta), want, rtol=0, atol=1e-12)


def test_rope_scores_depend_on_relative_position_and_keep_norms():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64))
    for m, n, shift in ((10, 3, 100), (5000, 4000, 77), (0, 9, 131000)):
        a = oracle.rope(q, m, 10000.0) @ oracle.rope(k, n, 10000.0)
        b = oracle.rope(q, m + shift, 10000.0) @ oracle.rope(k, n + shift, 10000.0)
        assert abs(a - b) < 1e-9
        np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, m, 10000.0)),
                                   np.linalg.norm(q), rtol=1e-14)


def test_alibi_matches_sdpa_with_additive_bias():
    rng = np.random.default_rng(3)
    ctx, n_q, d, scale = 23, 6, 8, 0.4
    q, k, v = (rng.standard_normal(s) for s in ((n_q, d), (ctx, d), (ctx, d)))
    slope = np.array([0.5, 0.25, 0.125, 2 ** -0.5, 1.0, 0.0])
    vis = ctx - n_q + np.arange(n_q) + 1
    out, lse = oracle.attend(q, k, v, vis, scale, slope=slope)
    pos = vis - 1
    bias = -slope[:, None] * (pos[:, None] - np.arange(ctx)[None, :])
    mask = _bottom_right_mask(n_q, ctx, ctx)
    add = torch.from_numpy(np.where(mask, bias, -np.inf))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=add[None], scale=scale)[0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    sc = torch.from_numpy(q) @ torch.from_numpy(k).T * scale + add
    np.testing.assert_allclose(lse, torch.logsumexp(sc, -1).numpy(), rtol=0, atol=1e-12)


def test_alibi_zero_query_gives_geometric_weights():
    # q = 0: weight of the key i tokens back is r^i, r = exp(-slope)
    n, d, slope = 40, 40, 0.3
    r = math.exp(-slope)
    v = np.eye(n, d)  # one-hot rows expose the weights
    out, lse = oracle.attend(np.zeros((1, d)), np.ones((n, d)), v, [n], 1.0, slope=[slope])
    z = (1 - r ** n) / (1 - r)
    np.testing.assert_allclose(out[0], [r ** (n - 1 - j) / z for j in range(n)], atol=1e-15)
    assert abs(lse[0] - math.log(z)) < 1e-13
    # slope 0 is the plain softmax
    q = np.random.default_rng(4).standard_normal((3, d))
    kk = np.random.default_rng(5).standard_normal((n, d))
    a = oracle.attend(q, kk, v, [5, 20, 40], 0.2, slope=[0.0, 0.0, 0.0])
    b = oracle.attend(q, kk, v, [5, 20, 40], 0.2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_reference_positional_policy():
    # decode and prefill rows: the reference rotates every query row by its
    # own position and biases by head slope, which equals attending the
    # rotated rows with the explicit bias; regenerated keys are rotated by
    # their token position
    w = synth.build(dict(num_seqs=2, context_lens=[45, 70], query_lens=[3, 1], num_heads=4,
                         num_kv_heads=2, head_dim=8, page_tokens=16, kv_dtype="bf16",
                         positional=dict(alibi=True, rope_theta=10000.0)), seed=17)
    np.testing.assert_allclose(w.alibi_slopes, [2 ** -2, 2 ** -4, 2 ** -6, 2 ** -8])
    out, lse = oracle.reference(w)
    qh = oracle.widen(w.q)
    seqs, vis = oracle.row_info(w)
    for row in range(w.total_q):
        s = int(seqs[row])
        K, V = oracle.logical_kv(w, s, 0)
        K1, V1 = oracle.logical_kv(w, s, 1)
        for h in range(4):
            Kh, Vh = (K, V) if h < 2 else (K1, V1)
            n = int(vis[row])
            qr = oracle.rope(qh[row, h], n - 1, 10000.0)
            sc = Kh[:n] @ qr * w.scale - w.alibi_slopes[h] * (n - 1 - np.arange(n))
            p = np.exp(sc - sc.max())
            np.testing.assert_allclose(out[row, h], p @ Vh[:n] / p.sum(), atol=1e-12)
            assert abs(lse[row, h] - (sc.max() + math.log(p.sum()))) < 1e-12
    wr = synth.build(dict(num_seqs=1, context_lens=100, query_lens=4, num_heads=2,
                          num_kv_heads=1, head_dim=8, page_tokens=32, kv_dtype="bf16",
                          regen=dict(seed=5, layer=1, fraction=0.5),
                          positional=dict(rope_theta=100.0)), seed=18)
    K, V = oracle.logical_kv(wr, 0, 0)
    raw = oracle.regen_values(5, 1, 0, 0, 100, 8, 0)
    rot = oracle.rope(raw, np.arange(100), 100.0)
    assert np.all(np.abs(K - rot) <= np.abs(rot) * 2.0 ** -8)  # one bf16 rounding
    bits = (K.astype(np.float32).view(np.uint32) & 0xFFFF).astype(np.int64)
    assert not bits.any()  # bf16 values
    np.testing.assert_array_equal(V, oracle.regen_values(5, 1, 0, 0, 100, 8, 1))


def test_round_bf16_is_nearest_even():
    # agrees with torch's f32 -> bf16 conversion (nearest, ties to even) on
    # f32 inputs, including exact ties
    rng = np.random.default_rng(6)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -100 * (1 + 2 ** -8),
                     1.5 + 2 ** -8], dtype=np.float32)
    x32 = np.concatenate([x32, ties])
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x32.astype(np.float64)), want)
    # directly from f64: a value just above a tie rounds up (f32 would round
    # it onto the tie first and then to even, i.e. down)
    x = 1 + 2 ** -8 + 2 ** -40
    assert oracle.round_bf16(x) == 1 + 2 ** -7
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0


# ---------------------------------------------------------------------------
# 11. FP8 (E4M3) cold tier
# ---------------------------------------------------------------------------

def test_fp8_values_match_torch_e4m3fn_and_named_codes():
    v = oracle.fp8_e4m3_value(np.arange(256))
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    np.testing.assert_array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    named = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x7E: 448.0, 0xC0: -2.0, 0xFE: -448.0}
    for c, val in named.items():
        assert v[c] == val, hex(c)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])


def test_fp8_encode_is_nearest_even_and_matches_torch():
    rng = np.random.default_rng(8)
    y = (rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-14, 1, 20000))).astype(np.float32)
    ties = oracle.fp8_e4m3_value(np.arange(0x7E))  # midpoints between neighbours
    mids = ((ties[:-1] + ties[1:]) / 2).astype(np.float32)
    y = np.concatenate([y, mids, -mids, [0.0, -0.0, 448.0, -448.0, 3e-5, -3e-5]]).astype(np.float32)
    got = oracle.fp8_e4m3_encode(y)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)
    # every finite code's value encodes to itself; above 448 saturates
    c = np.array([k for k in range(256) if (k & 0x7F) != 0x7F])
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_value(c)), c)
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(np.float32([460.0, 1e9, -500.0])),
                                  [0x7E, 0x7E, 0xFE])


def test_fp8_block_scale_extremes_and_round_trip():
    x = np.random.default_rng(9).standard_normal((16, 64)).astype(np.float32)
    codes, scale = oracle.quantize_block_fp8(x)
    assert scale == np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] in (0x7E, 0xFE)
    back = oracle.fp8_e4m3_value(codes) * np.float64(scale)
    normal = np.abs(x) >= 2.0 ** -6 * scale
    assert np.all(np.abs(back - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4)
    assert np.all(np.abs(back - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale))
    c2, s2 = oracle.quantize_block_fp8(-x)
    np.testing.assert_array_equal(c2, codes ^ 0x80)
    z, sz = oracle.quantize_block_fp8(np.zeros((4, 8), np.float32))
    assert sz == 0 and not z.any()


def test_tiered_reference_reads_fp8_pages():
    w = synth.build(dict(num_seqs=2, context_lens=[70, 130], num_heads=4, num_kv_heads=2,
                         head_dim=8, page_tokens=16, kv_dtype="f16",
                         tiers=dict(hot_tokens=16, p_int8=0.3, p_fp8=0.4)), seed=19)
    assert w.tiers["counts"][3] > 0
    ta = oracle.HostView(w).tier_arrays()
    for s in range(2):
        for p in range(w.pages_of(s)):
            e = int(w.page_table[s, p]) & 0xFFFFFFFF
            if e >> 30 != 3:
                continue
            slot = e & ((1 << 30) - 1)
            K, V = oracle.logical_kv(w, s, 1)
            n = min(16, int(w.context_lens[s]) - 16 * p)
            want = oracle.fp8_e4m3_value(ta["f8_k"][slot, 1, :n]) * np.float64(ta["f8_k_scale"][slot, 1])
            np.testing.assert_array_equal(K[16 * p:16 * p + n], want)


def test_block_f32_reads_each_tier():
    w = synth.build(dict(num_seqs=1, context_lens=200, num_heads=4, num_kv_heads=2,
                         head_dim=8, page_tokens=16, kv_dtype="bf16",
                         tiers=dict(hot_tokens=40, p_int8=0.4, p_fp8=0.3)), seed=23)
    ta = oracle.HostView(w).tier_arrays()
    seen = set()
    for e in w.page_table[0, :w.pages_of(0)].view(np.uint32):
        tier, slot = int(e) >> 30, int(e) & ((1 << 30) - 1)
        got = oracle.block_f32(w, e, 1, "v")
        if tier == 0:
            want = w.v_pool[slot, 1].float().numpy()
        elif tier == 3:
            want = (torch.from_numpy(ta["f8_v"][slot, 1]).view(torch.float8_e4m3fn).float()
                    * float(ta["f8_v_scale"][slot, 1])).numpy()
        else:
            key = "i8" if tier == 1 else "i4"
            c = ta[f"{key}_v"][slot, 1]
            c = oracle.int4_codes(c) if key == "i4" else c
            want = oracle.dequant_f32(c[None, None], ta[f"{key}_v_scale"][slot, 1:2][None])[0, 0]
        np.testing.assert_array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))
        seen.add(tier)
    assert seen == {0, 1, 2, 3}



# ---------------------------------------------------------------------------
# 12. INT2 cold tier (tier 3, kind 1)
# ---------------------------------------------------------------------------

def test_int2_packing_by_hand_and_round_trip():
    # byte 0b01_11_00_10: elements -2, 0, -1, 1 (element 4i + j in bits 2j)
    assert oracle.int2_codes(np.array([0b01110010], np.uint8)).tolist() == [-2, 0, -1, 1]
    allb = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.pack_int2(oracle.int2_codes(allb)), allb)
    assert oracle.pack_int2(np.array([1, -1, 0, 1])).tolist() == [0b01001101]


def test_entry_classes():
    assert oracle.entry_class(5) == (0, 5)
    assert oracle.entry_class((1 << 30) | 7) == (1, 7)
    assert oracle.entry_class((2 << 30) | 9) == (2, 9)
    assert oracle.entry_class((3 << 30) | 11) == (3, 11)
    assert oracle.entry_class((3 << 30) | (1 << 28) | 13) == (4, 13)
    assert oracle.entry_class((3 << 30) | (2 << 28) | 1)[0] == 5
    assert oracle.entry_class(np.uint32((3 << 30) | (3 << 28)).view(np.int32))[0] == 6


def test_tiered_reference_reads_int2_pages():
    w = synth.build(dict(num_seqs=2, context_lens=[90, 130], num_heads=4, num_kv_heads=2,
                         head_dim=8, page_tokens=16, kv_dtype="f16",
                         tiers=dict(hot_tokens=16, p_int8=0.2, p_fp8=0.2, p_int2=0.4)), seed=29)
    assert w.tiers["counts"][4] > 0
    ta = oracle.HostView(w).tier_arrays()
    seen = 0
    for s in range(2):
        K, V = oracle.logical_kv(w, s, 0)
        for p in range(w.pages_of(s)):
            cls, slot = oracle.entry_class(w.page_table[s, p])
            if cls != 4:
                continue
            n = min(16, int(w.context_lens[s]) - 16 * p)
            codes = oracle.int2_codes(ta["i2_v"][slot, 0, :n])
            assert set(np.unique(codes)) <= {-1, 0, 1}
            np.testing.assert_array_equal(V[16 * p:16 * p + n],
                                          codes * np.float64(ta["i2_v_scale"][slot, 0]))
            seen += 1
    assert seen > 0


# ---------------------------------------------------------------------------
# 13. 1-bit archival tier (tier 3, kind 2): signs + FP16 outliers
# ---------------------------------------------------------------------------

def test_1bit_hand_decoded_block():
    # 16 elements; the two largest magnitudes (3.0 at 2, 10.0 at 8) are the
    # outliers, listed by index with their FP16 bits (3.0 = 0x4200, 10.0 =
    # 0x4900); signs: elements 1, 3, 7 and 9 are negative (-0.0 is not)
    x = np.array([0.5, -2.0, 3.0, -0.25, 0.0, -0.0, 1.0, -1.0,
                  10.0, -0.5, 0, 0, 0, 0, 0, 0], np.float32)
    signs, scale, out = oracle.encode_1bit(x, 2)
    assert signs.tolist() == [0b10001010, 0b00000010]
    assert out.tolist() == [0x42000002, 0x49000008]
    # mean |x| of the 14 other elements: (0.5+2+0.25+1+1+0.5) / 14
    assert scale == np.float32(5.25 / 14)
    dec = oracle.decode_1bit(signs, scale, out, 16)
    s = np.float32(5.25 / 14)
    want = np.array([s, -s, 3.0, -s, s, s, s, -s, 10.0, -s, s, s, s, s, s, s], np.float32)
    np.testing.assert_array_equal(dec, want)


def test_1bit_outliers_are_the_largest_magnitudes_ties_to_lower_index():
    x = np.array([1, -1, 1, -1, 1, -1, 1, -1], np.float32)
    _, scale, out = oracle.encode_1bit(x, 3)
    assert [int(e) & 0xFFFF for e in out] == [0, 1, 2]
    assert scale == 1.0
    rng = np.random.default_rng(7)
    for n_out in (0, 1, 5, 64):
        x = (rng.standard_normal(512) * rng.choice([0.1, 1, 30], 512)).astype(np.float32)
        x[rng.integers(0, 512, 40)] = 0.75  # ties
        _, _, out = oracle.encode_1bit(x, n_out)
        idx = np.array([int(e) & 0xFFFF for e in out], dtype=np.int64)
        assert len(idx) == n_out and np.all(np.diff(idx) > 0)
        rest = np.setdiff1d(np.arange(512), idx)
        if n_out:
            # brute force: every kept magnitude >= every dropped one, and a
            # dropped element equal to the smallest kept one has a higher index
            lo = np.abs(x[idx]).min()
            assert np.all(np.abs(x[rest]) <= lo)
            tied_rest = rest[np.abs(x[rest]) == lo]
            tied_kept = idx[np.abs(x[idx]) == lo]
            assert tied_rest.size == 0 or tied_rest.min() > tied_kept.max()
        # the FP16 values are the nearest-even halves of the elements
        vals = np.array([np.uint16(int(e) >> 16).view(np.float16) for e in out], np.float16)
        np.testing.assert_array_equal(vals, x[idx].astype(np.float16))


def test_1bit_scale_minimises_the_sign_code_error():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(1024) * 2).astype(np.float32)
    signs, scale, out = oracle.encode_1bit(x, 16)
    idx = np.array([int(e) & 0xFFFF for e in out])
    rest = np.delete(x, idx).astype(np.float64)
    err = lambda s: np.sum((np.abs(rest) - s) ** 2)  # noqa: E731
    grid = np.linspace(0.5 * scale, 1.5 * scale, 2001)
    assert abs(grid[np.argmin([err(g) for g in grid])] - scale) <= (grid[1] - grid[0])
    # decoded error on the non-outliers equals err(scale); signs follow x
    dec = oracle.decode_1bit(signs, scale, out, 1024)
    keep = np.ones(1024, bool)
    keep[idx] = False
    np.testing.assert_array_equal(np.signbit(dec[keep]) & (x[keep] != 0), x[keep] < 0)
    assert np.all(np.abs(dec[keep]) == scale)


def test_1bit_exact_when_the_outliers_cover_every_nonzero():
    rng = np.random.default_rng(11)
    x = np.zeros(256, np.float32)
    pos = rng.choice(256, 20, replace=False)
    x[pos] = rng.standard_normal(20).astype(np.float16).astype(np.float32)
    signs, scale, out = oracle.encode_1bit(x, 20)
    assert scale == 0.0
    np.testing.assert_array_equal(oracle.decode_1bit(signs, scale, out, 256), x)


def test_1bit_special_cases():
    z = np.zeros(64, np.float32)
    signs, scale, out = oracle.encode_1bit(z, 4)
    assert scale == 0 and not signs.any() and out.tolist() == [0, 1, 2, 3]
    # no outliers: a pure sign code with the mean |x| of the whole block
    x = np.array([1, -3, 2, -2, 0, 4, -4, 4], np.float32)
    signs, scale, out = oracle.encode_1bit(x, 0)
    assert out.size == 0 and scale == np.float32(20 / 8) and signs.tolist() == [0b01001010]
    # NaN outranks every magnitude; inf too
    x = np.array([1, np.nan, -np.inf, 2, 0, 0, 0, 0], np.float32)
    _, _, out = oracle.encode_1bit(x, 2)
    assert [int(e) & 0xFFFF for e in out] == [1, 2]
    # decoder rules: an out-of-range index is ignored, a later duplicate wins
    dec = oracle.decode_1bit(np.array([0], np.uint8), 1.0,
                             np.array([3 | (0x3C00 << 16), 9 | (0x4000 << 16),
                                       3 | (0xC000 << 16)], np.uint32), 8)
    assert dec.tolist() == [1, 1, 1, -2, 1, 1, 1, 1]


def test_entry_classes_with_archival_kind():
    assert oracle.entry_class((3 << 30) | (2 << 28) | 5) == (5, 5)
    assert oracle.entry_class((3 << 30) | (3 << 28) | 5)[0] == 6


def test_hot_bits_rounds_to_nearest_even():
    # 1 + 2^-11 is halfway between two f16 values: ties to even (1.0); 1 +
    # 3 * 2^-11 rounds up to 1 + 2^-9; bf16 keeps 8 significant bits
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -2.5], np.float32)
    assert oracle.hot_bits(x, "f16").tolist() == [0x3C00, 0x3C02, 0xC100]
    y = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5], np.float32)
    assert oracle.hot_bits(y, "bf16").tolist() == [0x3F80, 0x3F82, 0xC020]
    assert oracle.hot_bits(np.float32(1.5), "f32").tolist() == 0x3FC00000
