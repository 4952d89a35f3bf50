"""GPU parity of the 1-bit archival tier (the extension tier, kind 2) and of
page reconstruction (atlas_promote_pages) through the C ABI.

Archiving: sign bits and outlier entries bit-exact against the oracle's
encoder, the scale within one f32 ulp (the device sums |x| in f64 in its own
order; the oracle's sum is exact to f64 rounding, then both round the mean to
f32).  Promotion of every class into hot blocks: bit-exact against the
oracle's values rounded to the hot type.  Attention and the validator refuse
1-bit entries (NaN rows, counted)."""

import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from tests.test_gpu_parity import check, run

pytestmark = pytest.mark.gpu

B1 = (3 << 30) | (2 << 28)
KIND3 = (3 << 30) | (3 << 28)


def _case(gpu, hot="f16", Hkv=2, P=16, D=128, ctx=(900, 1700), seed=41, H=None):
    return synth.build(dict(num_seqs=len(ctx), context_lens=list(ctx), num_heads=H or 8 * Hkv,
                            num_kv_heads=Hkv, head_dim=D, page_tokens=P, q_dtype="bf16",
                            kv_dtype=hot, placement="permuted",
                            tiers=dict(hot_tokens=max(ctx) // 2, p_int8=0.3, p_fp8=0.2,
                                       p_int2=0.2)),
                       device=gpu, seed=seed, name=f"1bit-{hot}-P{P}-D{D}")


def _add_b1_pool(w, n, n_out, gpu):
    Hkv, P, D = w.num_kv_heads, w.page_tokens, w.head_dim
    for kv in ("k", "v"):
        w.tiers[f"b1_{kv}"] = torch.full((n, Hkv, P * D // 8), 0xAA, dtype=torch.uint8, device=gpu)
        w.tiers[f"b1_{kv}_scale"] = torch.full((n, Hkv), -1.0, device=gpu)
        w.tiers[f"b1_{kv}_out"] = torch.full((n, Hkv, n_out), -1, dtype=torch.int32, device=gpu)


def _full_pages_by_class(w, per_class=2):
    """(seq, page, entry) of full pages, up to per_class of each class 0-4."""
    picked = {c: [] for c in range(5)}
    for s in range(w.num_seqs):
        full = int(w.context_lens[s]) // w.page_tokens
        for p in range(full):
            e = int(w.page_table[s, p]) & 0xFFFFFFFF
            c = oracle.entry_class(e)[0]
            if c < 5 and len(picked[c]) < per_class:
                picked[c].append((s, p, e))
    return [x for c in range(5) for x in picked[c]]


def _scale_close(got, want):
    want = np.float32(want)
    return got == want or abs(np.float64(got) - np.float64(want)) <= np.spacing(np.abs(want))


@pytest.mark.parametrize("hot,P,D,n_out", [("f16", 16, 128, 8), ("bf16", 16, 128, 64),
                                           ("f16", 64, 128, 64), ("bf16", 16, 64, 0),
                                           ("f16", 256, 64, 16), ("bf16", 48, 64, 16)])
def test_archive_matches_oracle(gpu, hot, P, D, n_out):
    w = _case(gpu, hot=hot, P=P, D=D, ctx=(1300, 2700), seed=P + D + n_out)
    pages = _full_pages_by_class(w)
    classes = {oracle.entry_class(e)[0] for _, _, e in pages}
    assert 0 in classes and len(classes) >= (5 if P == 16 else 2), classes
    n = len(pages)
    _add_b1_pool(w, n, n_out, gpu)
    src_np = np.array([e for _, _, e in pages], dtype=np.uint32)
    dst_np = np.array([B1 | i for i in range(n)], dtype=np.uint32)
    host = oracle.HostView(w)
    want = {}
    for i, e in enumerate(src_np):
        for kv in ("k", "v"):
            for g in range(w.num_kv_heads):
                want[(i, kv, g)] = oracle.encode_1bit(
                    oracle.block_f32(w, int(e), g, kv, host=host).ravel(), n_out)
    prob = atlas.Problem(w)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    print(f"[archive {hot} P{P} D{D} K{n_out}] {n} pages", flush=True)
    atlas.atlas_demote_pages(prob.args, prob.tiers,
                             torch.from_numpy(src_np.view(np.int32)).to(gpu),
                             torch.from_numpy(dst_np.view(np.int32)).to(gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    for kv in ("k", "v"):
        signs = w.tiers[f"b1_{kv}"].cpu().numpy()
        scales = w.tiers[f"b1_{kv}_scale"].cpu().numpy()
        outs = w.tiers[f"b1_{kv}_out"].cpu().numpy().view(np.uint32)
        for i in range(n):
            for g in range(w.num_kv_heads):
                ws, wscale, wout = want[(i, kv, g)]
                assert np.array_equal(signs[i, g], ws), (i, kv, g)
                assert np.array_equal(outs[i, g], wout), (i, kv, g)
                assert _scale_close(scales[i, g], wscale), (i, kv, g, scales[i, g], wscale)


def _edge_blocks(n_elem, rng):
    """Hot blocks that steer the encoder's threshold search into each of its
    paths: spikes well above the rest, ties at the threshold among a few
    dozen keys, more than 64 keys tied, an all-zero block, and signed zeros."""
    base = lambda: (0.1 * rng.standard_normal(n_elem)).astype(np.float32)
    out = []
    x = base(); x[rng.choice(n_elem, 16, replace=False)] = 40.0 + np.arange(16); out.append(x)
    x = base(); idx = rng.choice(n_elem, 30, replace=False)
    x[idx[:10]] = 9.0; x[idx[10:]] = -5.0; out.append(x)
    x = base(); x[rng.choice(n_elem, 100, replace=False)] = 5.0; out.append(x)
    out.append(np.zeros(n_elem, np.float32))
    x = base(); x[::7] = -0.0; x[rng.choice(n_elem, 70, replace=False)] = -3.0
    x[rng.choice(n_elem, 8, replace=False)] = 6.0; out.append(x)
    return out


def _encoder_path(x, k):
    """Which threshold search the encoder takes for a 2,048-element block of
    f32 values x (lane l holds chunks l + 64 j, j < 4, of 8 elements): its
    lower bound t0 is found over the 64 lane maxima, bit by bit from the top
    and stopping at the first prefix that exactly k maxima reach; the
    candidate search follows when t0 >= 1 and at most 64 keys reach t0, else
    the full-block search.  (Coverage bookkeeping for this test only.)"""
    keys = (x.astype(np.float32).view(np.uint32) & 0x7FFFFFFF).reshape(4, 64, 8)
    lane_max = keys.max(axis=(0, 2))
    any_bits = int(np.bitwise_or.reduce(lane_max))
    t0 = 0
    for b in range(30, -1, -1):
        if not (any_bits >> b) & 1:
            continue
        cand = t0 | (1 << b)
        c = int((lane_max >= cand).sum())
        if c >= k:
            t0 = cand
        if c == k:
            break
    return "candidates" if t0 >= 1 and int((keys >= t0).sum()) <= 64 else "full"


@pytest.mark.parametrize("hot,n_out", [("f16", 16), ("bf16", 16), ("bf16", 64), ("f16", 1)])
def test_archive_threshold_edge_cases(gpu, hot, n_out):
    """Constructed 2,048-element hot blocks, encoded into 1-bit slots, against
    the oracle's encoder: the outliers are the n_out largest magnitudes, ties
    taken in index order, whichever search the encoder takes."""
    w = _case(gpu, hot=hot, Hkv=2, P=16, D=128, ctx=(1300, 700), seed=5 + n_out)
    P, D, Hkv = w.page_tokens, w.head_dim, w.num_kv_heads
    hot_pages = [e for _, _, e in _full_pages_by_class(w, per_class=3)
                 if oracle.entry_class(e)[0] == 0]
    assert len(hot_pages) == 3
    rng = np.random.default_rng(17 + n_out)
    cases = _edge_blocks(P * D, rng)
    dt = torch.float16 if hot == "f16" else torch.bfloat16
    k = 0
    for e in hot_pages:
        slot = oracle.entry_class(e)[1]
        for pool in (w.k_pool, w.v_pool):
            for g in range(Hkv):
                x = torch.from_numpy(cases[k % len(cases)].reshape(P, D)).to(dt)
                pool[slot, g] = x.to(gpu)
                k += 1
    n = len(hot_pages)
    _add_b1_pool(w, n, n_out, gpu)
    src_np = np.array(hot_pages, dtype=np.uint32)
    dst_np = np.array([B1 | i for i in range(n)], dtype=np.uint32)
    host = oracle.HostView(w)
    paths = {_encoder_path(oracle.block_f32(w, int(e), g, kv, host=host).ravel(), n_out)
             for e in src_np for kv in ("k", "v") for g in range(Hkv)}
    if n_out == 16:
        assert paths == {"candidates", "full"}, paths
    prob = atlas.Problem(w)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    print(f"[archive edge cases {hot} K{n_out}] {n} pages, paths {sorted(paths)}", flush=True)
    atlas.atlas_demote_pages(prob.args, prob.tiers,
                             torch.from_numpy(src_np.view(np.int32)).to(gpu),
                             torch.from_numpy(dst_np.view(np.int32)).to(gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    for kv in ("k", "v"):
        signs = w.tiers[f"b1_{kv}"].cpu().numpy()
        scales = w.tiers[f"b1_{kv}_scale"].cpu().numpy()
        outs = w.tiers[f"b1_{kv}_out"].cpu().numpy().view(np.uint32)
        for i, e in enumerate(src_np):
            for g in range(Hkv):
                ws, wscale, wout = oracle.encode_1bit(
                    oracle.block_f32(w, int(e), g, kv, host=host).ravel(), n_out)
                assert np.array_equal(signs[i, g], ws), (i, kv, g)
                assert np.array_equal(outs[i, g], wout), (i, kv, g)
                assert _scale_close(scales[i, g], wscale), (i, kv, g, scales[i, g], wscale)


def _oracle_b1_pool(w, n, n_out, gpu, seed):
    """A 1-bit pool written on the host by the oracle's encoder from seeded
    blocks (normal values with a few large outliers and some exact ties)."""
    rng = np.random.default_rng(seed)
    Hkv, P, D = w.num_kv_heads, w.page_tokens, w.head_dim
    for kv in ("k", "v"):
        signs = np.zeros((n, Hkv, P * D // 8), np.uint8)
        scales = np.zeros((n, Hkv), np.float32)
        outs = np.zeros((n, Hkv, n_out), np.uint32)
        for i in range(n):
            for g in range(Hkv):
                x = rng.standard_normal(P * D).astype(np.float16).astype(np.float32)
                x[rng.integers(0, P * D, 12)] *= 40
                x[rng.integers(0, P * D, 30)] = 0.5
                signs[i, g], scales[i, g], outs[i, g] = oracle.encode_1bit(x, n_out)
        w.tiers[f"b1_{kv}"] = torch.from_numpy(signs).to(gpu)
        w.tiers[f"b1_{kv}_scale"] = torch.from_numpy(scales).to(gpu)
        w.tiers[f"b1_{kv}_out"] = torch.from_numpy(outs.view(np.int32)).to(gpu)


def _with_spare_blocks(w, extra):
    """Appends `extra` blocks (zeros) to the hot pool; returns their ids."""
    nb = w.num_blocks
    z = torch.zeros((extra,) + tuple(w.k_pool.shape[1:]), dtype=w.k_pool.dtype,
                    device=w.k_pool.device)
    w.k_pool = torch.cat([w.k_pool, z]).contiguous()
    w.v_pool = torch.cat([w.v_pool, z]).contiguous()
    return list(range(nb, nb + extra))


@pytest.mark.parametrize("hot", ["f16", "bf16"])
def test_promote_every_class_bit_exact(gpu, hot):
    w = _case(gpu, hot=hot, seed=17)
    n_out = 16
    _oracle_b1_pool(w, 3, n_out, gpu, seed=5)
    pages = [e for _, _, e in _full_pages_by_class(w)] + [B1 | 0, B1 | 2]
    dst = _with_spare_blocks(w, len(pages))
    host = oracle.HostView(w)
    want = {(i, kv, g): oracle.hot_bits(oracle.block_f32(w, e, g, kv, host=host), hot)
            for i, e in enumerate(pages) for kv in ("k", "v") for g in range(w.num_kv_heads)}
    prob = atlas.Problem(w)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    src = torch.from_numpy(np.array(pages, dtype=np.uint32).view(np.int32)).to(gpu)
    atlas.atlas_promote_pages(prob.args, prob.tiers, src,
                              torch.tensor(dst, dtype=torch.int32, device=gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    for kv, pool in (("k", w.k_pool), ("v", w.v_pool)):
        got = pool.cpu().view(torch.int16).numpy().view(np.uint16)
        for i, b in enumerate(dst):
            for g in range(w.num_kv_heads):
                assert np.array_equal(got[b, g], want[(i, kv, g)]), (i, kv, g)


def test_promote_rejections(gpu):
    w = _case(gpu, seed=23)
    _oracle_b1_pool(w, 1, 4, gpu, seed=1)
    dst = _with_spare_blocks(w, 3)
    before = w.k_pool[dst[2]].clone()
    prob = atlas.Problem(w)
    n_b1 = w.tiers["b1_k"].shape[0]
    src = np.array([B1 | n_b1, KIND3 | 0, B1 | 0], dtype=np.uint32)  # past the pool, kind 3, ok
    blocks = [dst[0], dst[1], w.num_blocks]  # the last names no block
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_promote_pages(prob.args, prob.tiers, torch.from_numpy(src.view(np.int32)).to(gpu),
                              torch.tensor(blocks, dtype=torch.int32, device=gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 3
    assert torch.isnan(w.k_pool[dst[0]].float()).all() and torch.isnan(w.v_pool[dst[1]].float()).all()
    assert torch.equal(w.k_pool[dst[2]], before)


def test_archive_rejections(gpu):
    """A source outside its pool poisons the 1-bit slot: after a valid
    archive into slot 1, archiving a bad source there makes every value of
    the slot NaN (no stale outlier survives).  A 1-bit source and a slot
    outside the pool are rejected with nothing written."""
    w = _case(gpu, seed=29)
    n_b1 = 3
    _add_b1_pool(w, n_b1, 8, gpu)
    hot = next(e for _, _, e in _full_pages_by_class(w) if oracle.entry_class(e)[0] == 0)
    prob = atlas.Problem(w)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)

    def demote(src, dst):
        atlas.atlas_demote_pages(
            prob.args, prob.tiers,
            torch.from_numpy(np.array(src, np.uint32).view(np.int32)).to(gpu),
            torch.from_numpy(np.array(dst, np.uint32).view(np.int32)).to(gpu), rej)

    demote([hot, hot], [B1 | 1, B1 | 2])
    torch.cuda.synchronize()
    assert int(rej) == 0
    before = {kv: [w.tiers[f"b1_{kv}{x}"][2].clone() for x in ("", "_scale", "_out")]
              for kv in ("k", "v")}
    demote([w.num_blocks, B1 | 0, hot], [B1 | 1, B1 | 2, B1 | n_b1])
    torch.cuda.synchronize()
    assert int(rej) == 3
    for kv in ("k", "v"):
        assert torch.isnan(w.tiers[f"b1_{kv}_scale"][1]).all()
        for t, x in zip(before[kv], ("", "_scale", "_out")):
            assert torch.equal(w.tiers[f"b1_{kv}{x}"][2], t), (kv, x)
    k = torch.empty((2, w.num_kv_heads, w.page_tokens, w.head_dim), device=gpu)
    v = torch.empty_like(k)
    ent = torch.from_numpy(np.array([B1 | 1, B1 | 2], np.uint32).view(np.int32)).to(gpu)
    atlas.atlas_dequant_pages(prob.args, prob.tiers, ent, k, v)
    torch.cuda.synchronize()
    assert torch.isnan(k[0]).all() and torch.isnan(v[0]).all()
    assert torch.isfinite(k[1]).all() and torch.isfinite(v[1]).all()


def test_dequant_1bit_bit_exact(gpu):
    w = _case(gpu, seed=31)
    _oracle_b1_pool(w, 4, 64, gpu, seed=9)
    prob = atlas.Problem(w)
    ent = np.array([B1 | i for i in range(4)], dtype=np.uint32)
    k = torch.empty((4, w.num_kv_heads, w.page_tokens, w.head_dim), device=gpu)
    v = torch.empty_like(k)
    atlas.atlas_dequant_pages(prob.args, prob.tiers, torch.from_numpy(ent.view(np.int32)).to(gpu),
                              k, v)
    torch.cuda.synchronize()
    host = oracle.HostView(w)
    for i, e in enumerate(ent):
        for got, kv in ((k[i], "k"), (v[i], "v")):
            want = np.stack([oracle.block_f32(w, int(e), g, kv, host=host)
                             for g in range(w.num_kv_heads)])
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), i


@pytest.mark.parametrize("kernel", ["default", "valu"])
def test_attention_refuses_1bit_entries(gpu, monkeypatch, kernel):
    if kernel == "valu":
        monkeypatch.setenv("ATLAS_DECODE_VALU", "1")
    w = _case(gpu, seed=47)
    _oracle_b1_pool(w, 2, 8, gpu, seed=2)
    prob = atlas.Problem(w)
    assert prob.validate() == [0, 0, 0, 0]
    prob.table[0, 3] = int(np.uint32(B1 | 1).view(np.int32))
    assert prob.validate()[0] == 1
    out, lse = prob.run()
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isfinite(out[1]).all()


def _bits16(t):
    """Raw 16-bit patterns of an f16 / bf16 tensor as uint16."""
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _rebuilt_matches(got, want, same_scale):
    """A reconstructed block against the oracle's reconstruction of its own
    encoding: bit-exact when the device's scale equals the oracle's, else
    (one f32 ulp apart, which the encoding allows) every +-scale element may
    round to the neighbouring 16-bit value; the FP16 outliers are exact."""
    if same_scale:
        return np.array_equal(got, want)
    return int(np.abs(got.astype(np.int32) - want.astype(np.int32)).max()) <= 1


@pytest.mark.parametrize("hot", ["f16", "bf16"])
def test_archive_then_promote_then_attend(gpu, hot):
    """The ARGUS loop for deep-cold pages: archive hot and cold pages into
    1-bit slots, reconstruct them into hot blocks, attend.  Expected values
    come from the oracle alone: its encoding of each source block, decoded
    and rounded to the hot type, checked against the reconstruction; the
    attention is checked against the oracle over a pool holding those
    oracle blocks."""
    w = _case(gpu, hot=hot, ctx=(1100, 2300), seed=53)
    pages = _full_pages_by_class(w, per_class=3)
    n, n_out = len(pages), 16
    host = oracle.HostView(w)
    blocks = {(i, kv, g): oracle.block_f32(w, e, g, kv, host=host).ravel()
              for i, (_, _, e) in enumerate(pages) for kv in ("k", "v")
              for g in range(w.num_kv_heads)}
    _add_b1_pool(w, n, n_out, gpu)
    dst = _with_spare_blocks(w, n)
    prob = atlas.Problem(w)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    src = torch.from_numpy(np.array([e for _, _, e in pages], np.uint32).view(np.int32)).to(gpu)
    b1 = torch.from_numpy(np.array([B1 | i for i in range(n)], np.uint32).view(np.int32)).to(gpu)
    atlas.atlas_demote_pages(prob.args, prob.tiers, src, b1, rej)
    atlas.atlas_promote_pages(prob.args, prob.tiers, b1,
                              torch.tensor(dst, dtype=torch.int32, device=gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    exp_pool = {"k": w.k_pool.clone(), "v": w.v_pool.clone()}
    for (i, kv, g), x in blocks.items():
        ws, wscale, wout = oracle.encode_1bit(x, n_out)
        want = oracle.hot_bits(oracle.decode_1bit(ws, wscale, wout, x.size), hot)
        want = want.reshape(w.page_tokens, w.head_dim)
        pool = w.k_pool if kv == "k" else w.v_pool
        same = float(w.tiers[f"b1_{kv}_scale"][i, g]) == float(np.float32(wscale))
        assert _rebuilt_matches(_bits16(pool[dst[i], g]), want, same), (i, kv, g)
        exp_pool[kv][dst[i], g] = torch.from_numpy(want.view(np.int16)).to(gpu).view(pool.dtype)
    table = w.page_table.copy()
    for i, (s, p, _) in enumerate(pages):
        table[s, p] = dst[i]
    w.page_table = table
    out, lse = run(w)
    ref = copy.copy(w)
    ref.k_pool, ref.v_pool = exp_pool["k"], exp_pool["v"]
    check(ref, out, lse)


def test_archive_and_promote_full_size_sampled(gpu):
    """The benchmarked archive and promote, in the launch configuration the
    benchmark times: every full page of the 64-sequence bf16 GQA decode
    workload archived into 1-bit slots with 16 outliers, then rebuilt into
    the blocks it came from.  Sampled (page, kv head) blocks, the first and
    the last included, against the oracle's encoding of the source block
    (signs and outliers bit-exact, scale within one f32 ulp) and against the
    oracle's reconstruction of that encoding."""
    import bench
    w = synth.config(3, device=gpu, seed=42)
    Hkv, P, D, K = w.num_kv_heads, w.page_tokens, w.head_dim, 16
    src, _, _, _ = bench.demote_plan(w)
    n = len(src)
    tiers = {}
    for kv in ("k", "v"):
        for t in ("i8", "i4"):
            tiers[f"{t}_{kv}"] = torch.empty((0,), dtype=torch.uint8, device=gpu)
            tiers[f"{t}_{kv}_scale"] = torch.empty((0,), dtype=torch.float32, device=gpu)
        tiers[f"b1_{kv}"] = torch.full((n, Hkv, P * D // 8), 0xAA, dtype=torch.uint8, device=gpu)
        tiers[f"b1_{kv}_scale"] = torch.full((n, Hkv), -1.0, device=gpu)
        tiers[f"b1_{kv}_out"] = torch.full((n, Hkv, K), -1, dtype=torch.int32, device=gpu)
    pools = atlas.make_tiers(tiers)
    prob = atlas.Problem(w)
    src_t = torch.from_numpy(src).to(gpu)
    b1_t = torch.from_numpy((np.arange(n, dtype=np.int64) | B1).astype(np.uint32)
                            .view(np.int32)).to(gpu)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    print(f"[archive/promote full size] {n} pages x {Hkv} kv heads", flush=True)
    atlas.atlas_demote_pages(prob.args, pools, src_t, b1_t, rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    for kv in ("k", "v"):
        assert bool((tiers[f"b1_{kv}_scale"] >= 0).all()), kv
    host = oracle.HostView(w)
    (ka, kind), (va, _) = host.pools()  # the source blocks, before the rebuild
    rng = np.random.default_rng(5)
    pick = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 40)]))
    want = {}
    for i in pick:
        for arr, kv in ((ka, "k"), (va, "v")):
            signs = tiers[f"b1_{kv}"][i].cpu().numpy()
            scales = tiers[f"b1_{kv}_scale"][i].cpu().numpy()
            outs = tiers[f"b1_{kv}_out"][i].cpu().numpy().view(np.uint32)
            for g in range(Hkv):
                x = oracle.widen_bits(arr[int(src[i]), g], kind).astype(np.float32).ravel()
                ws, wscale, wout = oracle.encode_1bit(x, K)
                assert np.array_equal(signs[g], ws), (i, kv, g)
                assert np.array_equal(outs[g], wout), (i, kv, g)
                assert _scale_close(scales[g], wscale), (i, kv, g, scales[g], wscale)
                rebuilt = oracle.hot_bits(oracle.decode_1bit(ws, wscale, wout, x.size), "bf16")
                want[(i, kv, g)] = (rebuilt.reshape(P, D), scales[g] == np.float32(wscale))
    atlas.atlas_promote_pages(prob.args, pools, b1_t, src_t, rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    for (i, kv, g), (rebuilt, same) in want.items():
        pool = w.k_pool if kv == "k" else w.v_pool
        assert _rebuilt_matches(_bits16(pool[int(src[i]), g]), rebuilt, same), (i, kv, g)


def test_promote_into_an_f32_hot_pool(gpu):
    """Reconstruction into f32 blocks: every class's values exactly (no
    rounding step), through a pool of another element type than the one the
    pages were demoted from."""
    w = _case(gpu, seed=61)
    _oracle_b1_pool(w, 2, 8, gpu, seed=4)
    pages = [e for _, _, e in _full_pages_by_class(w) if oracle.entry_class(e)[0] != 0]
    pages += [B1 | 0, B1 | 1]
    n = len(pages)
    pool_k = torch.zeros((n, w.num_kv_heads, w.page_tokens, w.head_dim), device=gpu)
    pool_v = torch.zeros_like(pool_k)
    dummy_q = torch.zeros((1, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=gpu)
    args = atlas.make_args(q=dummy_q, k_pool=pool_k, v_pool=pool_v,
                           page_table=torch.zeros((1, 4), dtype=torch.int32, device=gpu),
                           context_lens=torch.ones(1, dtype=torch.int32, device=gpu),
                           num_heads=w.num_heads, num_kv_heads=w.num_kv_heads,
                           head_dim=w.head_dim, page_tokens=w.page_tokens, max_context_len=1,
                           scale=0.1, out=torch.empty((1, w.num_heads, w.head_dim), device=gpu),
                           lse=torch.empty((1, w.num_heads), device=gpu), kv_dtype=atlas.F32,
                           q_dtype=atlas.BF16)
    tiers = atlas.make_tiers(w.tiers)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_promote_pages(args, tiers,
                              torch.from_numpy(np.array(pages, np.uint32).view(np.int32)).to(gpu),
                              torch.arange(n, dtype=torch.int32, device=gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    host = oracle.HostView(w)
    for kv, pool in (("k", pool_k), ("v", pool_v)):
        got = pool.cpu().numpy()
        for i, e in enumerate(pages):
            for g in range(w.num_kv_heads):
                want = oracle.hot_bits(oracle.block_f32(w, e, g, kv, host=host), "f32")
                assert np.array_equal(got[i, g].view(np.uint32), want), (i, kv, g)
