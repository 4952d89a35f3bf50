"""GPU parity: the HIP path (through the C ABI) against the f64 oracle.

Tolerances (max-abs on out and on lse): 2e-5 for f32 K/V, 2e-3 for bf16 /
f16 / int8 / int4 / regenerated K/V, all with f32 accumulation.  Integer and
byte-level steps (page gather, regenerated values, tier decoding) must match
bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from tests.paging import relayout

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 2e-3, "f16": 2e-3}


def _tol(w):
    if w.tiers is not None or w.regen is not None:
        return 2e-3
    return TOL[w.kv_dtype]


def run(w, split_tokens=0, fill=True):
    prob = atlas.Problem(w, split_tokens=split_tokens)
    if w.regen is not None and fill:
        prob.fill_resident_from_regenerator()
    out, lse = prob.run()
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(w, out, lse, rows=None, heads=None, tol=None, host=None):
    tol = _tol(w) if tol is None else tol
    rows = np.arange(w.total_q) if rows is None else np.asarray(rows)
    heads = np.arange(w.num_heads) if heads is None else np.asarray(heads)
    ref_o, ref_l = oracle.reference(w, rows=rows, heads=heads, host=host)
    got_o = out[rows][:, heads]
    got_l = lse[rows][:, heads]
    assert np.all(np.isfinite(got_o)), "non-finite output"
    finite = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), finite)
    eo = float(np.max(np.abs(got_o - ref_o))) if got_o.size else 0.0
    el = float(np.max(np.abs(got_l[finite] - ref_l[finite]))) if finite.any() else 0.0
    print(f"[{w.name or 'case'}] max|out-ref|={eo:.3e} max|lse-ref|={el:.3e} tol={tol:g}",
          flush=True)
    assert eo <= tol and el <= tol
    return eo, el


def cuda():
    return torch.device("cuda:0")


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def test_config1_full(gpu):
    w = synth.config(1, device=gpu)
    out, lse = run(w)
    check(w, out, lse)


def test_config2_reduced_all_heads(gpu):
    w = synth.config(2, device=gpu, context_lens=5000)
    out, lse = run(w)
    check(w, out, lse)


def test_config2_full_sampled_heads(gpu):
    w = synth.config(2, device=gpu)
    out, lse = run(w)
    check(w, out, lse, heads=[0, 7, 19, 31])


def test_config3_reduced(gpu):
    w = synth.config(3, device=gpu, num_seqs=10,
                     context_lens=[1, 15, 16, 17, 300, 1023, 1024, 2049, 4000, 777])
    out, lse = run(w)
    check(w, out, lse)


def test_config3_full_sampled(gpu):
    w = synth.config(3, device=gpu)
    out, lse = run(w)
    seqs = [0, 13, 37, 63, int(np.argmax(w.context_lens))]
    check(w, out, lse, rows=seqs, heads=[0, 5, 17, 31])


def test_config4_reduced(gpu):
    w = synth.config(4, device=gpu, num_seqs=6, context_lens=[5, 1000, 1030, 2500, 4097, 3000])
    counts = w.tiers["counts"]
    assert counts[1] > 0 and counts[2] > 0
    out, lse = run(w)
    check(w, out, lse)


def test_config4_full_sampled(gpu):
    w = synth.config(4, device=gpu)
    out, lse = run(w)
    seqs = [1, 22, 50, int(np.argmax(w.context_lens))]
    check(w, out, lse, rows=seqs, heads=[0, 9, 30])


def test_config5_reduced_prefill_with_regen(gpu):
    w = synth.config(5, device=gpu, context_lens=3000, query_lens=200, num_heads=16,
                     num_kv_heads=2)
    out, lse = run(w)
    check(w, out, lse, rows=[0, 1, 57, 100, 199])


# ---------------------------------------------------------------------------
# Shapes, head maps, splits, prefill rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 4), (8, 2), (8, 1)])
def test_head_maps_dtypes_dims(gpu, kv, D, H, Hkv):
    w = synth.build(dict(num_seqs=3, context_lens=[70, 513, 1200], num_heads=H,
                         num_kv_heads=Hkv, head_dim=D, page_tokens=32, kv_dtype=kv,
                         placement="permuted"), device=gpu, seed=D + H + Hkv,
                    name=f"{kv}-D{D}-H{H}/{Hkv}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("split", [64, 128, 512, 2048])
def test_split_sizes(gpu, split):
    w = synth.build(dict(num_seqs=2, context_lens=[3001, 64], num_heads=8, num_kv_heads=2,
                         head_dim=128, page_tokens=16, kv_dtype="bf16"), device=gpu, seed=5,
                    name=f"split{split}")
    out, lse = run(w, split_tokens=split)
    check(w, out, lse)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_chunked_prefill_rows(gpu, kv):
    w = synth.build(dict(num_seqs=3, context_lens=[50, 700, 333], query_lens=[50, 37, 5],
                         num_heads=8, num_kv_heads=2, head_dim=64, page_tokens=16,
                         kv_dtype=kv), device=gpu, seed=9, name=f"prefill-{kv}")
    out, lse = run(w)
    check(w, out, lse)


def test_regen_decode_rows(gpu):
    w = synth.build(dict(num_seqs=3, context_lens=[900, 17, 2050], num_heads=8,
                         num_kv_heads=2, head_dim=128, page_tokens=64, kv_dtype="bf16",
                         regen=dict(seed=7, layer=3, fraction=0.75)), device=gpu, seed=3,
                    name="regen-decode")
    out, lse = run(w)
    check(w, out, lse)


# ---------------------------------------------------------------------------
# Invariants: determinism, page size, placement, regen vs resident
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", ["default", "valu"])
@pytest.mark.parametrize("P,split", [(16, 0), (16, 64), (64, 128), (256, 64), (256, 0)])
@pytest.mark.parametrize("H,Hkv,hot", [(8, 4, "f16"), (8, 2, "f16"), (16, 2, "f16"),
                                       (8, 2, "bf16")])
def test_tiered_page_walk(gpu, monkeypatch, kernel, P, split, H, Hkv, hot):
    """Tiered splits visit their pages grouped by tier; splits that start
    inside a page (page 256, split 64) mask the tokens before their start."""
    if kernel == "valu":
        monkeypatch.setenv("ATLAS_DECODE_VALU", "1")
    w = synth.build(dict(num_seqs=4, context_lens=[37, 700, 1500, 2600], num_heads=H,
                         num_kv_heads=Hkv, head_dim=128, page_tokens=P, q_dtype="bf16",
                         kv_dtype=hot, placement="permuted",
                         tiers=dict(hot_tokens=300, p_int8=0.5)),
                    device=gpu, seed=P + split + H + Hkv, name=f"tiered-P{P}-s{split}-{H}/{Hkv}")
    counts = w.tiers["counts"]
    assert counts[1] > 0 and counts[2] > 0
    o1, l1 = run(w, split_tokens=split)
    check(w, o1, l1)
    o2, l2 = run(w, split_tokens=split)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("H,cold", [(8, "i4"), (16, "i4"), (8, "i8"), (16, "i8"), (8, "i2"),
                                    (16, "i2")])
def test_tiered_cold_spike_large_v_scale(gpu, H, cold):
    """A cold key scoring 7.5 log2 units above every earlier key (just under
    the lazy-rescale threshold) on a page with a V scale far above 1: p *
    scale must stay a finite f16 operand.  q is the unit vector of dim 0, so
    each score is dim 0 of its key; hot keys and all but one cold page score
    about 0."""
    w = synth.build(dict(num_seqs=1, context_lens=[4096], num_heads=H, num_kv_heads=2,
                         head_dim=128, page_tokens=64, q_dtype="bf16", kv_dtype="f16",
                         placement="permuted",
                         tiers=dict(hot_tokens=1024, p_int8=1.0 if cold == "i8" else 0.0,
                                    p_int2=1.0 if cold == "i2" else 0.0)),
                    device=gpu, seed=5, name=f"tiered-spike-{cold}-H{H}")
    t = w.tiers
    w.q.zero_()
    w.q[..., 0] = 1.0
    w.k_pool[..., 0] = 0.0  # hot scores 0 (poisoned rows keep NaN elsewhere)
    # dim-0 codes of every cold slot, [n][Hkv][P]
    raw = t[f"{cold}_k"][..., 0].to(torch.int16)
    if cold == "i4":
        code0 = ((raw & 0xF) ^ 0x8) - 0x8
    elif cold == "i2":
        code0 = ((raw & 0x3) ^ 0x2) - 0x2
    else:
        code0 = raw
    ent = w.page_table[0].view(np.uint32)
    if cold == "i2":  # extension tier 3, kind 1, 28-bit slot
        cold_slots = [int(e & ((1 << 28) - 1)) for e in ent
                      if (e >> 30) == 3 and ((e >> 28) & 3) == 1]
    else:
        tier = 2 if cold == "i4" else 1
        cold_slots = [int(e & ((1 << 30) - 1)) for e in ent if (e >> 30) == tier]
    assert len(cold_slots) > 4
    spike = cold_slots[-1]  # the newest cold page
    c = w.scale * np.log2(np.e)  # score (log2 units) per unit of q.k
    ks = t[f"{cold}_k_scale"]
    ks.mul_(1e-3)  # other cold pages score about 0
    for h in range(2):
        top = float(code0[spike, h].max())
        assert top > 0
        ks[spike, h] = 7.5 / (top * c)
    vmul = {"i4": 64.0, "i8": 256.0, "i2": 8.0}[cold]
    qmax = {"i4": 7, "i8": 127, "i2": 1}[cold]
    t[f"{cold}_v_scale"].mul_(vmul)
    out, lse = run(w, split_tokens=8192)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    ref_o, ref_l = oracle.reference(w)
    vmax = float(t[f"{cold}_v_scale"].max()) * qmax
    tol_o = 2e-3 * max(1.0, vmax / 4.0)
    eo = float(np.max(np.abs(out - ref_o)))
    el = float(np.max(np.abs(lse - ref_l)))
    print(f"[{w.name}] max|out-ref|={eo:.3e} (tol {tol_o:.3g}, max|v| {vmax:.1f}) "
          f"max|lse-ref|={el:.3e}", flush=True)
    assert eo <= tol_o and el <= 2e-3


def test_determinism_bitwise(gpu):
    w = synth.config(3, device=gpu, num_seqs=6, context_lens=("uniform", 100, 5000))
    o1, l1 = run(w)
    o2, l2 = run(w)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("kv,D", [("bf16", 128), ("f32", 64)])
def test_page_size_and_placement_do_not_change_bits(gpu, kv, D):
    w = synth.build(dict(num_seqs=4, context_lens=[1, 100, 1500, 2600], num_heads=8,
                         num_kv_heads=2, head_dim=D, page_tokens=16, kv_dtype=kv),
                    device=gpu, seed=21, name="pagesize")
    o0, l0 = run(w, split_tokens=512)
    check(w, o0, l0)
    for P, seed, spare in ((16, 1, 5), (32, 2, 0), (64, 3, 9), (256, 4, 1), (512, 5, 0)):
        w2 = relayout(w, P, seed, spare_blocks=spare)
        o2, l2 = run(w2, split_tokens=512)
        assert np.array_equal(o0.view(np.uint32), o2.view(np.uint32)), P
        assert np.array_equal(l0.view(np.uint32), l2.view(np.uint32)), P


def test_regenerated_equals_resident_bitwise(gpu):
    # CFR-Atlas contract: when regeneration reproduces the stored rows, the
    # folded result equals the all-resident result.
    base = dict(num_seqs=2, context_lens=[1000, 2100], num_heads=8, num_kv_heads=2,
                head_dim=128, page_tokens=64, kv_dtype="bf16")
    w_regen = synth.build(dict(base, regen=dict(seed=11, layer=1, fraction=0.75)),
                          device=gpu, seed=4)
    w_res = synth.build(dict(base, regen=dict(seed=11, layer=1, fraction=0.0)),
                        device=gpu, seed=4)
    o1, l1 = run(w_regen, split_tokens=512)
    o2, l2 = run(w_res, split_tokens=512)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    check(w_regen, o1, l1)


# ---------------------------------------------------------------------------
# Edge cases and loud failures
# ---------------------------------------------------------------------------

def test_empty_and_single_token_contexts(gpu):
    w = synth.build(dict(num_seqs=3, context_lens=[0, 1, 2], num_heads=4, num_kv_heads=2,
                         head_dim=64, page_tokens=16, kv_dtype="f32"), device=gpu, seed=2)
    out, lse = run(w)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    v0 = w.v_pool[int(w.page_table[1, 0])][:, 0].cpu().numpy()  # [Hkv][D]
    assert np.array_equal(out[1], v0[np.arange(4) // 2])
    check(w, out, lse, rows=[1, 2])


def test_identical_v_rows_return_that_row(gpu):
    w = synth.build(dict(num_seqs=2, context_lens=[3000, 50], num_heads=4, num_kv_heads=1,
                         head_dim=128, page_tokens=16, kv_dtype="bf16"), device=gpu, seed=8)
    row = torch.randn(128, device=gpu).to(torch.bfloat16)
    w.v_pool[:] = row
    out, _ = run(w)
    np.testing.assert_allclose(out, np.broadcast_to(row.float().cpu().numpy(), out.shape),
                               rtol=0, atol=1e-6)


def test_bad_page_ids_and_context_lengths_give_nan(gpu):
    w = synth.build(dict(num_seqs=3, context_lens=[100, 200, 300], num_heads=4,
                         num_kv_heads=2, head_dim=64, page_tokens=16, kv_dtype="f32"),
                    device=gpu, seed=6)
    w.page_table[1, 3] = w.num_blocks + 7   # outside the pool: guarded, row -> NaN
    w.page_table[2, 0] = -5
    out, lse = run(w)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert np.all(np.isnan(out[2])) and np.all(np.isnan(lse[2]))
    check(w, out, lse, rows=[0])
    # a context longer than the host bound: guarded, row -> NaN, others intact
    w2 = synth.build(dict(num_seqs=2, context_lens=[100, 200], num_heads=4, num_kv_heads=2,
                          head_dim=64, page_tokens=16, kv_dtype="f32", max_pages=16),
                     device=gpu, seed=6)
    prob = atlas.Problem(w2)
    prob.args.max_context_len = 150
    prob.ctx[1] = 200
    out2, lse2 = prob.run()
    torch.cuda.synchronize()
    assert torch.isnan(out2[1]).all() and torch.isnan(lse2[1]).all()
    assert torch.isfinite(out2[0]).all()


# ---------------------------------------------------------------------------
# Bit-exact inspection entry points
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv", ["f32", "bf16", "f16"])
def test_gather_pages_bit_exact(gpu, kv):
    w = synth.build(dict(num_seqs=3, context_lens=[33, 1000, 517], num_heads=8,
                         num_kv_heads=4, head_dim=64, page_tokens=16, kv_dtype=kv),
                    device=gpu, seed=31)
    prob = atlas.Problem(w)
    host = oracle.HostView(w)
    for s in range(3):
        n = int(w.context_lens[s])
        k = torch.empty((n, 4, 64), device=gpu, dtype=w.k_pool.dtype)
        v = torch.empty_like(k)
        atlas.atlas_gather_pages(prob.args, s, n, k, v)
        torch.cuda.synchronize()
        for g in range(4):
            K, V = oracle.logical_kv(w, s, g, host=host)
            assert np.array_equal(k[:, g].double().cpu().numpy(), K)
            assert np.array_equal(v[:, g].double().cpu().numpy(), V)


@pytest.mark.parametrize("kv_name,code", [("bf16", atlas.BF16), ("f32", atlas.F32)])
def test_regenerate_pages_bit_exact(gpu, kv_name, code):
    Hkv, D, P = 3, 128, 32
    logical = torch.tensor([0, 5, 2, 1000], dtype=torch.int32, device=gpu)
    blocks = torch.tensor([3, 0, 1, 2], dtype=torch.int32, device=gpu)
    dt = synth.DTYPES[kv_name]
    kp = torch.full((4, Hkv, P, D), float("nan"), dtype=dt, device=gpu)
    vp = torch.full_like(kp, float("nan"))
    atlas.atlas_regenerate_pages(123456789, 5, Hkv, D, P, code, logical, blocks, 4, kp, vp)
    torch.cuda.synchronize()
    for lp, b in zip(logical.tolist(), blocks.tolist()):
        for g in range(Hkv):
            for kv, pool in ((0, kp), (1, vp)):
                ref = oracle.regen_values(123456789, 5, g, lp * P, P, D, kv)
                got = pool[b, g].float().cpu().numpy()
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_regenerate_config5_pages_bit_exact(gpu):
    # every value of four regenerated pages of the 2,048-query prefill, all kv heads
    Hkv, D, P = 8, 128, 256
    lps = [0, 1, 200, 383]
    logical = torch.tensor(lps, dtype=torch.int32, device=gpu)
    blocks = torch.arange(4, dtype=torch.int32, device=gpu)
    kp = torch.empty((4, Hkv, P, D), dtype=torch.bfloat16, device=gpu)
    vp = torch.empty_like(kp)
    atlas.atlas_regenerate_pages(42, 0, Hkv, D, P, atlas.BF16, logical, blocks, 4, kp, vp)
    torch.cuda.synchronize()
    for i, lp in enumerate(lps):
        for g in range(Hkv):
            for kv, pool in ((0, kp), (1, vp)):
                ref = oracle.regen_values(42, 0, g, lp * P, P, D, kv)
                got = pool[i, g].float().cpu().numpy()
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_regenerate_config5_all_pages_bit_exact(gpu):
    """Every regenerated element of the 2,048-query prefill: 384 pages x 8 kv
    heads x 256 tokens x 128 dims, K and V (201,326,592 values), from the
    page regenerator, against the oracle's SplitMix64 stream bit for bit."""
    Hkv, D, P, n = 8, 128, 256, 384
    logical = torch.arange(n, dtype=torch.int32, device=gpu)
    blocks = torch.arange(n, dtype=torch.int32, device=gpu)
    kp = torch.empty((n, Hkv, P, D), dtype=torch.bfloat16, device=gpu)
    vp = torch.empty_like(kp)
    atlas.atlas_regenerate_pages(42, 0, Hkv, D, P, atlas.BF16, logical, blocks, n, kp, vp)
    torch.cuda.synchronize()
    checked = 0
    for g in range(Hkv):
        for kv, pool in ((0, kp), (1, vp)):
            ref = oracle.regen_values(42, 0, g, 0, n * P, D, kv)
            got = pool[:, g].reshape(n * P, D).float().cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (g, kv)
            checked += got.size
    assert checked == 201_326_592


def test_prefill_window_ring_holds_regenerated_values(gpu):
    """The values the matrix-core prefill folds: with one window covering the
    whole 131,072-token context of the 2,048-query workload, the workspace
    ring holds every key of the window after the call -- K as stored (bf16)
    [kv head][key][dim], V converted to f16 and stored per 64-key tile
    dims-major, [kv head][tile][dim][slot], key 16 (s / 16) + t(s % 16) in
    slot s, t swapping bits 2 and 3.  Its regenerated rows (the oldest 98,304
    keys) must equal the oracle's stream bit for bit (V through a
    round-to-nearest f16 conversion of the oracle's value).  The ring layout
    is internal to the library; this test reads it on purpose."""
    w = synth.config(5, device=gpu)
    ctx = int(w.context_lens[0])
    prob = atlas.Problem(w, split_tokens=ctx)
    out, lse = prob.run()
    torch.cuda.synchronize()
    Hkv, D = w.num_kv_heads, w.head_dim
    n_regen = int(w.regen["regen_pages"][0]) * w.page_tokens
    assert n_regen == 98_304
    ring = prob.args.workspace_bytes // 2
    ws = prob.workspace
    rk = ws[:Hkv * ctx * D * 2].view(torch.int16).view(Hkv, ctx, D)
    rvt = ws[ring:ring + Hkv * ctx * D * 2].view(torch.float16).view(Hkv, ctx // 64, D, 64)
    slot = np.arange(64)
    slot = (slot & ~12) | ((slot & 4) << 1) | ((slot & 8) >> 1)  # key k sits in slot slot[k]
    rv = rvt.permute(0, 1, 3, 2)[:, :, torch.from_numpy(slot).to(gpu), :].reshape(Hkv, ctx, D)
    for g in range(Hkv):
        ref_k = oracle.regen_values(42, 0, g, 0, n_regen, D, 0)
        ref_v = oracle.regen_values(42, 0, g, 0, n_regen, D, 1)
        got_k = rk[g, :n_regen].cpu().numpy().view(np.uint16)
        assert np.array_equal(got_k, (ref_k.view(np.uint32) >> 16).astype(np.uint16)), g
        got_v = rv[g, :n_regen].cpu().numpy()
        assert np.array_equal(got_v.view(np.uint16), ref_v.astype(np.float16).view(np.uint16)), g


def test_dequant_pages_bit_exact(gpu):
    w = synth.config(4, device=gpu, num_seqs=3, context_lens=[3000, 2000, 1500])
    prob = atlas.Problem(w)
    entries_np = np.concatenate([w.page_table[s, :w.pages_of(s)] for s in range(3)])
    entries = torch.from_numpy(entries_np).to(gpu)
    n = entries.numel()
    k = torch.empty((n, 8, 16, 128), device=gpu)
    v = torch.empty_like(k)
    atlas.atlas_dequant_pages(prob.args, prob.tiers, entries, k, v)
    torch.cuda.synchronize()
    host = oracle.HostView(w)
    ta = host.tier_arrays()
    (hk, kind), (hv, _) = host.pools()
    kc, vc = k.cpu().numpy(), v.cpu().numpy()
    for i, e in enumerate(entries_np.view(np.uint32)):
        tier, slot = int(e) >> 30, int(e) & ((1 << 30) - 1)
        if tier == 0:
            rk = oracle.widen_bits(hk[slot], kind).astype(np.float32)
            rv = oracle.widen_bits(hv[slot], kind).astype(np.float32)
        else:
            key = "i8" if tier == 1 else "i4"
            ck, cv = ta[f"{key}_k"][slot], ta[f"{key}_v"][slot]
            if key == "i4":
                ck, cv = oracle.int4_codes(ck), oracle.int4_codes(cv)
            rk = oracle.dequant_f32(ck[None], ta[f"{key}_k_scale"][slot][None])[0]
            rv = oracle.dequant_f32(cv[None], ta[f"{key}_v_scale"][slot][None])[0]
        ok_k = np.array_equal(kc[i].view(np.uint32), rk.view(np.uint32)) or \
            (tier == 0 and np.array_equal(np.isnan(kc[i]), np.isnan(rk)) and
             np.array_equal(kc[i][~np.isnan(rk)], rk[~np.isnan(rk)]))
        ok_v = np.array_equal(vc[i].view(np.uint32), rv.view(np.uint32)) or \
            (tier == 0 and np.array_equal(np.isnan(vc[i]), np.isnan(rv)) and
             np.array_equal(vc[i][~np.isnan(rv)], rv[~np.isnan(rv)]))
        assert ok_k and ok_v, (i, tier)


@pytest.mark.parametrize("lse_std", [4.0, 20.0])
def test_fold_partials_matches_oracle_merge(gpu, lse_std):
    """Max-abs 2e-5 on out and on lse against the f64 merge.  Partial lse
    values of attention are log-sums of up to 2^17 weights (|lse| <~ 16 in
    scaled units); with lse_std 20 (|lse| up to ~80) an f32 lse cannot be
    closer than half an ulp (3.8e-6 at 64), so there lse is held to 2e-5 or
    4 ulp of its magnitude, whichever is larger, and out stays at 2e-5."""
    rng = np.random.default_rng(17)
    splits, rows, D = 7, 300, 128
    po = rng.standard_normal((splits, rows, D)).astype(np.float32)
    pl = (rng.standard_normal((splits, rows)) * lse_std).astype(np.float32)
    pl[rng.random((splits, rows)) < 0.3] = -np.inf
    pl[:, 5] = -np.inf   # an all-empty row
    out = torch.empty((rows, D), device=gpu)
    lse = torch.empty(rows, device=gpu)
    atlas.atlas_fold_partials(torch.from_numpy(po).to(gpu), torch.from_numpy(pl).to(gpu),
                              out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_splits(po, pl)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(o[5] == 0) and l[5] == -np.inf
    fin = np.isfinite(ref_l)
    eo = float(np.max(np.abs(o - ref_o)))
    el = np.abs(l[fin] - ref_l[fin])
    bound = np.maximum(2e-5, 4.0 * np.spacing(np.abs(ref_l[fin]).astype(np.float32)))
    print(f"fold lse_std {lse_std}: max|out-ref| {eo:.3e}, max|lse-ref| {el.max():.3e}",
          flush=True)
    assert eo <= 2e-5
    assert np.all(el <= bound)
    if lse_std <= 4.0:
        assert float(el.max()) <= 2e-5
    # a single split is the identity
    out1 = torch.empty((rows, D), device=gpu)
    lse1 = torch.empty(rows, device=gpu)
    atlas.atlas_fold_partials(torch.from_numpy(po[:1]).to(gpu),
                              torch.from_numpy(np.where(np.isfinite(pl[:1]), pl[:1], 0.0)
                                               .astype(np.float32)).to(gpu), out1, lse1)
    torch.cuda.synchronize()
    assert np.array_equal(out1.cpu().numpy(), po[0])


# ---------------------------------------------------------------------------
# Chunked prefill on the matrix cores (bf16 / f16, head_dim 128)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv", ["bf16", "f16"])
@pytest.mark.parametrize("H,Hkv", [(8, 8), (8, 4), (8, 2), (16, 2)])
def test_mfma_prefill_shapes(gpu, kv, H, Hkv):
    w = synth.build(dict(num_seqs=3, context_lens=[300, 77, 1500], query_lens=[300, 20, 133],
                         num_heads=H, num_kv_heads=Hkv, head_dim=128, page_tokens=16,
                         kv_dtype=kv), device=gpu, seed=H * 10 + Hkv, name=f"mfma-{kv}-{H}/{Hkv}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("kv,split", [("bf16", 64), ("bf16", 192), ("f16", 128), ("bf16", 1024)])
def test_mfma_prefill_small_windows(gpu, kv, split):
    """The keys folded window by window through the ring (split_tokens keys
    per window, each window after the first merged into out / lse), with
    ragged contexts and chunks: a window shorter than the query chunk, windows
    that end inside a chunk's causal diagonal, and (bf16, the regenerator's
    type) a regenerated prefix."""
    spec = dict(num_seqs=3, context_lens=[1000, 333, 1777], query_lens=[200, 333, 77],
                num_heads=16, num_kv_heads=2, head_dim=128, page_tokens=16, kv_dtype=kv)
    if kv == "bf16":
        spec["regen"] = dict(seed=11, layer=1, fraction=0.5)
    w = synth.build(spec, device=gpu, seed=split + 3, name=f"mfma-window{split}-{kv}")
    out, lse = run(w, split_tokens=split)
    check(w, out, lse)


@pytest.mark.parametrize("P", [16, 64, 256])
def test_mfma_prefill_regen_page_sizes(gpu, P):
    w = synth.build(dict(num_seqs=2, context_lens=[2000, 900], query_lens=[257, 64],
                         num_heads=16, num_kv_heads=2, head_dim=128, page_tokens=P,
                         kv_dtype="bf16", regen=dict(seed=5, layer=2, fraction=0.75)),
                    device=gpu, seed=P, name=f"mfma-regen-P{P}")
    out, lse = run(w)
    check(w, out, lse)


def test_mfma_prefill_page_size_and_placement_do_not_change_bits(gpu):
    w = synth.build(dict(num_seqs=2, context_lens=[1111, 700], query_lens=[150, 700],
                         num_heads=16, num_kv_heads=4, head_dim=128, page_tokens=16,
                         kv_dtype="bf16"), device=gpu, seed=77, name="mfma-pagesize")
    o0, l0 = run(w)
    check(w, o0, l0)
    for P, seed in ((32, 1), (64, 2), (256, 3)):
        w2 = relayout(w, P, seed, spare_blocks=3)
        w2.query_lens = w.query_lens
        o2, l2 = run(w2)
        assert np.array_equal(o0.view(np.uint32), o2.view(np.uint32)), P
        assert np.array_equal(l0.view(np.uint32), l2.view(np.uint32)), P


def test_config5_regenerated_equals_resident_bitwise(gpu):
    # CFR-Atlas contract on the prefill path: 75 % regenerated vs all pages
    # resident (filled by the regenerator) give identical bits.
    kw = dict(context_lens=4096, query_lens=512, num_heads=16, num_kv_heads=2)
    w_regen = synth.config(5, device=gpu, **kw)
    w_res = synth.config(5, device=gpu, regen=dict(seed=42, layer=0, fraction=0.0), **kw)
    o1, l1 = run(w_regen)
    o2, l2 = run(w_res)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    check(w_regen, o1, l1, rows=[0, 100, 511])


def test_config5_full_sampled(gpu):
    w = synth.config(5, device=gpu)
    out, lse = run(w)
    check(w, out, lse, rows=[0, 1, 777, 1500, 2047], heads=[0, 13, 40, 63])


# ---------------------------------------------------------------------------
# Debug table validation
# ---------------------------------------------------------------------------

def test_validate_tables_counts_planted_faults(gpu):
    w = synth.config(3, device=gpu, num_seqs=4, context_lens=[1, 100, 1500, 2600])
    prob = atlas.Problem(w)
    # clean problem: the NaN poison sits only in unused entries and page tails
    assert prob.validate(check_values=True) == [0, 0, 0, 0]
    prob.table[2, 5] = w.num_blocks + 7        # visible entry naming no page
    prob.table[3, 2] = -1
    assert prob.validate() == [2, 0, 0, 0]
    prob.table.copy_(torch.from_numpy(w.page_table).to(gpu))
    blk = int(w.page_table[3, 4])
    w.k_pool[blk, 1, 3, 7] = float("nan")      # visible token 4 * 16 + 3 of seq 3
    w.v_pool[blk, 0, 0, 0] = float("inf")
    assert prob.validate(check_values=True) == [0, 0, 2, 0]
    assert prob.validate(check_values=False) == [0, 0, 0, 0]
    prob.ctx[1] = w.max_context_len + 1        # beyond the host bound
    assert prob.validate()[1] == 1


def test_validate_tables_tiered_and_regen(gpu):
    w = synth.config(4, device=gpu, num_seqs=3, context_lens=[1000, 2500, 3000])
    prob = atlas.Problem(w)
    assert prob.validate(check_values=True) == [0, 0, 0, 0]
    e = int(w.page_table[1, 3]) & 0xFFFFFFFF
    tier, slot = e >> 30, e & ((1 << 30) - 1)
    assert tier in (1, 2)
    scales = w.tiers["i8_k_scale" if tier == 1 else "i4_k_scale"]
    scales[slot, 2] = float("inf")
    assert prob.validate(check_values=True) == [0, 0, 0, 1]
    prob.table[0, 1] = -(1 << 30)              # 0xC0000000: FP8 slot 0, FP8 pool empty
    assert prob.validate()[0] == 1

    w5 = synth.config(5, device=gpu, context_lens=3000, query_lens=200, num_heads=16,
                      num_kv_heads=2)
    p5 = atlas.Problem(w5)
    assert p5.validate() == [0, 0, 0, 0]
    p5.regen_pages[0] = int(w5.regen["regen_pages"].max()) + 1
    assert p5.validate()[1] == 1


def test_read_probe_reads_every_word(gpu):
    n = (1 << 20) + 4 * 37  # words; not a multiple of the grid stride
    x = torch.randint(0, 2**31 - 1, (n,), dtype=torch.int32, device=gpu)
    out = torch.zeros(64, dtype=torch.int32, device=gpu)
    atlas.atlas_read_probe(x, out, 64)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(x.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want
