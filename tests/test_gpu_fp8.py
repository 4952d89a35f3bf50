"""GPU parity of the FP8 (E4M3) cold tier through the C ABI: decoded values
bit-exact, tiered attention over FP8 pages on both decode kernels, demotion
into FP8 bit-exact against the oracle's encoder, and the validator's FP8
checks."""

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from tests.test_gpu_parity import check, run

pytestmark = pytest.mark.gpu


def _fp8_case(gpu, hot="f16", H=32, Hkv=8, P=16, ctx=(700, 1900, 3100), seed=5, **kw):
    return synth.build(dict(num_seqs=len(ctx), context_lens=list(ctx), num_heads=H,
                            num_kv_heads=Hkv, head_dim=128, page_tokens=P, q_dtype="bf16",
                            kv_dtype=hot, placement="permuted",
                            tiers=dict(hot_tokens=300, p_int8=0.3, p_fp8=0.4), **kw),
                       device=gpu, seed=seed, name=f"fp8-{hot}-{H}/{Hkv}-P{P}")


def test_dequant_fp8_pages_bit_exact(gpu):
    w = _fp8_case(gpu)
    assert w.tiers["counts"][3] > 0
    prob = atlas.Problem(w)
    ent = np.concatenate([w.page_table[s, :w.pages_of(s)] for s in range(w.num_seqs)])
    f8 = ent[(ent.view(np.uint32) >> 30) == 3]
    entries = torch.from_numpy(f8).to(gpu)
    k = torch.empty((len(f8), 8, 16, 128), device=gpu)
    v = torch.empty_like(k)
    atlas.atlas_dequant_pages(prob.args, prob.tiers, entries, k, v)
    torch.cuda.synchronize()
    ta = oracle.HostView(w).tier_arrays()
    for i, e in enumerate(f8.view(np.uint32)):
        slot = int(e) & ((1 << 30) - 1)
        for got, kv in ((k[i], "k"), (v[i], "v")):
            vals = oracle.fp8_e4m3_value(ta[f"f8_{kv}"][slot])
            want = (vals * ta[f"f8_{kv}_scale"][slot][:, None, None].astype(np.float64))
            want = want.astype(np.float32)  # one rounding of the exact product
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), i


@pytest.mark.parametrize("kernel", ["default", "valu"])
@pytest.mark.parametrize("hot,H,Hkv,P", [("f16", 32, 8, 16), ("f16", 8, 4, 64),
                                         ("bf16", 16, 2, 16), ("f16", 8, 1, 256)])
def test_tiered_attention_with_fp8_pages(gpu, monkeypatch, kernel, hot, H, Hkv, P):
    if kernel == "valu":
        monkeypatch.setenv("ATLAS_DECODE_VALU", "1")
    w = _fp8_case(gpu, hot=hot, H=H, Hkv=Hkv, P=P, seed=H + P)
    assert w.tiers["counts"][3] > 0
    out, lse = run(w)
    check(w, out, lse)


def test_fp8_mix_full_size_sampled(gpu):
    # the 64-sequence tiered decode with a third of its cold pages in FP8
    w = synth.config(4, device=gpu, tiers=dict(hot_tokens=1024, p_int8=0.34, p_fp8=0.33))
    assert w.tiers["counts"][3] > 1000
    out, lse = run(w)
    check(w, out, lse, rows=[0, 9, 33, 63], heads=[0, 7, 20, 31])


@pytest.mark.parametrize("hot", ["f16", "bf16"])
def test_demote_to_fp8_bit_exact_and_attention(gpu, hot):
    w = synth.build(dict(num_seqs=2, context_lens=[900, 1700], num_heads=16, num_kv_heads=2,
                         head_dim=128, page_tokens=16, q_dtype="bf16", kv_dtype=hot,
                         tiers=dict(hot_tokens=1000, p_int8=0.5)), device=gpu, seed=31,
                    name=f"demote-fp8-{hot}")
    Hkv, P, D = 2, 16, 128
    s = 1
    ent = w.page_table[s].view(np.uint32)
    pages = [p for p in range(int(w.context_lens[s]) // P) if int(ent[p]) >> 30 == 0][:5]
    assert len(pages) == 5
    n = len(pages)
    for kv in ("k", "v"):
        w.tiers[f"f8_{kv}"] = torch.zeros((n, Hkv, P, D), dtype=torch.uint8, device=gpu)
        w.tiers[f"f8_{kv}_scale"] = torch.full((n, Hkv), -1.0, device=gpu)
    # make one block hit the saturation and subnormal corners: an element far
    # above the rest and one tiny element
    blk0 = int(ent[pages[0]]) & ((1 << 30) - 1)
    w.k_pool[blk0, 0, 0, 0] = 300.0
    w.k_pool[blk0, 0, 0, 1] = 1e-4
    prob = atlas.Problem(w)
    src = torch.tensor([int(ent[p]) & ((1 << 30) - 1) for p in pages], dtype=torch.int32,
                       device=gpu)
    dst_np = np.array([(3 << 30) | i for i in range(n)], dtype=np.uint32)
    dst = torch.from_numpy(dst_np.view(np.int32)).to(gpu)
    rejected = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_demote_pages(prob.args, prob.tiers, src, dst, rejected)
    torch.cuda.synchronize()
    assert int(rejected) == 0
    host = oracle.HostView(w)
    (ka, kind), (va, _) = host.pools()
    for i, b in enumerate(src.cpu().numpy()):
        for arr, kv in ((ka, "k"), (va, "v")):
            for g in range(Hkv):
                x = oracle.widen_bits(arr[b, g], kind).astype(np.float32)
                codes, scale = oracle.quantize_block_fp8(x)
                got_s = w.tiers[f"f8_{kv}_scale"][i, g].cpu().numpy()
                assert got_s.tobytes() == scale.tobytes(), (i, kv, g)
                got = w.tiers[f"f8_{kv}"][i, g].cpu().numpy()
                assert np.array_equal(got, codes), (i, kv, g, int((got != codes).sum()))
    # repoint the pages at their FP8 copies and attend
    new = ent.copy()
    for i, p in enumerate(pages):
        new[p] = dst_np[i]
    w.page_table[s] = new.view(np.int32)
    prob = atlas.Problem(w)
    out, lse = prob.run()
    torch.cuda.synchronize()
    check(w, out.cpu().numpy(), lse.cpu().numpy())


def test_validate_counts_fp8_nan_codes_and_bad_slots(gpu):
    w = _fp8_case(gpu, ctx=(1000, 2500))
    prob = atlas.Problem(w)
    assert prob.validate(check_values=True) == [0, 0, 0, 0]
    ent = w.page_table.view(np.uint32)
    s, p = next((s, p) for s in range(2) for p in range(w.pages_of(s)) if ent[s, p] >> 30 == 3)
    slot = int(ent[s, p]) & ((1 << 30) - 1)
    w.tiers["f8_v"][slot, 1, 0, 5] = 0x7F   # NaN code on a visible row
    assert prob.validate(check_values=True) == [0, 0, 1, 0]
    prob.table[s, p] = int(np.uint32((3 << 30) | w.tiers["f8_k"].shape[0]).view(np.int32))
    assert prob.validate()[0] == 1
