"""GPU parity of the INT2 cold tier (the extension tier, kind 1) through the C
ABI: decoded values bit-exact, tiered attention over pages of every class on
both decode kernels, demotion into INT2 (from hot and from int4 slots)
bit-exact against the oracle's encoder, and the validator's class checks."""

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from tests.test_gpu_parity import check, run

pytestmark = pytest.mark.gpu

I2 = (3 << 30) | (1 << 28)


def _case(gpu, hot="f16", H=32, Hkv=8, P=16, ctx=(700, 1900, 3100), seed=5):
    return synth.build(dict(num_seqs=len(ctx), context_lens=list(ctx), num_heads=H,
                            num_kv_heads=Hkv, head_dim=128, page_tokens=P, q_dtype="bf16",
                            kv_dtype=hot, placement="permuted",
                            tiers=dict(hot_tokens=300, p_int8=0.2, p_fp8=0.2, p_int2=0.3)),
                       device=gpu, seed=seed, name=f"int2-{hot}-{H}/{Hkv}-P{P}")


def test_dequant_int2_pages_bit_exact(gpu):
    w = _case(gpu)
    assert w.tiers["counts"][4] > 0
    prob = atlas.Problem(w)
    ent = np.concatenate([w.page_table[s, :w.pages_of(s)] for s in range(w.num_seqs)])
    sel = np.array([oracle.entry_class(e)[0] == 4 for e in ent])
    entries = torch.from_numpy(ent[sel]).to(gpu)
    k = torch.empty((int(sel.sum()), 8, 16, 128), device=gpu)
    v = torch.empty_like(k)
    atlas.atlas_dequant_pages(prob.args, prob.tiers, entries, k, v)
    torch.cuda.synchronize()
    host = oracle.HostView(w)
    for i, e in enumerate(ent[sel]):
        for got, kv in ((k[i], "k"), (v[i], "v")):
            want = np.stack([oracle.block_f32(w, e, g, kv, host=host) for g in range(8)])
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), i


@pytest.mark.parametrize("kernel", ["default", "valu"])
@pytest.mark.parametrize("hot,H,Hkv,P", [("f16", 32, 8, 16), ("f16", 8, 4, 64),
                                         ("bf16", 16, 2, 16), ("f16", 16, 2, 256)])
def test_tiered_attention_with_int2_pages(gpu, monkeypatch, kernel, hot, H, Hkv, P):
    if kernel == "valu":
        monkeypatch.setenv("ATLAS_DECODE_VALU", "1")
    w = _case(gpu, hot=hot, H=H, Hkv=Hkv, P=P, seed=H + P)
    assert w.tiers["counts"][4] > 0
    out, lse = run(w)
    check(w, out, lse)


def test_all_classes_full_size_sampled(gpu):
    w = synth.config(4, device=gpu, tiers=dict(hot_tokens=1024, p_int8=0.25, p_fp8=0.25,
                                               p_int2=0.25))
    assert w.tiers["counts"][4] > 1000
    out, lse = run(w)
    check(w, out, lse, rows=[0, 9, 33, 63], heads=[0, 7, 20, 31])


@pytest.mark.parametrize("hot", ["f16", "bf16"])
def test_demote_to_int2_and_transcode_from_int4(gpu, hot):
    w = synth.build(dict(num_seqs=2, context_lens=[900, 1700], num_heads=16, num_kv_heads=2,
                         head_dim=128, page_tokens=16, q_dtype="bf16", kv_dtype=hot,
                         tiers=dict(hot_tokens=1000, p_int8=0.5)), device=gpu, seed=41,
                    name=f"demote-int2-{hot}")
    Hkv, P, D = 2, 16, 128
    ent = w.page_table[1].view(np.uint32)
    full = int(w.context_lens[1]) // P
    hot_pages = [p for p in range(full) if int(ent[p]) >> 30 == 0][:3]
    i4_pages = [p for p in range(full) if int(ent[p]) >> 30 == 2][:3]
    assert len(hot_pages) == 3 and len(i4_pages) == 3
    n = 6
    for kv in ("k", "v"):
        w.tiers[f"i2_{kv}"] = torch.zeros((n, Hkv, P, D // 4), dtype=torch.uint8, device=gpu)
        w.tiers[f"i2_{kv}_scale"] = torch.full((n, Hkv), -1.0, device=gpu)
    pages = hot_pages + i4_pages
    src_np = np.array([int(ent[p]) for p in pages], dtype=np.uint32)
    dst_np = np.array([I2 | i for i in range(n)], dtype=np.uint32)
    prob = atlas.Problem(w)
    host = oracle.HostView(w)
    want = {}
    for i, e in enumerate(src_np):
        for kv in ("k", "v"):
            for g in range(Hkv):
                want[(i, kv, g)] = oracle.quantize_block(
                    oracle.block_f32(w, e, g, kv, host=host), 1)
    rej = torch.zeros(1, dtype=torch.int32, device=gpu)
    atlas.atlas_demote_pages(prob.args, prob.tiers, torch.from_numpy(src_np.view(np.int32)).to(gpu),
                             torch.from_numpy(dst_np.view(np.int32)).to(gpu), rej)
    torch.cuda.synchronize()
    assert int(rej) == 0
    for (i, kv, g), (codes, scale) in want.items():
        got_s = w.tiers[f"i2_{kv}_scale"][i, g].cpu().numpy()
        assert got_s.tobytes() == scale.tobytes(), (i, kv, g)
        got = w.tiers[f"i2_{kv}"][i, g].cpu().numpy()
        assert np.array_equal(got, oracle.pack_int2(codes)), (i, kv, g)
    new = ent.copy()
    for i, p in enumerate(pages):
        new[p] = dst_np[i]
    w.page_table[1] = new.view(np.int32)
    out, lse = run(w)
    check(w, out, lse)


def test_validate_counts_unknown_kinds_and_bad_int2_slots(gpu):
    w = _case(gpu, ctx=(1000, 2500))
    prob = atlas.Problem(w)
    assert prob.validate(check_values=True) == [0, 0, 0, 0]
    ent = w.page_table.view(np.uint32)
    s, p = next((s, p) for s in range(2) for p in range(w.pages_of(s))
                if oracle.entry_class(ent[s, p])[0] == 4)
    slot = oracle.entry_class(ent[s, p])[1]
    w.tiers["i2_k_scale"][slot, 3] = float("nan")
    assert prob.validate(check_values=True) == [0, 0, 0, 1]
    prob.table[s, p] = int(np.uint32(I2 | w.tiers["i2_k"].shape[0]).view(np.int32))
    prob.table[1 - s, 0] = int(np.uint32((3 << 30) | (3 << 28)).view(np.int32))  # kind 3
    assert prob.validate()[0] == 2
    out, lse = prob.run()
    torch.cuda.synchronize()
    assert torch.isnan(out[s]).all() and torch.isnan(out[1 - s]).all()
