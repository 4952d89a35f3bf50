"""GPU parity of the positional policy (ALiBi and the rotary embedding)
through the C ABI against the f64 oracle, on every attention path: the
vector-ALU and matrix-core decode, tiered and regenerated decode, and the
matrix-core and vector-ALU chunked prefill; plus the rotation of new keys in
the write path.  Tolerances as for the plain paths (2e-5 f32, 2e-3 16-bit,
dequantised or regenerated K/V)."""

import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from tests.test_gpu_parity import check, run

pytestmark = pytest.mark.gpu

POLICIES = {"alibi": dict(alibi=True), "rope": dict(rope_theta=10000.0),
            "both": dict(alibi=True, rope_theta=500000.0)}


@pytest.mark.parametrize("policy", list(POLICIES))
@pytest.mark.parametrize("kv,D,H,Hkv", [("f32", 64, 4, 4), ("f32", 128, 8, 1),
                                        ("bf16", 128, 8, 4), ("bf16", 128, 16, 4),
                                        ("bf16", 128, 16, 2), ("f16", 128, 8, 2),
                                        ("bf16", 64, 8, 2)])
def test_decode(gpu, policy, kv, D, H, Hkv):
    w = synth.build(dict(num_seqs=3, context_lens=[70, 1100, 2500], num_heads=H,
                         num_kv_heads=Hkv, head_dim=D, page_tokens=16, kv_dtype=kv,
                         placement="permuted", positional=POLICIES[policy]),
                    device=gpu, seed=D + H + Hkv, name=f"decode-{policy}-{kv}-D{D}-{H}/{Hkv}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("policy", list(POLICIES))
@pytest.mark.parametrize("kernel", ["default", "valu"])
@pytest.mark.parametrize("H,Hkv,hot", [(8, 2, "f16"), (16, 2, "bf16")])
def test_tiered_decode(gpu, monkeypatch, policy, kernel, H, Hkv, hot):
    if kernel == "valu":
        monkeypatch.setenv("ATLAS_DECODE_VALU", "1")
    w = synth.build(dict(num_seqs=3, context_lens=[40, 900, 2600], num_heads=H,
                         num_kv_heads=Hkv, head_dim=128, page_tokens=16, q_dtype="bf16",
                         kv_dtype=hot, tiers=dict(hot_tokens=300, p_int8=0.5),
                         positional=POLICIES[policy]),
                    device=gpu, seed=H + Hkv, name=f"tiered-{policy}-{kernel}-{H}/{Hkv}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("policy", list(POLICIES))
def test_regen_decode(gpu, policy):
    w = synth.build(dict(num_seqs=3, context_lens=[900, 17, 2050], num_heads=8,
                         num_kv_heads=2, head_dim=128, page_tokens=64, kv_dtype="bf16",
                         regen=dict(seed=7, layer=3, fraction=0.75),
                         positional=POLICIES[policy]),
                    device=gpu, seed=3, name=f"regen-decode-{policy}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("policy", list(POLICIES))
@pytest.mark.parametrize("kv,H,Hkv", [("bf16", 8, 8), ("bf16", 16, 2), ("f16", 8, 2),
                                      ("bf16", 8, 4)])
def test_mfma_prefill(gpu, policy, kv, H, Hkv):
    w = synth.build(dict(num_seqs=3, context_lens=[300, 77, 1500], query_lens=[300, 20, 133],
                         num_heads=H, num_kv_heads=Hkv, head_dim=128, page_tokens=16,
                         kv_dtype=kv, positional=POLICIES[policy]),
                    device=gpu, seed=H * 10 + Hkv, name=f"mfma-{policy}-{kv}-{H}/{Hkv}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("policy", list(POLICIES))
@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_valu_prefill(gpu, policy, kv):
    w = synth.build(dict(num_seqs=3, context_lens=[50, 700, 333], query_lens=[50, 37, 5],
                         num_heads=8, num_kv_heads=2, head_dim=64, page_tokens=16,
                         kv_dtype=kv, positional=POLICIES[policy]),
                    device=gpu, seed=9, name=f"valu-prefill-{policy}-{kv}")
    out, lse = run(w)
    check(w, out, lse)


@pytest.mark.parametrize("policy", list(POLICIES))
@pytest.mark.parametrize("P", [16, 256])
def test_mfma_prefill_regen(gpu, policy, P):
    w = synth.build(dict(num_seqs=2, context_lens=[2000, 900], query_lens=[257, 64],
                         num_heads=16, num_kv_heads=2, head_dim=128, page_tokens=P,
                         kv_dtype="bf16", regen=dict(seed=5, layer=2, fraction=0.75),
                         positional=POLICIES[policy]),
                    device=gpu, seed=P, name=f"mfma-regen-{policy}-P{P}")
    out, lse = run(w)
    check(w, out, lse)


def test_full_size_shapes_sampled(gpu):
    # the benchmarked decode and prefill shapes with both policies on,
    # checked on sampled rows and heads
    for n, rows, heads in ((3, [0, 17, 63], [0, 5, 31]), (5, [0, 1000, 2047], [0, 33, 63])):
        w = synth.config(n, device=gpu, positional=POLICIES["both"])
        out, lse = run(w)
        check(w, out, lse, rows=rows, heads=heads)


@pytest.mark.parametrize("kv", ["f32", "bf16", "f16"])
def test_write_kv_stores_rotated_keys(gpu, kv):
    theta = 10000.0
    spec = dict(num_seqs=3, context_lens=[40, 300, 70001], query_lens=[1, 16, 5],
                num_heads=8, num_kv_heads=2, head_dim=128, page_tokens=16, kv_dtype=kv,
                positional=dict(rope_theta=theta))
    w = synth.build(spec, device=gpu, seed=21, name=f"write-rope-{kv}")
    gen = torch.Generator(device=gpu).manual_seed(8)
    shape = (w.total_q, w.num_kv_heads, w.head_dim)
    k_new = torch.randn(shape, generator=gen, device=gpu).to(w.k_pool.dtype)
    v_new = torch.randn(shape, generator=gen, device=gpu).to(w.v_pool.dtype)
    # the oracle's cache: the generated pool with the oracle's own rotation of
    # each new K row (rounded to the pool's type) and the new V rows placed in
    # it; the attention reference is computed over it, not over the pool the
    # device wrote
    ref_k, ref_v = w.k_pool.clone(), w.v_pool.clone()
    prob = atlas.Problem(w)
    atlas.atlas_write_kv(prob.args, k_new, v_new)
    torch.cuda.synchronize()
    kn = k_new.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    r = 0
    for s in range(w.num_seqs):
        n_q, c = int(w.query_lens[s]), int(w.context_lens[s])
        for t in range(n_q):
            pos = c - n_q + t
            blk, off = int(w.page_table[s, pos // 16]), pos % 16
            got = w.k_pool[blk, :, off].float().cpu().numpy().astype(np.float64)
            want = oracle.rope(kn[r], pos, theta)
            # f32: the rotation itself (hardware sine/cosine, about 1e-6);
            # 16-bit: one rounding of the rotated value
            ulp = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}[kv]
            bound = 4e-6 * (1 + np.abs(want)) + ulp * np.abs(want)
            err = np.abs(got - want)
            assert np.all(err <= bound), (s, t, float(err.max()))
            worst = max(worst, float((err / (1 + np.abs(want))).max()))
            assert torch.equal(w.v_pool[blk, :, off], v_new[r])
            bits = oracle.hot_bits(want, kv)
            bits = bits.view(np.int32) if kv == "f32" else bits.view(np.int16)
            ref_k[blk, :, off] = torch.from_numpy(bits).to(gpu).view(ref_k.dtype)
            ref_v[blk, :, off] = v_new[r]
            r += 1
    print(f"[write-rope-{kv}] worst relative error {worst:.3e}")
    out, lse = run(w)
    ref = copy.copy(w)
    ref.k_pool, ref.v_pool = ref_k, ref_v
    check(ref, out, lse)


@pytest.mark.parametrize("prefill", [False, True])
def test_regenerated_equals_resident_bitwise(gpu, prefill):
    # CFR-Atlas contract under RoPE: resident pages written by the library's
    # regenerator (rotated keys in bf16) and pages regenerated inside the
    # call give identical bits
    base = dict(num_seqs=2, context_lens=[1000, 2100], num_heads=8, num_kv_heads=2,
                head_dim=128, page_tokens=64, kv_dtype="bf16",
                positional=dict(alibi=True, rope_theta=10000.0))
    if prefill:
        base["query_lens"] = [130, 77]
    w_regen = synth.build(dict(base, regen=dict(seed=11, layer=1, fraction=0.75)),
                          device=gpu, seed=4, name=f"rope-regen-{prefill}")
    w_res = synth.build(dict(base, regen=dict(seed=11, layer=1, fraction=0.0)),
                        device=gpu, seed=4)
    o1, l1 = run(w_regen, split_tokens=512)
    o2, l2 = run(w_res, split_tokens=512)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    check(w_regen, o1, l1)
