"""End-to-end decode loops driven by the host residency runtime on the GPU:
the runtime's tables feed atlas_write_kv and the attention calls, its jobs
run through atlas_demote_pages / atlas_promote_pages /
atlas_regenerate_pages, and the attention results are checked against the
oracle.  The oracle never reads a device-written pool: tiered loops keep
host shadow pools that the oracle writes (the same rows, encodings and
reconstructions the runtime asks of the device), and the regenerated loop
is checked on the call whose every page is regenerated."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_runtime_amd import atlas
from kv_cache_runtime_amd.residency import REGEN, TIERED, Residency
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu

H, HKV, D, P = 8, 2, 128, 16


def _args(dev, q, k_pool, v_pool, table, ctx, out, lse, qstart=None, max_q=1, ws=None,
          kv=atlas.F16, qdt=atlas.BF16):
    a = atlas.make_args(q=q, k_pool=k_pool, v_pool=v_pool, page_table=table, context_lens=ctx,
                        num_heads=H, num_kv_heads=HKV, head_dim=D, page_tokens=P,
                        max_context_len=int(ctx.max()), scale=float(np.float32(D ** -0.5)),
                        out=out, lse=lse, query_start=qstart, max_query_len=max_q,
                        total_q=q.shape[0], kv_dtype=kv, q_dtype=qdt)
    return a


_NP = {torch.int8: np.int8, torch.uint8: np.uint8, torch.float32: np.float32,
       torch.int32: np.int32}


class _Shadow:
    """Host copies of the f16 hot pool and the cold pools, written by the
    oracle alone: new rows go where the runtime's table puts them, each
    demotion is the oracle's encoding of its reading of the source block
    (sources are all read before any destination is written, as the device
    does within one call), and each reconstruction is the oracle's reading
    of the entry rounded to f16."""

    def __init__(self, n_hot, tiers, n_out=0):
        self.k = np.zeros((n_hot, HKV, P, D), np.float16)
        self.v = np.zeros_like(self.k)
        self.t = {key: np.zeros(tuple(a.shape), _NP[a.dtype]) for key, a in tiers.items()}
        self.n_out = n_out

    def paged(self, q, table, ctx, counts, name=""):
        tiers = {key: torch.from_numpy(a) for key, a in self.t.items()}
        return synth.Paged(num_seqs=3, num_heads=H, num_kv_heads=HKV, head_dim=D,
                           page_tokens=P, q_dtype="bf16", kv_dtype="f16", context_lens=ctx,
                           query_lens=np.ones(3, np.int32), scale=float(np.float32(D ** -0.5)),
                           q=q, k_pool=torch.from_numpy(self.k), v_pool=torch.from_numpy(self.v),
                           page_table=table, tiers=dict(tiers, counts=counts), name=name)

    def write(self, table, ctx, n_new, k_new, v_new):
        """Rows of the last n_new[i] tokens of sequence i, in row order."""
        k, v = k_new.cpu().numpy(), v_new.cpu().numpy()
        j = 0
        for i, n in enumerate(n_new):
            for t in range(n):
                pos = int(ctx[i]) - n + t
                b = int(np.uint32(table[i, pos // P]))
                assert b < self.k.shape[0], (i, pos, b)  # a hot page
                self.k[b, :, pos % P] = k[j]
                self.v[b, :, pos % P] = v[j]
                j += 1

    def _reader(self):
        w = self.paged(None, np.zeros((3, 1), np.int32), np.ones(3, np.int32), None)
        return w, oracle.HostView(w)

    def demote(self, src, dst):
        w, host = self._reader()
        new = []
        for se, de in zip(np.asarray(src).view(np.uint32), np.asarray(dst).view(np.uint32)):
            cls, slot = oracle.entry_class(int(de))
            for kv in ("k", "v"):
                for g in range(HKV):
                    x = oracle.block_f32(w, int(se), g, kv, host=host)
                    if cls == 5:
                        enc = oracle.encode_1bit(x.ravel(), self.n_out)
                    elif cls == 3:
                        enc = oracle.quantize_block_fp8(x)
                    else:
                        codes, sc = oracle.quantize_block(x, {1: 127, 2: 7, 4: 1}[cls])
                        codes = (codes.astype(np.int8) if cls == 1 else
                                 oracle.pack_int4(codes) if cls == 2 else oracle.pack_int2(codes))
                        enc = (codes, sc)
                    new.append((cls, slot, kv, g, enc))
        for cls, slot, kv, g, enc in new:
            if cls == 5:
                signs, sc, outs = enc
                self.t[f"b1_{kv}"][slot, g] = signs
                self.t[f"b1_{kv}_scale"][slot, g] = sc
                self.t[f"b1_{kv}_out"][slot, g] = np.asarray(outs, np.uint32).view(np.int32)
            else:
                key = {1: "i8", 2: "i4", 3: "f8", 4: "i2"}[cls]
                self.t[f"{key}_{kv}"][slot, g] = enc[0]
                self.t[f"{key}_{kv}_scale"][slot, g] = enc[1]

    def promote(self, src, dst):
        w, host = self._reader()
        new = [(int(b), kv, g, oracle.hot_bits(oracle.block_f32(w, int(e), g, kv, host=host), "f16"))
               for e, b in zip(np.asarray(src).view(np.uint32), dst)
               for kv in ("k", "v") for g in range(HKV)]
        for b, kv, g, bits in new:
            (self.k if kv == "k" else self.v)[b, g] = bits.reshape(P, D).view(np.float16)


def _attend(a, dev, tiers=None, regen=None):
    n = atlas.atlas_workspace_size(a, regen)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    a.workspace = atlas._ptr(ws)
    a.workspace_bytes = n
    a.tensors.append(ws)
    if tiers is not None:
        atlas.atlas_paged_attention_tiered(a, tiers)
    elif regen is not None:
        atlas.atlas_paged_attention_regen(a, regen)
    torch.cuda.synchronize()


def test_tiered_decode_loop_through_the_runtime(gpu):
    rt = Residency(mode=TIERED, page_tokens=P, max_seqs=3, max_pages_per_seq=64, hot_blocks=64,
                   recent_tokens=64, sink_tokens=16, fp8_pages=2, int8_pages=3, num_fp8=16,
                   num_int8=24, num_int4=40, int4_pages=3, num_int2=160)
    gen = torch.Generator(device=gpu).manual_seed(1)
    hot_k = torch.zeros((64, HKV, P, D), dtype=torch.float16, device=gpu)
    hot_v = torch.zeros_like(hot_k)
    tiers = {}
    for key, n, shape_d, dt in (("f8", 16, D, torch.uint8), ("i8", 24, D, torch.int8),
                                ("i4", 40, D // 2, torch.uint8), ("i2", 160, D // 4, torch.uint8)):
        for kv in ("k", "v"):
            tiers[f"{key}_{kv}"] = torch.zeros((n, HKV, P, shape_d), dtype=dt, device=gpu)
            tiers[f"{key}_{kv}_scale"] = torch.zeros((n, HKV), device=gpu)
    pools = atlas.make_tiers(tiers)
    shadow = _Shadow(64, tiers)
    seqs = [0, 1, 2]
    prompt = [100, 37, 250]
    for s in seqs:
        rt.add_seq(s)

    def write(n_new, qstart, max_q):
        table, ctx, _ = rt.tables(seqs)
        rows = int(sum(n_new))
        k_new = torch.randn((rows, HKV, D), generator=gen, device=gpu).half()
        v_new = torch.randn((rows, HKV, D), generator=gen, device=gpu).half()
        q = torch.zeros((rows, H, D), dtype=torch.bfloat16, device=gpu)
        out = torch.empty((rows, H, D), device=gpu)
        lse = torch.empty((rows, H), device=gpu)
        tt, ct = torch.from_numpy(table).to(gpu), torch.from_numpy(ctx).to(gpu)
        qs = None if qstart is None else torch.from_numpy(qstart).to(gpu)
        a = _args(gpu, q, hot_k, hot_v, tt, ct, out, lse, qstart=qs, max_q=max_q)
        a.num_blocks = 64
        atlas.atlas_write_kv(a, k_new, v_new)
        shadow.write(table, ctx, n_new, k_new, v_new)

    def run_jobs():
        src, dst, _, _ = rt.plan()
        if len(src):
            a = _args(gpu, torch.zeros((3, H, D), dtype=torch.bfloat16, device=gpu), hot_k, hot_v,
                      torch.zeros((3, 64), dtype=torch.int32, device=gpu),
                      torch.ones(3, dtype=torch.int32, device=gpu),
                      torch.empty((3, H, D), device=gpu), torch.empty((3, H), device=gpu))
            a.num_blocks = 64
            rej = torch.zeros(1, dtype=torch.int32, device=gpu)
            atlas.atlas_demote_pages(a, pools, torch.from_numpy(src).to(gpu),
                                     torch.from_numpy(dst).to(gpu), rej)
            torch.cuda.synchronize()
            assert int(rej) == 0
            shadow.demote(src, dst)
        return len(src)

    for s, n in zip(seqs, prompt):
        rt.append(s, n)
    qstart = np.concatenate([[0], np.cumsum(prompt)]).astype(np.int32)
    write(prompt, qstart, max(prompt))
    run_jobs()
    checked = 0
    for step in range(48):
        for s in seqs:
            rt.append(s, 1)
        write([1, 1, 1], None, 1)
        if step % 12 == 11:
            table, ctx, _ = rt.tables(seqs)
            q = torch.randn((3, H, D), generator=gen, device=gpu).bfloat16()
            out = torch.empty((3, H, D), device=gpu)
            lse = torch.empty((3, H), device=gpu)
            a = _args(gpu, q, hot_k, hot_v, torch.from_numpy(table).to(gpu),
                      torch.from_numpy(ctx).to(gpu), out, lse)
            a.num_blocks = 64
            _attend(a, gpu, tiers=pools)
            counts = [64, tiers["i8_k"].shape[0], tiers["i4_k"].shape[0],
                      tiers["f8_k"].shape[0], tiers["i2_k"].shape[0]]
            w = shadow.paged(q, table, ctx, counts, name=f"runtime-tiered-{step}")
            check(w, out.cpu().numpy(), lse.cpu().numpy())
            checked += 1
        run_jobs()
    st = rt.stats()
    assert checked == 4 and st["demotions"] > 0 and st["transcodes"] > 0
    assert st["fp8_used"] > 0 and st["int8_used"] > 0 and st["int4_used"] > 0
    assert st["int2_used"] > 0


def test_tiered_decode_loop_with_the_1bit_archive(gpu):
    """The full ARGUS loop through the runtime: plans archive the oldest cold
    pages into 1-bit slots, and before each checked attention call the
    transient tables rebuild them into reserved hot blocks
    (atlas_promote_pages); the result matches the oracle over the pools."""
    HOT, TRANS, K_OUT = 48, 40, 16
    rt = Residency(mode=TIERED, page_tokens=P, max_seqs=3, max_pages_per_seq=64, hot_blocks=HOT,
                   recent_tokens=48, sink_tokens=16, fp8_pages=1, int8_pages=2, num_fp8=8,
                   num_int8=16, num_int4=24, int4_pages=2, num_int2=24, int2_pages=2,
                   num_1bit=96, transient_blocks=TRANS)
    gen = torch.Generator(device=gpu).manual_seed(3)
    hot_k = torch.zeros((HOT + TRANS, HKV, P, D), dtype=torch.float16, device=gpu)
    hot_v = torch.zeros_like(hot_k)
    tiers = {}
    for key, n, shape_d, dt in (("f8", 8, D, torch.uint8), ("i8", 16, D, torch.int8),
                                ("i4", 24, D // 2, torch.uint8), ("i2", 24, D // 4, torch.uint8)):
        for kv in ("k", "v"):
            tiers[f"{key}_{kv}"] = torch.zeros((n, HKV, P, shape_d), dtype=dt, device=gpu)
            tiers[f"{key}_{kv}_scale"] = torch.zeros((n, HKV), device=gpu)
    for kv in ("k", "v"):
        tiers[f"b1_{kv}"] = torch.zeros((96, HKV, P * D // 8), dtype=torch.uint8, device=gpu)
        tiers[f"b1_{kv}_scale"] = torch.zeros((96, HKV), device=gpu)
        tiers[f"b1_{kv}_out"] = torch.zeros((96, HKV, K_OUT), dtype=torch.int32, device=gpu)
    pools = atlas.make_tiers(tiers)
    shadow = _Shadow(HOT + TRANS, tiers, n_out=K_OUT)
    seqs = [0, 1, 2]
    prompt = [120, 45, 260]
    for s in seqs:
        rt.add_seq(s)

    def dummy_args():
        a = _args(gpu, torch.zeros((3, H, D), dtype=torch.bfloat16, device=gpu), hot_k, hot_v,
                  torch.zeros((3, 64), dtype=torch.int32, device=gpu),
                  torch.ones(3, dtype=torch.int32, device=gpu),
                  torch.empty((3, H, D), device=gpu), torch.empty((3, H), device=gpu))
        a.num_blocks = HOT + TRANS
        return a

    def tables():
        table, ctx, _, psrc, pdst = rt.tables_transient(seqs)
        if len(psrc):
            rej = torch.zeros(1, dtype=torch.int32, device=gpu)
            atlas.atlas_promote_pages(dummy_args(), pools, torch.from_numpy(psrc).to(gpu),
                                      torch.from_numpy(pdst).to(gpu), rej)
            torch.cuda.synchronize()
            assert int(rej) == 0
            shadow.promote(psrc, pdst)
        return table, ctx, len(psrc)

    def write(n_new, qstart, max_q):
        table, ctx, _ = rt.tables(seqs)
        rows = int(sum(n_new))
        k_new = torch.randn((rows, HKV, D), generator=gen, device=gpu).half()
        v_new = torch.randn((rows, HKV, D), generator=gen, device=gpu).half()
        q = torch.zeros((rows, H, D), dtype=torch.bfloat16, device=gpu)
        tt, ct = torch.from_numpy(table).to(gpu), torch.from_numpy(ctx).to(gpu)
        qs = None if qstart is None else torch.from_numpy(qstart).to(gpu)
        a = _args(gpu, q, hot_k, hot_v, tt, ct, torch.empty((rows, H, D), device=gpu),
                  torch.empty((rows, H), device=gpu), qstart=qs, max_q=max_q)
        a.num_blocks = HOT + TRANS
        atlas.atlas_write_kv(a, k_new, v_new)
        shadow.write(table, ctx, n_new, k_new, v_new)

    def run_jobs():
        src, dst, _, _ = rt.plan()
        if len(src):
            rej = torch.zeros(1, dtype=torch.int32, device=gpu)
            atlas.atlas_demote_pages(dummy_args(), pools, torch.from_numpy(src).to(gpu),
                                     torch.from_numpy(dst).to(gpu), rej)
            torch.cuda.synchronize()
            assert int(rej) == 0
            shadow.demote(src, dst)

    for s, n in zip(seqs, prompt):
        rt.append(s, n)
    qstart = np.concatenate([[0], np.cumsum(prompt)]).astype(np.int32)
    write(prompt, qstart, max(prompt))
    run_jobs()
    checked, rebuilt = 0, 0
    for step in range(40):
        for s in seqs:
            rt.append(s, 1)
        write([1, 1, 1], None, 1)
        if step % 10 == 9:
            table, ctx, n_promoted = tables()
            rebuilt += n_promoted
            q = torch.randn((3, H, D), generator=gen, device=gpu).bfloat16()
            out = torch.empty((3, H, D), device=gpu)
            lse = torch.empty((3, H), device=gpu)
            a = _args(gpu, q, hot_k, hot_v, torch.from_numpy(table).to(gpu),
                      torch.from_numpy(ctx).to(gpu), out, lse)
            a.num_blocks = HOT + TRANS
            print(f"[archive loop] step {step}: {n_promoted} pages rebuilt", flush=True)
            _attend(a, gpu, tiers=pools)
            counts = [HOT + TRANS, 16, 24, 8, 24]
            w = shadow.paged(q, table, ctx, counts, name=f"runtime-archive-{step}")
            check(w, out.cpu().numpy(), lse.cpu().numpy())
            checked += 1
        run_jobs()
    st = rt.stats()
    assert checked == 4 and rebuilt > 0 and st["archive_used"] > 0
    assert st["reconstructions"] == rebuilt and st["int2_used"] > 0


def test_regen_decode_loop_through_the_runtime(gpu):
    """KeepRecent + LRU hot cache + admission over regenerated pages: the
    result equals the all-regenerated call bit for bit (CFR-Atlas core
    contract) and the oracle within tolerance."""
    seed, layer = 77, 2
    rt = Residency(mode=REGEN, page_tokens=P, max_seqs=3, max_pages_per_seq=64, hot_blocks=20,
                   recent_tokens=48, admit_per_plan=2)
    hot_k = torch.zeros((20, HKV, P, D), dtype=torch.bfloat16, device=gpu)
    hot_v = torch.zeros_like(hot_k)
    seqs = [0, 1, 2]
    prompt = [150, 40, 300]
    gen = torch.Generator(device=gpu).manual_seed(2)
    known = {s: set() for s in seqs}  # resident pages already regenerated into their block

    def fill_new_pages():
        # resident pages hold the generator's values: regenerate every page
        # that got a block and has not been written yet
        table, ctx, regen = rt.tables(seqs)
        pages, blocks = [], []
        for i, s in enumerate(seqs):
            n = -(-int(ctx[i]) // P)
            for p in range(int(regen[i]), n):
                b = int(table[i, p])
                if (p, b) not in known[s]:
                    pages.append(p)
                    blocks.append(b)
                    known[s].add((p, b))
        if pages:
            atlas.atlas_regenerate_pages(seed, layer, HKV, D, P, atlas.BF16,
                                         torch.tensor(pages, dtype=torch.int32, device=gpu),
                                         torch.tensor(blocks, dtype=torch.int32, device=gpu),
                                         20, hot_k, hot_v)

    def forget_stale():
        table, ctx, regen = rt.tables(seqs)
        for i, s in enumerate(seqs):
            n = -(-int(ctx[i]) // P)
            live = {(p, int(table[i, p])) for p in range(int(regen[i]), n)}
            known[s] &= live

    for s, n in zip(seqs, prompt):
        rt.add_seq(s)
        rt.append(s, n)
    fill_new_pages()
    planted = [0]
    for step in range(40):
        for s in seqs:
            rt.append(s, 1)
        forget_stale()
        fill_new_pages()
        if step % 10 == 9:
            table, ctx, regen = rt.tables(seqs)
            q = torch.randn((3, H, D), generator=gen, device=gpu).bfloat16()
            outs = []
            for rp in (regen, -(-ctx // P)):  # as planned, then everything regenerated
                out = torch.empty((3, H, D), device=gpu)
                lse = torch.empty((3, H), device=gpu)
                a = _args(gpu, q, hot_k, hot_v, torch.from_numpy(table).to(gpu),
                          torch.from_numpy(ctx).to(gpu), out, lse, kv=atlas.BF16)
                a.num_blocks = 20
                a.split_tokens = 256
                rpt = torch.from_numpy(np.ascontiguousarray(rp, dtype=np.int32)).to(gpu)
                spec = atlas.make_regen(seed, layer, rpt, int(rpt.max()))
                _attend(a, gpu, regen=spec)
                outs.append((out.cpu().numpy(), lse.cpu().numpy()))
            # the oracle reads no pool here: every page of the reference
            # problem is regenerated (its pool is a host placeholder)
            all_regen = (-(-ctx // P)).astype(np.int32)
            zeros = torch.zeros((1, HKV, P, D), dtype=torch.bfloat16)
            w = synth.Paged(num_seqs=3, num_heads=H, num_kv_heads=HKV, head_dim=D,
                            page_tokens=P, q_dtype="bf16", kv_dtype="bf16", context_lens=ctx,
                            query_lens=np.ones(3, np.int32), scale=float(np.float32(D ** -0.5)),
                            q=q, k_pool=zeros, v_pool=zeros, page_table=np.zeros_like(table),
                            regen=dict(seed=seed, layer=layer, regen_pages=all_regen),
                            name=f"runtime-regen-{step}")
            check(w, *outs[1])  # everything regenerated
            check(w, *outs[0])  # as the runtime planned
            assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
            assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
        _, _, pages, blocks = rt.plan()
        if len(pages):
            # finite-value validation before admission: the regenerator counts
            # the non-finite values it stored per page
            nf = torch.full((len(pages),), 99, dtype=torch.int32, device=gpu)
            atlas.atlas_regenerate_pages(seed, layer, HKV, D, P, atlas.BF16,
                                         torch.from_numpy(pages).to(gpu),
                                         torch.from_numpy(blocks).to(gpu), 20, hot_k, hot_v,
                                         nonfinite=nf)
            counts = nf.cpu().numpy()
            assert (counts == 0).all()
            if step >= 1 and planted[0] < 2:  # a flagged block (planted on the host)
                counts[0] = 3                  # is taken back
                planted[0] += 1
            rt.refuse_admissions(pages, blocks, counts)
            forget_stale()
    st = rt.stats()
    assert st["evictions"] > 0 and st["admissions"] > 0 and st["regenerated_pages"] > 0
    assert st["refused_admissions"] >= 1


def test_promote_and_regenerate_count_nonfinite_values(gpu):
    """The finite check behind admission: a rebuilt page whose source has a
    NaN scale is all NaN (every element counted), a rejected destination
    reports -1, and regenerated pages count 0."""
    hot = torch.zeros((6, HKV, P, D), dtype=torch.float16, device=gpu)
    hot_v = torch.zeros_like(hot)
    pools = atlas.TierPools()
    pools.struct_size = ctypes.sizeof(atlas.TierPools)
    codes = torch.randint(-127, 128, (2, HKV, P, D), dtype=torch.int8, device=gpu)
    scales = torch.ones((2, HKV), dtype=torch.float32, device=gpu)
    scales[1, 1] = float("nan")  # slot 1, kv head 1: a corrupt scale
    pools.num_int8 = 2
    pools.int8_k, pools.int8_v = atlas._ptr(codes), atlas._ptr(codes)
    pools.int8_k_scale, pools.int8_v_scale = atlas._ptr(scales), atlas._ptr(scales)
    a = _args(gpu, torch.zeros((1, H, D), dtype=torch.bfloat16, device=gpu), hot, hot_v,
              torch.zeros((1, 4), dtype=torch.int32, device=gpu),
              torch.ones(1, dtype=torch.int32, device=gpu), torch.empty((1, H, D), device=gpu),
              torch.empty((1, H), device=gpu), kv=atlas.F16)
    a.num_blocks = 6
    src = torch.tensor([(1 << 30) | 0, (1 << 30) | 1, (1 << 30) | 0], dtype=torch.int32,
                       device=gpu)
    dst = torch.tensor([2, 3, 9], dtype=torch.int32, device=gpu)  # block 9 is outside
    nf = torch.full((3,), 99, dtype=torch.int32, device=gpu)
    atlas.atlas_promote_pages(a, pools, src, dst, nonfinite=nf)
    torch.cuda.synchronize()
    assert nf.cpu().tolist() == [0, 2 * P * D, -1]  # K and V of kv head 1
    kp = torch.empty((3, HKV, P, D), dtype=torch.bfloat16, device=gpu)
    vp = torch.empty_like(kp)
    nf2 = torch.full((2,), 99, dtype=torch.int32, device=gpu)
    atlas.atlas_regenerate_pages(9, 1, HKV, D, P, atlas.BF16,
                                 torch.tensor([0, 7], dtype=torch.int32, device=gpu),
                                 torch.tensor([2, 5], dtype=torch.int32, device=gpu), 3, kp, vp,
                                 nonfinite=nf2)
    torch.cuda.synchronize()
    assert nf2.cpu().tolist() == [0, -1]

