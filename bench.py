"""Benchmark of the paged, folded attention path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--no-cpu]

A step is one call of the library's attention entry point (all kernels of
the path: split-K attention plus the log-sum-exp merge) over one batch of
synthetic inputs already resident in HBM.  The default workload is the
CFR-Atlas-shaped decode (32 MHA heads, 65,536-token context, head_dim 64,
page_tokens 512, f32 K/V, pages shuffled by a seeded permutation); --config
selects one of the other four workloads (1-5).

Prints ONE JSON line: KV bytes/s of the whole call (value, GB/s, from K
plain calls between two synchronisations), context tokens/s per head, the
roofline of the main attention kernel (timed alone, in K further calls, with
HIP events recorded around it on the launch stream), and the f64 CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
BF16_DENSE_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "paged decode attention: KV bytes/s vs HBM peak; context tokens/s per head"


def algorithmic_work(w):
    """Bytes the method must read from HBM (resident K/V + scales) and FLOPs."""
    import numpy as np
    D, Hkv, P = w.head_dim, w.num_kv_heads, w.page_tokens
    G = w.num_heads // Hkv
    elem = {"f32": 4, "bf16": 2, "f16": 2}[w.kv_dtype]
    ctx = w.context_lens.astype(np.int64)
    kv_bytes = 0
    if w.tiers is not None:
        # K+V bytes per (token, kv head) by entry class: hot, int8, int4, FP8, INT2
        per_tok = {0: 2 * D * elem, 1: 2 * D, 2: D, 3: 2 * D, 4: D // 2}
        for s in range(w.num_seqs):
            for p in range(w.pages_of(s)):
                e = int(w.page_table[s, p]) & 0xFFFFFFFF
                tier = e >> 30 if e >> 30 < 3 else 3 + ((e >> 28) & 3)
                ntok = min(P, int(ctx[s]) - p * P)
                kv_bytes += ntok * Hkv * per_tok[tier]
                if tier:
                    kv_bytes += 8 * Hkv  # one f32 scale each for K and V
    elif w.regen is not None:
        for s in range(w.num_seqs):
            resident = max(0, int(ctx[s]) - int(w.regen["regen_pages"][s]) * P)
            kv_bytes += resident * Hkv * 2 * D * elem
    else:
        kv_bytes = int(ctx.sum()) * Hkv * 2 * D * elem
    # (q-head, key) pairs actually attended (causal)
    pairs = 0
    for s in range(w.num_seqs):
        n_q, c = int(w.query_lens[s]), int(ctx[s])
        pairs += sum(c - n_q + t + 1 for t in range(n_q)) if n_q > 1 else c
    pairs *= w.num_heads
    regen_elems = 0
    if w.regen is not None:
        regen_elems = int(sum(min(int(ctx[s]), int(w.regen["regen_pages"][s]) * P)
                              for s in range(w.num_seqs))) * Hkv * D * 2
    return dict(kv_bytes=kv_bytes, pairs=pairs, flops=4 * D * pairs,
                ctx_head_tokens=int(ctx.sum()) * w.num_heads, group=G,
                regen_elems=regen_elems)


PROBE_MIXES = {  # mix: (products, exponentials, multiply-adds, LDS bytes) per wave-iteration
    0: (0, 16, 0, 0), 1: (0, 0, 16, 0), 2: (16, 0, 0, 0), 3: (16, 16, 16, 0),
    4: (0, 0, 0, 16384), 5: (16, 0, 0, 16384), 6: (16, 0, 0, 16384), 7: (32, 0, 0, 16384)}


def issue_probe(torch, dev, iters: int = 2048) -> None:
    """Times each mix of atlas_issue_probe at one and two waves per SIMD and
    prints one JSON line per (mix, waves): the shader clock of the run, the
    SIMD cycles one wave-iteration takes, the fraction of them the matrix core
    is busy (32 cycles per 32x32x16 product) and the LDS bytes a CU reads per
    cycle."""
    from kv_cache_runtime_amd import atlas
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    sink = torch.zeros(1024, dtype=torch.float32, device=dev)
    blocks, cus, simds = 1024, 256, 1024
    for wps in (1, 2):
        for mix, (nm, ne, nf, lds) in PROBE_MIXES.items():
            atlas.atlas_issue_probe(mix, wps, iters, clocks, sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            atlas.atlas_issue_probe(mix, wps, iters, clocks, sink)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            ticks, real = (int(v) for v in clocks.cpu())
            ghz = ticks / real * 0.1 if real else 0.0
            cycles = ms * 1e-3 * ghz * 1e9
            wave_iters_per_simd = blocks * 4 * wps / simds * iters
            row = {"metric": "issue probe", "mix": mix, "waves_per_simd": wps,
                   "per_wave_iteration": {"mfma_32x32x16": nm, "exp": ne, "fma": nf,
                                          "lds_bytes": lds},
                   "ms": round(ms, 4), "clock_GHz": round(ghz, 3),
                   "simd_cycles_per_wave_iteration": round(cycles / wave_iters_per_simd, 2),
                   "mfma_busy": round(wave_iters_per_simd * nm * 32 / cycles, 3) if nm else None,
                   "lds_bytes_per_cu_cycle":
                       round(blocks * 4 * wps * iters * lds / cus / cycles, 1) if lds else None}
            print(json.dumps(row), flush=True)


def stream_read_gbps(torch, dev, nbytes: int = 2 << 30, reps: int = 10) -> float:
    """Read bandwidth of the library's plain streaming-read probe over nbytes
    (context for the fraction of the 8 TB/s peak)."""
    from kv_cache_runtime_amd import atlas
    blocks = 65536  # the best of 1024 .. 65536 workgroups on MI355X
    x = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    out = torch.empty(blocks, dtype=torch.int32, device=dev)
    for _ in range(2):
        atlas.atlas_read_probe(x, out, blocks)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        atlas.atlas_read_probe(x, out, blocks)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / reps / 1e3
    del x, out
    return round(nbytes / t / 1e9, 1)


def kernel_sources_digest() -> str:
    """Digest of the HIP sources: HBM byte counts taken with an older build
    no longer describe the kernels."""
    import hashlib
    csrc = os.path.join(ROOT, "kv_cache_runtime_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the main kernel for this workload, from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary (each counter scaled
    by its reading for a copy of known size), or None when the summary was
    taken with other kernel sources or does not cover the workload."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_digest()
    with open(path) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            tokens = line.split()
            if not all("=" in t for t in tokens):
                continue
            fields = dict(t.split("=", 1) for t in tokens)
            if fields.get("workload") == workload and fields.get("sources") == digest:
                return int(fields["bytes_per_launch"])
    return None


def measured_valu_busy(workload: str):
    """Fraction of the main kernel's resident-wave time spent issuing vector
    (VALU, MFMA included) instructions, SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES,
    from the committed rocprofv3 instruction-mix summary, or None when that
    summary was taken with other kernel sources or does not cover the
    workload."""
    path = os.path.join(ROOT, "profiles", "instruction_mix.txt")
    if not os.path.exists(path):
        return None
    digest, cur, vals = None, None, {}
    with open(path) as f:
        for line in f:
            if line.startswith("# kernel sources digest"):
                digest = line.split()[-1]
            elif line.startswith("workload="):
                cur = line.split()[0].split("=", 1)[1]
                vals[cur] = {}
            elif cur and line.startswith("  SQ_"):
                name, value = line.split()
                vals[cur][name] = float(value)
    v = vals.get(workload)
    if digest != kernel_sources_digest() or not v:
        return None
    return round(v["SQ_ACTIVE_INST_VALU"] / v["SQ_WAVE_CYCLES"], 3)


def alias_slots(w, n: int):
    """Rewrite the page table so that every entry names slot mod n of its own
    pool (tier bits kept): the same kernels and the same call shape, with
    every page read from a few cached blocks.  Diagnostic only; the results
    are not those of the workload."""
    import numpy as np
    t = w.page_table.astype(np.int64) & 0xFFFFFFFF
    tier = t >> 30
    low = np.where(tier == 3, (1 << 28) - 1, (1 << 30) - 1)
    slot = t & low
    out = (t & ~low) | (slot % n)
    w.page_table = out.astype(np.uint32).view(np.int32).copy()


def cpu_baseline(w, work, budget_s: float = 20.0):
    """Time the f64 oracle on a bounded sample of the same workload, running
    independent (sequence, kv head) groups on every host core this process
    may use (one worker thread per core; inside a worker the oracle's own
    OpenMP regions run single-threaded, so the cores are not oversubscribed)."""
    import ctypes
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    cores = max(1, len(os.sched_getaffinity(0)))
    host = oracle.HostView(w)
    host.pools()
    host.tier_arrays()
    G = w.num_heads // w.num_kv_heads
    seqs, _ = oracle.row_info(w)
    groups = []   # (rows, heads) per (sequence, kv head)
    for s in range(w.num_seqs):
        rows = np.nonzero(seqs == s)[0]
        for g in range(w.num_kv_heads):
            groups.append((s, rows, np.arange(g * G, (g + 1) * G)))
    # per-group cost estimate ~ pairs; sample whole groups until ~budget
    rng = np.random.default_rng(0)
    order = rng.permutation(len(groups))
    ctx = w.context_lens.astype(np.int64)

    def group_pairs(s, rows):
        n_q, c = int(w.query_lens[s]), int(ctx[s])
        return (sum(c - n_q + t + 1 for t in range(n_q)) if n_q > 1 else c) * G

    # roughly 25 ns per (pair, d) in f64 per core, measured pessimistically
    est_rate = 4e7 * cores / w.head_dim
    chosen, est = [], 0.0
    for i in order:
        s, rows, heads = groups[i]
        if w.regen is not None and len(rows) > 16:
            rows = rows[np.linspace(0, len(rows) - 1, 16).astype(int)]  # sample rows
        p = group_pairs(s, rows) if len(rows) == int(w.query_lens[s]) else \
            sum(int(ctx[s]) - int(w.query_lens[s]) + int(r - rows[0]) + 1 for r in rows) * G
        chosen.append((s, rows, heads, p))
        est += p / est_rate
        if est > budget_s:
            break

    def task(item):
        s, rows, heads, _ = item
        oracle.reference(w, rows=rows, heads=heads, host=host)

    cores = min(cores, len(chosen))  # threads actually used
    from oracle import oracle as oracle_impl
    oracle_impl.lib()  # loads the oracle and its OpenMP runtime
    gomp = ctypes.CDLL("libgomp.so.1")

    def one_thread_omp():
        gomp.omp_set_num_threads(1)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores, initializer=one_thread_omp) as ex:
        list(ex.map(task, chosen))
    dt = time.perf_counter() - t0
    done_pairs = sum(c[3] for c in chosen)
    frac = done_pairs / max(1, work["pairs"])
    kv_rate = work["kv_bytes"] * frac / dt / 1e9
    n_groups = len(chosen)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(kv_rate, 6), "unit": "GB/s",
        "cores": cores, "kind": "oracle", "cpu_model": cpu_model,
        "context_tokens_per_s_per_head": round(work["ctx_head_tokens"] * frac / dt, 1),
        "seconds": round(dt, 3),
        "sample": f"{n_groups} of {len(groups)} (sequence, kv head) groups "
                  f"({100 * frac:.2f}% of the (q-head, key) pairs), f64, "
                  f"{cores} host threads",
    }


def demote_plan(w, seed: int = 7):
    """Every full hot page of every sequence, each sent to int8 or int4 by a
    seeded fair coin (the cold split of the tiered workload), into fresh
    consecutive slots.  Returns (src blocks, dst entries (tier << 30 | slot),
    int8 count, int4 count)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    src, tiers = [], []
    for s in range(w.num_seqs):
        full = int(w.context_lens[s]) // w.page_tokens
        src.extend(int(b) for b in w.page_table[s, :full])
        tiers.extend(rng.integers(1, 3, size=full).tolist())
    tiers = np.asarray(tiers, dtype=np.int64)
    slot = np.zeros_like(tiers)
    slot[tiers == 1] = np.arange(int((tiers == 1).sum()))
    slot[tiers == 2] = np.arange(int((tiers == 2).sum()))
    dst = ((tiers << 30) | slot).astype(np.uint32)
    return (np.asarray(src, dtype=np.int32), dst.view(np.int32),
            int((tiers == 1).sum()), int((tiers == 2).sum()))


def write_path(args, torch, dev):
    """Time the KV write path: atlas_write_kv (a chunk's new K/V rows into
    their pages), atlas_demote_pages (hot pages encoded into int8 / int4, or
    into the 1-bit archive) or atlas_promote_pages (archived pages rebuilt
    into hot blocks), each against its HBM roofline, with the oracle's encoder
    or decoder timed on the host.""" 
    import numpy as np

    import synth
    from kv_cache_runtime_amd import atlas

    w = synth.config(args.config, device=dev, seed=42)
    if w.kv_dtype not in ("bf16", "f16") and args.op != "write_kv":
        sys.exit(f"{args.op} needs a bf16 or f16 hot pool (--config 3 or 5)")
    prob = atlas.Problem(w)
    D, Hkv, P = w.head_dim, w.num_kv_heads, w.page_tokens
    eb = w.k_pool.element_size()
    cpu = None
    if args.op == "write_kv":
        gen = torch.Generator(device=dev).manual_seed(5)
        k_new = torch.randn((w.total_q, Hkv, D), generator=gen, device=dev).to(w.k_pool.dtype)
        v_new = torch.randn((w.total_q, Hkv, D), generator=gen, device=dev).to(w.k_pool.dtype)
        units = w.total_q * Hkv                      # (row, kv head) pairs
        per_unit = 2 * 2 * D * eb                    # K and V: read the new row, write it

        def call():
            atlas.atlas_write_kv(prob.args, k_new, v_new)
        sample = None
        kernel = "write_kv_kernel"
    elif args.op in ("archive", "promote"):
        src, _, _, _ = demote_plan(w)
        n, K = len(src), args.outliers
        tiers = {}
        for kv in ("k", "v"):
            for t8 in ("i8", "i4"):
                tiers[f"{t8}_{kv}"] = torch.empty((0,), dtype=torch.uint8, device=dev)
                tiers[f"{t8}_{kv}_scale"] = torch.empty((0,), dtype=torch.float32, device=dev)
            tiers[f"b1_{kv}"] = torch.empty((n, Hkv, P * D // 8), dtype=torch.uint8, device=dev)
            tiers[f"b1_{kv}_scale"] = torch.empty((n, Hkv), dtype=torch.float32, device=dev)
            tiers[f"b1_{kv}_out"] = torch.empty((n, Hkv, K), dtype=torch.int32, device=dev)
        pools = atlas.make_tiers(tiers)
        src_t = torch.from_numpy(src).to(dev)
        b1_t = torch.from_numpy((np.arange(n, dtype=np.int64) | (0xE << 28)).astype(np.uint32)
                                .view(np.int32)).to(dev)
        rejected = torch.zeros(1, dtype=torch.int32, device=dev)
        units = n * Hkv
        per_unit = 2 * (P * D * eb + P * D // 8 + 4 + 4 * K)  # K and V: hot + archived bytes
        atlas.atlas_demote_pages(prob.args, pools, src_t, b1_t, rejected)  # fills the archive
        if args.op == "archive":
            def call():
                atlas.atlas_demote_pages(prob.args, pools, src_t, b1_t, rejected)
            kernel = "archive_kernel"
        else:
            def call():  # back into the blocks they came from
                atlas.atlas_promote_pages(prob.args, pools, b1_t, src_t, rejected)
            kernel = "promote_kernel"
        code_bytes = 0
    else:
        src, dst, n8, n4 = demote_plan(w)
        tiers = {}
        for kv in ("k", "v"):
            tiers[f"i8_{kv}"] = torch.empty((n8, Hkv, P, D), dtype=torch.int8, device=dev)
            tiers[f"i4_{kv}"] = torch.empty((n4, Hkv, P, D // 2), dtype=torch.uint8, device=dev)
            tiers[f"i8_{kv}_scale"] = torch.empty((n8, Hkv), dtype=torch.float32, device=dev)
            tiers[f"i4_{kv}_scale"] = torch.empty((n4, Hkv), dtype=torch.float32, device=dev)
        pools = atlas.make_tiers(tiers)
        src_t = torch.from_numpy(src).to(dev)
        dst_t = torch.from_numpy(dst).to(dev)
        rejected = torch.zeros(1, dtype=torch.int32, device=dev)
        units = len(src) * Hkv                       # (page, kv head) blocks
        # read K and V of the block, write their codes and two f32 scales
        code_bytes = (n8 * 2 * P * D + n4 * P * D) * Hkv
        per_unit = None

        def call():
            atlas.atlas_demote_pages(prob.args, pools, src_t, dst_t, rejected)
        kernel = "demote_kernel"
    alg_bytes = units * per_unit if per_unit else units * (2 * P * D * eb + 8) + code_bytes

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    # one kernel per call, launched on torch's current stream: per-call events
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    kern = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    kern_avg = sum(kern) / K
    if args.op != "write_kv":
        assert int(rejected) == 0

    if args.op == "demote" and not args.no_cpu:
        import oracle
        host = oracle.HostView(w)
        (ka, kind), (va, _) = host.pools()
        order = np.random.default_rng(0).permutation(len(src))
        t0, n_blocks, n_bytes = time.perf_counter(), 0, 0
        for i in order:
            e = int(np.uint32(dst[i]))
            qmax = 127 if e >> 30 == 1 else 7
            for arr in (ka, va):
                for g in range(Hkv):
                    x = oracle.widen_bits(arr[int(src[i]), g], kind).astype(np.float32)
                    codes, _ = oracle.quantize_block(x, qmax)
                    if qmax == 7:
                        oracle.pack_int4(codes)
                    n_bytes += P * D * eb + 4 + (P * D if qmax == 127 else P * D // 2)
            n_blocks += 1
            if time.perf_counter() - t0 > 10.0:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": round(n_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "seconds": round(dt, 3),
               "sample": f"{n_blocks} of {len(src)} pages (all {Hkv} kv heads, K and V), "
                         f"numpy f32 encoder, one host thread"}

    if args.op in ("archive", "promote") and not args.no_cpu:
        import oracle
        host = oracle.HostView(w)
        (ka, kind), (va, _) = host.pools()
        order = np.random.default_rng(0).permutation(len(src))
        t0, n_blocks, n_bytes = time.perf_counter(), 0, 0
        for i in order:
            for arr in (ka, va):
                for g in range(Hkv):
                    x = oracle.widen_bits(arr[int(src[i]), g], kind).astype(np.float32).ravel()
                    enc = oracle.encode_1bit(x, args.outliers)
                    if args.op == "promote":
                        oracle.hot_bits(oracle.decode_1bit(*enc, x.size), w.kv_dtype)
                    n_bytes += P * D * eb + P * D // 8 + 4 + 4 * args.outliers
            n_blocks += 1
            if time.perf_counter() - t0 > 10.0:
                break
        dt = time.perf_counter() - t0
        what = "encoder" if args.op == "archive" else "encoder + decoder"
        cpu = {"value": round(n_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "seconds": round(dt, 3),
               "sample": f"{n_blocks} of {len(src)} pages (all {Hkv} kv heads, K and V), "
                         f"numpy 1-bit {what}, one host thread"}

    # context: a plain device copy (read + write bytes), the practical roof of
    # a kernel that streams reads and writes together
    src_c = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst_c = torch.empty_like(src_c)
    dst_c.copy_(src_c)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst_c.copy_(src_c)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = round(2 * (1 << 30) * 5 / (c0.elapsed_time(c1) / 1e3) / 1e9, 1)
    del src_c, dst_c

    achieved = alg_bytes / (kern_avg / 1e3) / 1e9
    line = {
        "metric": {"write_kv": "KV write: bytes/s moved into the pages",
                   "demote": "KV demotion: bytes/s of hot pages read + codes written",
                   "archive": "KV archiving: bytes/s of hot pages read + 1-bit pages written",
                   "promote": "KV reconstruction: bytes/s of 1-bit pages read + hot pages "
                              "written"}[args.op],
        "value": round(alg_bytes / (ms / 1e3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"write_kv": w.kv_dtype, "demote": f"{w.kv_dtype}->int8+int4",
                  "archive": f"{w.kv_dtype}->1bit", "promote": f"1bit->{w.kv_dtype}"}[args.op],
        "data": "synthetic",
        "config": {"workload": f"{args.op}:{w.name}", "rows": w.total_q,
                   "num_kv_heads": Hkv, "head_dim": D, "page_tokens": P,
                   "units": units, "bytes": alg_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{args.op}:{w.name}"),
                     "kernel": kernel, "kernel_avg_ms": round(kern_avg, 5),
                     "kernel_median_ms": round(kern[K // 2], 5),
                     "algorithmic_per_launch": alg_bytes},
        "copy_GBps": copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="workload: 1 one-head f32 decode over 4,096 keys; 2 (default) 32-head "
                         "f32 decode over 65,536 keys; 3 64-sequence bf16 GQA decode over "
                         "1k-32k keys; 4 the same with f16 hot and int8/int4 cold pages; 5 a "
                         "2,048-query bf16 prefill over 131,072 keys, 75 %% regenerated")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--stream", type=int, default=1,
                    help="also time a plain streaming read of 2 GiB (the library's read "
                         "probe) as context for the HBM fraction (0 = skip)")
    ap.add_argument("--flush-mib", type=int, default=-1,
                    help="after timing, time calls with this many MiB written between them "
                         "(Infinity Cache flushed); -1 = 512 for config 1, else off")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain device-to-device copy of this many "
                         "bytes three times (calibrates the HBM byte counters)")
    ap.add_argument("--alibi", action="store_true",
                    help="attention with ALiBi slopes 2^(-8 (h + 1) / H)")
    ap.add_argument("--rope-theta", type=float, default=0.0,
                    help="attention with a rotary embedding of this base (0 = none)")
    ap.add_argument("--p-fp8", type=float, default=0.0,
                    help="tiered 64-sequence workload (--config 4): share of the cold pages stored as FP8 "
                         "E4M3, the rest split evenly between int8 and int4")
    ap.add_argument("--p-int2", type=float, default=0.0,
                    help="tiered 64-sequence workload (--config 4): share of the cold pages stored as INT2")
    ap.add_argument("--alias-slots", type=int, default=0,
                    help="diagnostic: map every page-table entry's slot to slot mod N in "
                         "its own pool, so the call reads N blocks per pool from cache "
                         "instead of HBM (the kernel's floor without memory traffic)")
    ap.add_argument("--op", choices=("attention", "write_kv", "demote", "archive", "promote",
                                     "probe"),
                    default="attention",
                    help="attention (default): the attention call of --config; write_kv: "
                         "writing a chunk's new K/V into its pages; demote: encoding every "
                         "full hot page of --config into the int8 / int4 tiers; archive: "
                         "encoding them into the 1-bit archive; promote: rebuilding the "
                         "archived pages into hot blocks; probe: the issue rates of "
                         "matrix products, exponentials, multiply-adds and LDS reads the "
                         "matrix-core prefill is built from (one JSON line per mix)")
    ap.add_argument("--outliers", type=int, default=16,
                    help="FP16 outliers per (page, kv head) block for archive / promote")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the attention path has no multi-GPU "
              "mode (each GPU would run its own shard of sequences or kv heads "
              "independently); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from kv_cache_runtime_amd import atlas

    dev = torch.device("cuda:0")
    atlas.load()
    if args.op == "probe":
        issue_probe(torch, dev)
        return
    if args.op != "attention":
        write_path(args, torch, dev)
        return
    positional = {}
    if args.alibi:
        positional["alibi"] = True
    if args.rope_theta:
        positional["rope_theta"] = args.rope_theta
    extra = {"positional": positional} if positional else {}
    if args.p_fp8 > 0 or args.p_int2 > 0:
        if args.config != 4:
            sys.exit("--p-fp8 / --p-int2 apply to the tiered workload (--config 4)")
        rest = 1.0 - args.p_fp8 - args.p_int2
        extra["tiers"] = dict(hot_tokens=1024, p_int8=rest / 2, p_fp8=args.p_fp8,
                              p_int2=args.p_int2)
    w = synth.config(args.config, device=dev, seed=42, **extra)
    if args.alias_slots > 0:
        alias_slots(w, args.alias_slots)
    prob = atlas.Problem(w, split_tokens=args.split_tokens)
    if w.regen is not None:
        prob.fill_resident_from_regenerator()
    torch.cuda.synchronize()
    work = algorithmic_work(w)

    for _ in range(args.warmup):
        prob.run()
    torch.cuda.synchronize()

    K = args.steps
    # the K timed steps: calls as a caller makes them, nothing recorded inside
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(K):
        prob.run()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K

    # K more steps with HIP events recorded by the library on the launch
    # stream around the main attention kernel (the roofline's kernel time)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in kev:  # create the underlying HIP events
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(K):
        prob.args.profile_events[0] = kev[i][0].cuda_event
        prob.args.profile_events[1] = kev[i][1].cuda_event
        prob.run()
    torch.cuda.synchronize()
    kern_ms = sorted(a.elapsed_time(b) for a, b in kev)
    kern_avg = sum(kern_ms) / K
    prob.args.profile_events[0] = None
    prob.args.profile_events[1] = None

    t = ms_per_step / 1e3
    value = work["kv_bytes"] / t / 1e9
    ctx_per_head = work["ctx_head_tokens"] / t
    prefill = not w.is_decode
    if prefill:
        achieved = work["flops"] / (kern_avg / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": BF16_DENSE_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_DENSE_TFLOPS, 4),
                "traffic": None}
    else:
        achieved = work["kv_bytes"] / (kern_avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None}
    # the committed counter summaries describe the default call of each
    # workload: a positional policy, another cold mix, aliased slots, another
    # window or an environment-selected kernel runs other code or other bytes
    variant = bool(positional or "tiers" in extra or args.alias_slots > 0 or args.split_tokens
                   or any(k in os.environ for k in ("ATLAS_DECODE_VALU", "ATLAS_NO_MFMA",
                                                    "ATLAS_SPLIT_TOKENS")))
    roof["traffic"] = None if variant else measured_traffic(w.name)
    # issue-side view of the same kernel (rocprofv3 SQ counters, committed summary)
    roof["valu_busy"] = None if variant else measured_valu_busy(w.name)
    roof["kernel_avg_ms"] = round(kern_avg, 5)
    roof["kernel_median_ms"] = round(kern_ms[K // 2], 5)
    roof["kernel_min_ms"] = round(kern_ms[0], 5)
    roof["kernel_max_ms"] = round(kern_ms[-1], 5)
    roof["algorithmic_per_launch"] = work["flops"] if prefill else work["kv_bytes"]

    stream = stream_read_gbps(torch, dev) if args.stream else None

    # cold calls: the Infinity Cache (MALL) is flushed by writing flush_mib
    # MiB between calls, so a small working set is read from HBM again
    flush_mib = args.flush_mib if args.flush_mib >= 0 else (512 if args.config == 1 else 0)
    cold = None
    if flush_mib > 0:
        junk = torch.empty(flush_mib << 18, dtype=torch.float32, device=dev)
        reps = min(K, 20)
        calls, kerns = [], []
        for i in range(reps):
            junk.fill_(float(i))
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0.record()  # creates the HIP events; re-recorded by the library
            k1.record()
            c0.record()
            prob.args.profile_events[0] = k0.cuda_event
            prob.args.profile_events[1] = k1.cuda_event
            prob.run()
            c1.record()
            torch.cuda.synchronize()
            calls.append(c0.elapsed_time(c1))
            kerns.append(k0.elapsed_time(k1))
        prob.args.profile_events[0] = None
        prob.args.profile_events[1] = None
        del junk
        calls.sort()
        kerns.sort()
        cold = {"flush_mib": flush_mib, "reps": reps,
                "call_ms_median": round(calls[reps // 2], 5),
                "kernel_ms_median": round(kerns[reps // 2], 5),
                "kv_GBps_call": round(work["kv_bytes"] / (calls[reps // 2] / 1e3) / 1e9, 2)}

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, work)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "f16": "f16"}[w.kv_dtype] if w.tiers is None
        else "f16+int8+int4",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs, "context_tokens": int(w.context_lens.sum()),
            "query_rows": w.total_q, "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "page_tokens": w.page_tokens, "kv_bytes": work["kv_bytes"],
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "context_tokens_per_s_per_head": round(ctx_per_head, 1),
        "roofline": roof,
        "stream_read_GBps": stream,
        "cold": cold,
        "cpu_baseline": cpu,
    }
    if positional:
        line["config"]["positional"] = positional
    if args.alias_slots > 0:
        # the same calls over N blocks per pool: achieved bytes/s are not HBM's
        line["config"]["alias_slots"] = args.alias_slots
        line["metric"] += " (diagnostic: slots aliased, reads served from cache)"
    if args.p_fp8 > 0 or args.p_int2 > 0:
        line["config"]["cold_fp8_share"] = args.p_fp8
        line["config"]["cold_int2_share"] = args.p_int2
        line["dtype"] = "f16+fp8+int8+int4+int2"
    if prefill:
        line["tflops"] = round(work["flops"] / t / 1e12, 3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
