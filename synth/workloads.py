"""Seeded synthetic paged-attention workloads.

Everything here is input preparation: random draws, page placement, storage
rounding (round-to-nearest-even casts done by torch) and the symmetric int8 /
int4 storage encoding of cold pages.  The encoding produces the codes and
scales that the attention path and the oracle both consume as given; neither
side ever re-quantises.  No attention arithmetic lives here.

Shapes and distributions follow the workloads of the source pages:
  * CFR-Atlas README, "known-good deterministic benchmark run": one head,
    65,536-token context, head_dim 64, page_tokens 512, f32 K/V.
  * ARGUS (argus-cache 0.2.0), "Visual Architecture" and "Benchmark
    Methodology": an FP16 hot pool for recent tokens, INT8 and 2-way packed
    INT4 cold pages, fixed seed 42, batch-of-sequences decode of length 1.
  * CFR-Atlas README, overview: cold pages regenerated deterministically,
    hot pages resident.

Layouts (all row-major):
  q            [total_q][num_heads][head_dim]
  k_pool/v_pool[num_blocks][num_kv_heads][page_tokens][head_dim]
  page_table   [num_seqs][max_pages] int32 (physical block of each logical page)
  context_lens [num_seqs] int32, query_start [num_seqs + 1] int32
Tiered page-table entries carry the tier in bits 30-31 and the slot in bits
0-29.  Unused table entries and the tails of last pages point at / hold NaN
poison so that any read outside the causal context shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
TIER_HOT, TIER_I8, TIER_I4, TIER_F8, TIER_I2 = 0, 1, 2, 3, 4  # classes; INT2 is tier 3, kind 1
TIER_SHIFT = 30
SLOT_MASK = (1 << TIER_SHIFT) - 1


@dataclass
class Paged:
    """One seeded paged-attention problem (host metadata + tensors on `device`)."""

    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    page_tokens: int
    q_dtype: str
    kv_dtype: str
    context_lens: np.ndarray  # int32 [S]
    query_lens: np.ndarray  # int32 [S]
    scale: float  # exactly representable in f32
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    page_table: np.ndarray  # int32 [S][max_pages]
    tiers: Optional[dict] = None
    regen: Optional[dict] = None
    name: str = ""
    meta: dict = field(default_factory=dict)
    # positional policy: ALiBi slopes (f32, one per query head) and the
    # rotary base (0 = no rotary embedding)
    alibi_slopes: Optional[np.ndarray] = None
    rope_theta: float = 0.0

    @property
    def total_q(self) -> int:
        return int(self.query_lens.sum())

    @property
    def query_start(self) -> np.ndarray:
        qs = np.zeros(self.num_seqs + 1, dtype=np.int32)
        qs[1:] = np.cumsum(self.query_lens)
        return qs

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.query_lens == 1))

    @property
    def device(self) -> torch.device:
        return self.q.device

    def pages_of(self, s: int) -> int:
        return -(-int(self.context_lens[s]) // self.page_tokens)

    def to(self, device) -> "Paged":
        """Copy every tensor to `device` (metadata stays on the host)."""

        def mv(x):
            return x.to(device) if isinstance(x, torch.Tensor) else x

        tiers = None
        if self.tiers is not None:
            tiers = {k: mv(v) for k, v in self.tiers.items()}
        return Paged(
            self.num_seqs, self.num_heads, self.num_kv_heads, self.head_dim,
            self.page_tokens, self.q_dtype, self.kv_dtype, self.context_lens,
            self.query_lens, self.scale, mv(self.q), mv(self.k_pool),
            mv(self.v_pool), self.page_table, tiers, self.regen, self.name,
            dict(self.meta), self.alibi_slopes, self.rope_theta,
        )


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, gen, device, std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _context_lens(spec, rng: np.random.Generator) -> np.ndarray:
    c = spec["context_lens"]
    if isinstance(c, tuple) and c[0] == "uniform":
        _, lo, hi = c
        return rng.integers(lo, hi + 1, size=spec["num_seqs"]).astype(np.int32)
    arr = np.asarray(c, dtype=np.int32).reshape(-1)
    if arr.size == 1:
        arr = np.full(spec["num_seqs"], arr[0], dtype=np.int32)
    assert arr.size == spec["num_seqs"]
    return arr


def _query_lens(spec, ctx: np.ndarray) -> np.ndarray:
    ql = spec.get("query_lens", 1)
    arr = np.asarray(ql, dtype=np.int32).reshape(-1)
    if arr.size == 1:
        arr = np.full(ctx.size, arr[0], dtype=np.int32)
    return np.minimum(arr, np.maximum(ctx, 1)).astype(np.int32)


def _place(n_pages: np.ndarray, n_phys: int, placement: str, rng, offset=0):
    """Assign physical slots [offset, offset + n_phys) to logical pages."""
    if placement == "identity":
        ids = np.arange(n_phys, dtype=np.int64)
    else:
        ids = rng.permutation(n_phys).astype(np.int64)
    return ids + offset


def _poison_tails(pool: torch.Tensor, table: np.ndarray, ctx: np.ndarray, P: int):
    """NaN the rows past the context end in each sequence's last page."""
    for s in range(ctx.size):
        c = int(ctx[s])
        if c % P:
            blk = int(table[s, c // P])
            pool[blk, :, c % P:, :] = float("nan")


def _quantize(src: torch.Tensor, qmax: int):
    """Symmetric per-(page, kv_head) storage encoding of cold pages.

    scale = max|x| / qmax (f32), code = clamp(rint_half_even(x / scale), -qmax, qmax).
    An all-zero page gets scale 0 and codes 0.
    """
    amax = src.abs().amax(dim=(2, 3))  # [n][Hkv]
    scale = (amax / float(qmax)).to(torch.float32)
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = torch.round(src / safe[:, :, None, None]).clamp_(-qmax, qmax)
    codes = torch.where(scale[:, :, None, None] > 0, codes, torch.zeros_like(codes))
    return codes.to(torch.int8), scale


def _quantize_fp8(src: torch.Tensor):
    """FP8 (E4M3) storage encoding of cold pages: scale = max|x| / 448 (f32) per
    (page, kv head), codes from torch's float8_e4m3fn conversion of x / scale."""
    amax = src.abs().amax(dim=(2, 3))
    scale = (amax / 448.0).to(torch.float32)
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = (src / safe[:, :, None, None]).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def _pack_int2(codes: torch.Tensor) -> torch.Tensor:
    """Two's-complement 2-bit fields, element 4i + j in bits 2j, 2j + 1 of byte i."""
    c = codes.to(torch.int16) & 0x3
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)
            ).to(torch.uint8)


def _pack_int4(codes: torch.Tensor) -> torch.Tensor:
    """Two's-complement nibbles, element 2i in the low nibble of byte i."""
    c = codes.to(torch.int16) & 0xF
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).to(torch.uint8)


def build(spec: dict, device="cpu", seed: int = 42, name: str = "") -> Paged:
    """Build a seeded problem from a spec dict (see CONFIG_SPECS for the keys)."""
    rng = np.random.default_rng(seed)
    S = int(spec["num_seqs"])
    H = int(spec["num_heads"])
    Hkv = int(spec["num_kv_heads"])
    D = int(spec["head_dim"])
    P = int(spec["page_tokens"])
    q_dtype = spec.get("q_dtype", spec["kv_dtype"])
    kv_dtype = spec["kv_dtype"]
    ctx = _context_lens(spec, rng)
    qlens = _query_lens(spec, ctx)
    placement = spec.get("placement", "permuted")
    n_pages = -(-ctx // P)
    max_pages = int(spec.get("max_pages", max(1, int(n_pages.max()))))
    gen = _gen(seed, device)

    q = _normal((int(qlens.sum()), H, D), gen, device, spec.get("q_std", 1.0))
    q = q.to(DTYPES[q_dtype])
    scale = float(np.float32(spec.get("scale", 1.0 / math.sqrt(D))))

    tiers_spec = spec.get("tiers")
    regen_spec = spec.get("regen")
    tiers = None
    regen = None

    if tiers_spec is None:
        regen_pages = np.zeros(S, dtype=np.int32)
        if regen_spec is not None:
            frac = float(regen_spec.get("fraction", 0.75))
            regen_pages = np.array(
                [int(math.floor(frac * n)) for n in n_pages], dtype=np.int32)
            if "pages" in regen_spec:
                regen_pages = np.minimum(
                    np.asarray(regen_spec["pages"], dtype=np.int32), n_pages)
        resident = n_pages - regen_pages
        n_phys = int(resident.sum())
        ids = _place(n_pages, n_phys, placement, rng)
        poison = n_phys
        table = np.full((S, max_pages), poison, dtype=np.int32)
        k = 0
        for s in range(S):
            for p in range(int(regen_pages[s]), int(n_pages[s])):
                table[s, p] = ids[k]
                k += 1
        shape = (n_phys + 1, Hkv, P, D)
        if regen_spec is None:
            k_pool = _normal(shape, gen, device).to(DTYPES[kv_dtype])
            v_pool = _normal(shape, gen, device).to(DTYPES[kv_dtype])
        else:
            # Resident pages of a regenerated sequence hold the generator's
            # values; they are written by the library's own page regenerator
            # before use.  Until then they are NaN.
            k_pool = torch.full(shape, float("nan"), device=device,
                                dtype=DTYPES[kv_dtype])
            v_pool = torch.full(shape, float("nan"), device=device,
                                dtype=DTYPES[kv_dtype])
            regen = {
                "seed": int(regen_spec.get("seed", 42)),
                "layer": int(regen_spec.get("layer", 0)),
                "regen_pages": regen_pages,
            }
        k_pool[poison] = float("nan")
        v_pool[poison] = float("nan")
        if regen is None:
            _poison_tails(k_pool, table, ctx, P)
            _poison_tails(v_pool, table, ctx, P)
    else:
        # Tiered storage: pages holding any of the newest `hot_tokens` tokens
        # are f16/bf16 (kv_dtype); older pages are int8 or int4 by a seeded
        # fair coin per (sequence, page), shared by K and V and all kv heads
        # (with p_fp8 > 0, that share of the cold pages is FP8 E4M3).
        hot_tokens = int(tiers_spec.get("hot_tokens", 1024))
        p_i8 = float(tiers_spec.get("p_int8", 0.5))
        p_f8 = float(tiers_spec.get("p_fp8", 0.0))
        p_i2 = float(tiers_spec.get("p_int2", 0.0))
        tier_of = []
        for s in range(S):
            first_hot = max(0, int(ctx[s]) - hot_tokens) // P
            t = np.full(int(n_pages[s]), TIER_HOT, dtype=np.int32)
            cold = np.arange(int(n_pages[s])) < first_hot
            u = rng.random(int(n_pages[s]))
            coin = u < p_i8
            f8 = ~coin & (u < p_i8 + p_f8)
            i2 = ~coin & ~f8 & (u < p_i8 + p_f8 + p_i2)
            t[cold & coin] = TIER_I8
            t[cold & f8] = TIER_F8
            t[cold & i2] = TIER_I2
            t[cold & ~coin & ~f8 & ~i2] = TIER_I4
            tier_of.append(t)
        counts = [sum(int((t == k).sum()) for t in tier_of) for k in range(5)]
        slots = [list(_place(None, counts[k], placement, rng)) for k in range(3)]
        for k in (TIER_F8, TIER_I2):
            slots.append(list(_place(None, counts[k], placement, rng)) if counts[k] else [])
        poison_hot = counts[TIER_HOT]
        # entries are 32-bit words (tier in the top two bits), kept in an
        # int32 array with the same bits
        table = np.full((S, max_pages), poison_hot, dtype=np.uint32)
        used = [0, 0, 0, 0, 0]
        for s in range(S):
            for p, t in enumerate(tier_of[s]):
                slot = int(slots[t][used[t]])
                used[t] += 1
                if t == TIER_I2:  # the extension tier, kind 1
                    table[s, p] = (3 << TIER_SHIFT) | (1 << 28) | slot
                else:
                    table[s, p] = (int(t) << TIER_SHIFT) | slot
        table = table.view(np.int32)
        hot_shape = (counts[TIER_HOT] + 1, Hkv, P, D)
        k_pool = _normal(hot_shape, gen, device).to(DTYPES[kv_dtype])
        v_pool = _normal(hot_shape, gen, device).to(DTYPES[kv_dtype])
        k_pool[poison_hot] = float("nan")
        v_pool[poison_hot] = float("nan")
        ut = table.view(np.uint32)
        hot_only = np.where((ut >> TIER_SHIFT) == TIER_HOT, ut, poison_hot).astype(np.int64)
        _poison_tails(k_pool, hot_only, ctx, P)
        _poison_tails(v_pool, hot_only, ctx, P)
        tiers = {}
        for t, qmax, key in ((TIER_I8, 127, "i8"), (TIER_I4, 7, "i4")):
            n = max(1, counts[t])  # keep one slot so pointers are never empty
            for kv in ("k", "v"):
                src = _normal((n, Hkv, P, D), gen, device)
                codes, sc = _quantize(src, qmax)
                if key == "i4":
                    codes = _pack_int4(codes)
                tiers[f"{key}_{kv}"] = codes.contiguous()
                tiers[f"{key}_{kv}_scale"] = sc.contiguous()
        if counts[TIER_F8]:
            for kv in ("k", "v"):
                src = _normal((counts[TIER_F8], Hkv, P, D), gen, device)
                codes, sc = _quantize_fp8(src)
                tiers[f"f8_{kv}"] = codes.contiguous()
                tiers[f"f8_{kv}_scale"] = sc.contiguous()
        if counts[TIER_I2]:
            for kv in ("k", "v"):
                src = _normal((counts[TIER_I2], Hkv, P, D), gen, device)
                codes, sc = _quantize(src, 1)
                tiers[f"i2_{kv}"] = _pack_int2(codes).contiguous()
                tiers[f"i2_{kv}_scale"] = sc.contiguous()
        tiers["counts"] = counts

    # Positional policy (inputs, not arithmetic): the geometric ALiBi slopes
    # 2^(-8 (h + 1) / H) of Press et al. and a rotary base.
    pos_spec = spec.get("positional") or {}
    slopes = None
    if pos_spec.get("alibi"):
        slopes = np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)
    rope_theta = float(np.float32(pos_spec.get("rope_theta", 0.0)))

    return Paged(
        alibi_slopes=slopes, rope_theta=rope_theta,
        num_seqs=S, num_heads=H, num_kv_heads=Hkv, head_dim=D, page_tokens=P,
        q_dtype=q_dtype, kv_dtype=kv_dtype, context_lens=ctx, query_lens=qlens,
        scale=scale, q=q.contiguous(), k_pool=k_pool.contiguous(),
        v_pool=v_pool.contiguous(), page_table=table, tiers=tiers, regen=regen,
        name=name or spec.get("name", ""), meta={"seed": seed, "spec": spec},
    )


# The five workloads the library is measured on (sizes exact).
CONFIG_SPECS = {
    1: dict(name="decode_1h_ctx4096_d64_p512_f32", num_seqs=1,
            context_lens=4096, num_heads=1, num_kv_heads=1, head_dim=64,
            page_tokens=512, kv_dtype="f32", placement="identity"),
    2: dict(name="decode_32h_ctx65536_d64_p512_f32", num_seqs=1,
            context_lens=65536, num_heads=32, num_kv_heads=32, head_dim=64,
            page_tokens=512, kv_dtype="f32", q_std=0.5, placement="permuted"),
    3: dict(name="decode_gqa_64seq_ctx1k-32k_32q8kv_d128_p16_bf16",
            num_seqs=64, context_lens=("uniform", 1024, 32768), num_heads=32,
            num_kv_heads=8, head_dim=128, page_tokens=16, kv_dtype="bf16",
            placement="permuted"),
    4: dict(name="decode_tiered_64seq_f16hot_int8int4cold_d128_p16",
            num_seqs=64, context_lens=("uniform", 1024, 32768), num_heads=32,
            num_kv_heads=8, head_dim=128, page_tokens=16, q_dtype="bf16",
            kv_dtype="f16", placement="permuted",
            tiers=dict(hot_tokens=1024, p_int8=0.5)),
    5: dict(name="prefill_2048q_ctx131072_64q8kv_d128_p256_regen75",
            num_seqs=1, context_lens=131072, query_lens=2048, num_heads=64,
            num_kv_heads=8, head_dim=128, page_tokens=256, kv_dtype="bf16",
            placement="permuted", regen=dict(seed=42, layer=0, fraction=0.75)),
}


def config(n: int, device="cpu", seed: int = 42, **overrides) -> Paged:
    """Config `n` (1-5), optionally with spec fields overridden (e.g. a smaller
    context for tests)."""
    spec = dict(CONFIG_SPECS[n])
    spec.update(overrides)
    return build(spec, device=device, seed=seed, name=spec["name"])
