"""Python side of the f64 CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the attention library.  It shares
no code with the GPU path: it has its own widening of stored values, its own
int8/int4 decoding, its own page-table walk and its own SplitMix64 (in
attention.c).

Definitions followed:
  * attention: RustAttention README, "Mathematical Framework Covered"
    (softmax(QK^T / sqrt(d_k) + Mask) V), causal mask and max subtraction from
    its "Architectural Features Included" list;
  * causal alignment of a chunk of new queries: the n_q new rows are the last
    n_q positions of the context, so row t of a sequence with context c sees
    keys 0 .. c - n_q + t (the chunk's own earlier tokens included);
  * paging: logical token j of sequence s lives in block table[s][j // P], row
    j % P (CFR-Atlas README, PageKey + token_range per page);
  * cold tiers: ARGUS "Visual Architecture" (FP8; INT8; INT4 2-way
    bit-packed; INT2 4-way bit-packed), symmetric: value = code * scale (FP8:
    E4M3 value of the code times scale), one scale per (page, kv head) for K
    and one for V; int4 element 2i in the low nibble, int2 element 4i + j in
    bits 2j of byte i, two's complement; INT2 and FP8 entries share tier 3;
  * the 1-bit archival tier: ARGUS "Visual Architecture" and its heatmap
    legend (8-way sign-packed with FP16 outlier preservation) and its
    "Limitations" (archival pages are not attended directly; the overview's
    transient FP16 reconstruction brings them back first);
  * regenerated pages: the value definition in attention.c;
  * split merge: log-sum-exp combination of normalised partial results
    (attnres AGENTS.md, "online softmax merge").
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

TIER_SHIFT = 30
SLOT_MASK = (1 << TIER_SHIFT) - 1
# tier 3 is the extension tier: bits 29-28 give the kind, bits 27-0 the slot
EXT_KIND_SHIFT = 28
EXT_SLOT_MASK = (1 << EXT_KIND_SHIFT) - 1


def entry_class(entry: int):
    """(class, slot) of a tiered page-table entry: class 0 hot, 1 int8, 2 int4,
    3 FP8 (tier 3, kind 0), 4 INT2 (tier 3, kind 1), 5 1-bit (tier 3, kind 2),
    6 names no pool (tier 3, kind 3)."""
    e = int(entry) & 0xFFFFFFFF
    tier = e >> TIER_SHIFT
    if tier < 3:
        return tier, e & SLOT_MASK
    kind = (e >> EXT_KIND_SHIFT) & 3
    return 3 + kind, e & EXT_SLOT_MASK


def build(force: bool = False) -> str:
    """Compile attention.c with gcc (-O2, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
            "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, dbl, p = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.oracle_attend.argtypes = [i64, i64, i64, p, p, p, p, dbl, p, p, p]
        L.oracle_attend.restype = None
        L.oracle_attend_folded.argtypes = [i64, i64, i64, p, p, p, p, dbl, i64, p, p]
        L.oracle_attend_folded.restype = None
        L.oracle_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.oracle_splitmix64.restype = ctypes.c_uint64
        L.oracle_regen_values.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, i64, i64, i64, i64, p]
        L.oracle_regen_values.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Core definitions
# ---------------------------------------------------------------------------

def attend(q, k, v, visible, scale, page_tokens=None, slope=None):
    """Exact causal attention of rows `q` [n][d] over one head's keys.

    k, v: [n_keys][d]; visible[r] = number of leading keys row r may see.
    slope: optional [n] ALiBi slopes, one per row (score j of row r gains
    -slope[r] * (visible[r] - 1 - j)).
    Returns (out [n][d] f64, lse [n] f64, natural log).  With `page_tokens`
    the folded (page-by-page online softmax) variant is used instead.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    vis = np.ascontiguousarray(visible, dtype=np.int64)
    n, d = q.shape
    n_keys = k.shape[0]
    assert k.shape == (n_keys, d) and v.shape == (n_keys, d) and vis.shape == (n,)
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    if page_tokens is None:
        sl = None if slope is None else np.ascontiguousarray(slope, dtype=np.float64)
        assert sl is None or sl.shape == (n,)
        lib().oracle_attend(n, d, n_keys, _ptr(q), _ptr(k), _ptr(v), _ptr(vis),
                            float(scale), None if sl is None else _ptr(sl),
                            _ptr(out), _ptr(lse))
    else:
        assert slope is None, "the folded variant has no positional bias"
        lib().oracle_attend_folded(n, d, n_keys, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(vis), float(scale), int(page_tokens),
                                   _ptr(out), _ptr(lse))
    return out, lse


def rope(x, pos, theta):
    """Rotary position embedding (Su et al., "RoFormer", 2021, section 3.4),
    the other positional policy the CFR-Atlas README lists: dims (2i, 2i + 1)
    of a row at position pos are rotated by the angle pos * theta^(-2i/d),
    (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).

    x: [..., d] (d even), pos: broadcastable to x[..., 0].  f64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    freq = np.float64(theta) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    ang = pos * freq
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def round_bf16(x):
    """Round f64 values to the nearest bfloat16 value (8 significant bits,
    ties to even), directly from f64 (no intermediate f32).  Finite inputs
    within the bf16 normal range, which is all this oracle feeds it."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)              # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def merge_splits(part_out, part_lse):
    """Log-sum-exp merge of normalised partials.

    part_out [splits][rows][d], part_lse [splits][rows] (natural log; -inf for
    an empty split).  lse = log sum_s exp(lse_s); out = sum_s exp(lse_s - lse)
    o_s.  All-empty rows give out 0 and lse -inf.
    """
    po = np.asarray(part_out, dtype=np.float64)
    pl = np.asarray(part_lse, dtype=np.float64)
    m = pl.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - m_safe[None, :]), 0.0)
    z = w.sum(axis=0)
    out = np.where(finite[:, None],
                   (w[:, :, None] * po).sum(axis=0) / np.where(z > 0, z, 1.0)[:, None],
                   0.0)
    lse = np.where(finite, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return out, lse


def splitmix64(seed: int, n: int) -> int:
    """n-th output (n >= 1) of SplitMix64 seeded with `seed`."""
    return int(lib().oracle_splitmix64(seed & (2**64 - 1), n))


def regen_values(seed, layer, kv_head, token0, n_tokens, d, kv) -> np.ndarray:
    """Regenerated K (kv=0) or V (kv=1) rows [n_tokens][d] as f32 (bf16-exact)."""
    dst = np.empty((int(n_tokens), int(d)), dtype=np.float32)
    if n_tokens:
        lib().oracle_regen_values(int(seed), int(layer), int(kv_head), int(token0),
                                  int(n_tokens), int(d), int(kv), _ptr(dst))
    return dst


# ---------------------------------------------------------------------------
# Stored values -> exact f64 (or f32 for the bit-exact decode checks)
# ---------------------------------------------------------------------------

def _np(t):
    """torch tensor (any device) -> numpy array of the same bits."""
    import torch
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), "bf16"
    if t.dtype == torch.float16:
        return t.numpy(), "f16"
    if t.dtype == torch.float32:
        return t.numpy(), "f32"
    return t.numpy(), str(t.dtype)


def widen_bits(a: np.ndarray, kind: str) -> np.ndarray:
    """Exact f64 value of stored f32 / bf16 (raw uint16 bits) / f16 numbers."""
    if kind == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def widen(t) -> np.ndarray:
    a, kind = _np(t)
    return widen_bits(a, kind)


def int4_codes(packed: np.ndarray) -> np.ndarray:
    """Unpack two's-complement nibbles: byte i holds element 2i (low nibble)
    and element 2i+1 (high nibble)."""
    b = packed.astype(np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_f32(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """f32(code * scale) with one scale per leading index pair [n][Hkv]."""
    return (codes.astype(np.float32) * scale.astype(np.float32)[:, :, None, None]
            ).astype(np.float32)


def quantize_block(x: np.ndarray, qmax: int):
    """Symmetric encoding of one (page, kv head) block of K or V into cold-tier
    codes (argus-cache, "Visual Architecture": INT8 and INT4 tiers; reading:
    one f32 scale per block, symmetric, round half to even).

    scale = f32(max |x|) / qmax and code = clamp(rint(f32(x) / scale), -qmax,
    qmax), both divisions in f32 with correct rounding, so that a device
    computing in f32 takes the same integer decisions.  An all-zero block gets
    scale 0 and codes 0.  A block holding a NaN or an infinity gets a NaN scale
    and codes 0, so that every value read back from it is NaN (reading: bad
    values fail loudly, attnres AGENTS.md, "Non-Negotiable Invariants").
    Returns (int16 codes of x's shape, np.float32 scale).
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        return np.zeros(x.shape, dtype=np.int16), np.float32(np.nan)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(qmax))
    if scale == 0:
        return np.zeros(x.shape, dtype=np.int16), np.float32(0.0)
    q = np.rint(np.divide(x, scale, dtype=np.float32))
    return np.clip(q, -qmax, qmax).astype(np.int16), scale


def fp8_e4m3_value(code):
    """Value of an OCP FP8 E4M3 code (the "e4m3fn" variant), the FP8 tier of
    argus-cache's "Visual Architecture" cascade as read here: sign in bit 7,
    exponent in bits 6-3 with bias 7, mantissa in bits 2-0; exponent 0 is
    subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN; there are no infinities.
    Largest finite magnitude 448."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = (code & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((code & 0x7F) == 0x7F, np.nan, sign * mag)


def fp8_e4m3_encode(y):
    """E4M3 code nearest to each value of y (f32), by brute force over the 127
    finite magnitudes: ties go to the even code, magnitudes above 448
    saturate to 448, and the sign bit is y's sign bit."""
    y = np.asarray(y, dtype=np.float32)
    codes = np.arange(0x7F)
    mags = fp8_e4m3_value(codes)
    a = np.abs(y.astype(np.float64))[..., None]
    d = np.abs(a - mags)
    cand = d == d.min(axis=-1, keepdims=True)
    first = np.where(cand, codes, 0x7F).min(axis=-1)
    even = np.where(cand & (codes % 2 == 0), codes, 0x7F).min(axis=-1)
    mag_code = np.where(cand.sum(axis=-1) > 1, even, first)
    return (mag_code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_block_fp8(x: np.ndarray):
    """FP8 (E4M3) encoding of one (page, kv head) block (reading: one f32
    scale per block, like the integer tiers): scale = f32(max |x|) / 448 and
    code = nearest E4M3 code to f32(x) / scale, both divisions correctly
    rounded f32.  An all-zero block gets scale 0 and codes 0; a block holding
    a NaN or an infinity a NaN scale and codes 0 (as for the integer tiers).
    Returns (uint8 codes of x's shape, np.float32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        return np.zeros(x.shape, dtype=np.uint8), np.float32(np.nan)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(448.0))
    if scale == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0.0)
    return fp8_e4m3_encode(np.divide(x, scale, dtype=np.float32)), scale


def int2_codes(packed: np.ndarray) -> np.ndarray:
    """INT2 (argus-cache "4-way Bit-Packed" as read here): element 4i + j is
    bits 2j, 2j + 1 of byte i, two's complement (-2 .. 1)."""
    p = np.asarray(packed).astype(np.int16)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 4,), dtype=np.int16)
    for j in range(4):
        f = (p >> (2 * j)) & 3
        out[..., j::4] = np.where(f >= 2, f - 4, f)
    return out


def pack_int2(codes: np.ndarray) -> np.ndarray:
    """Inverse of int2_codes: 4 codes per byte, element 4i + j in bits 2j, 2j+1."""
    c = np.asarray(codes).astype(np.int16) & 3
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)
            ).astype(np.uint8)


B1_MAX_OUTLIERS = 64


def f16_bits(x) -> np.ndarray:
    """IEEE half-precision bit patterns of x (f32), round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def encode_1bit(x: np.ndarray, n_out: int):
    """The 1-bit archival encoding of one (page, kv head) block, as read here
    from ARGUS's "8-way sign-packed with FP16 outlier preservation":

      * outliers: the n_out elements of largest magnitude (ordered by the bit
        pattern of f32 |x|, so NaN ranks above inf; ties go to the lower
        index), kept as (index, FP16 value) pairs, one uint32 each: index in
        bits 0-15, the FP16 bits (round to nearest even) in bits 16-31,
        sorted by index;
      * signs: bit j of byte i is 1 iff element 8 i + j is negative (x < 0;
        -0.0 and NaN give 0), for every element, outliers included;
      * scale: the mean |x| over the other elements (the scale that minimises
        the squared error of x ~ scale * sign), the sum taken in f64 and the
        quotient rounded to f32; 0 when every element is an outlier.

    x is the block flattened in storage order (row-major [P][D]).  Returns
    (uint8 signs [n / 8], np.float32 scale, uint32 outliers [min(n_out, n)]).
    """
    x = np.asarray(x, dtype=np.float32).ravel()
    n = x.size
    k = min(int(n_out), n)
    key = np.abs(x).view(np.uint32).astype(np.int64)
    order = np.lexsort((np.arange(n), -key))  # magnitude down, index up
    idx = np.sort(order[:k])
    is_out = np.zeros(n, dtype=bool)
    is_out[idx] = True
    rest = np.abs(x[~is_out]).astype(np.float64)
    scale = np.float32(rest.sum() / rest.size) if rest.size else np.float32(0.0)
    signs = np.packbits((x < 0).astype(np.uint8), bitorder="little")
    outliers = idx.astype(np.uint32) | (f16_bits(x[idx]).astype(np.uint32) << 16)
    return signs, scale, outliers


def decode_1bit(signs: np.ndarray, scale, outliers: np.ndarray, n: int) -> np.ndarray:
    """Values of a 1-bit block as f32: -scale where the sign bit is set,
    +scale elsewhere, then each outlier entry in list order writes its FP16
    value at its index (an index >= n is ignored; a later entry for the same
    index wins)."""
    bits = np.unpackbits(np.asarray(signs, dtype=np.uint8), bitorder="little")[:n]
    sc = np.float32(scale)
    out = np.where(bits == 1, -sc, sc).astype(np.float32)
    for e in np.asarray(outliers).astype(np.int64).ravel() & 0xFFFFFFFF:  # uint32 bits
        i = int(e) & 0xFFFF
        if i < n:
            out[i] = np.float32(np.uint16(int(e) >> 16).view(np.float16))
    return out


def hot_bits(x, kind: str) -> np.ndarray:
    """Bits of f32 values x stored in a hot pool of element type kind ("f32",
    "f16" or "bf16"), rounded to nearest even: what reconstructing a page
    into a hot block writes.  bf16 rounding goes through round_bf16 (normal
    range, which is all it is fed here)."""
    x = np.asarray(x, dtype=np.float32)
    if kind == "f32":
        return x.view(np.uint32)
    if kind == "f16":
        return f16_bits(x)
    r = round_bf16(x.astype(np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2i in the low nibble of byte i (the
    argus-cache INT4 "2-way bit-packed" layout as read here)."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Paged problems (synth.Paged) -> logical per-sequence K/V and references
# ---------------------------------------------------------------------------

class HostView:
    """Host copies of a problem's stored arrays, made once."""

    def __init__(self, w):
        self.w = w
        self.k = None
        self.v = None
        self.tiers = None

    def pools(self):
        if self.k is None:
            self.k = _np(self.w.k_pool)
            self.v = _np(self.w.v_pool)
        return self.k, self.v

    def tier_arrays(self):
        if self.tiers is None and self.w.tiers is not None:
            self.tiers = {}
            for key, val in self.w.tiers.items():
                if key == "counts":
                    continue
                self.tiers[key] = _np(val)[0]
        return self.tiers


def logical_kv(w, s: int, g: int, n_tokens: int | None = None, host=None):
    """Logical K, V of sequence s, kv head g: ([n][d] f64, [n][d] f64).

    Walks the page table page by page; each page comes from its storage tier
    or from the resident pool.  In a regenerated problem every K/V value is
    defined by the regenerator (its resident pages hold the same values by
    construction), so all pages are taken from the regenerator.

    Positional policy: with a rotary embedding (w.rope_theta > 0) stored K
    pages hold rotated keys, as a model caches them; regenerated keys are
    produced unrotated, rotated here by their token position and rounded to
    bf16, the value a bf16 cache holds for them."""
    host = host or HostView(w)
    theta = float(getattr(w, "rope_theta", 0.0) or 0.0)
    P, D = w.page_tokens, w.head_dim
    ctx = int(w.context_lens[s]) if n_tokens is None else int(n_tokens)
    K = np.zeros((ctx, D), dtype=np.float64)
    V = np.zeros((ctx, D), dtype=np.float64)
    n_regen = -(-ctx // P) if w.regen is not None else 0
    for p in range(-(-ctx // P)):
        t0, t1 = p * P, min(ctx, (p + 1) * P)
        rows = t1 - t0
        if p < n_regen:
            rs = w.regen
            K[t0:t1] = regen_values(rs["seed"], rs["layer"], g, t0, rows, D, 0)
            V[t0:t1] = regen_values(rs["seed"], rs["layer"], g, t0, rows, D, 1)
            if theta:
                # the regenerator replays K before its rotation; the cached
                # key it must reproduce is the rotated key in bf16
                K[t0:t1] = round_bf16(rope(K[t0:t1], np.arange(t0, t1), theta))
            continue
        entry = int(w.page_table[s, p]) & 0xFFFFFFFF
        if w.tiers is None:
            (ka, kind), (va, _) = host.pools()
            K[t0:t1] = widen_bits(ka[entry, g, :rows], kind)
            V[t0:t1] = widen_bits(va[entry, g, :rows], kind)
            continue
        tier, slot = entry_class(entry)
        if tier == 0:
            (ka, kind), (va, _) = host.pools()
            K[t0:t1] = widen_bits(ka[slot, g, :rows], kind)
            V[t0:t1] = widen_bits(va[slot, g, :rows], kind)
            continue
        if tier >= 5:
            # 1-bit archival pages are reconstructed before attention, never
            # read by it; a row that reaches one is undefined (NaN)
            K[t0:t1] = np.nan
            V[t0:t1] = np.nan
            continue
        ta = host.tier_arrays()
        key = {1: "i8", 2: "i4", 3: "f8", 4: "i2"}[tier]
        for dst, kv in ((K, "k"), (V, "v")):
            codes = ta[f"{key}_{kv}"][slot, g, :rows]
            if key == "i4":
                codes = int4_codes(codes)
            elif key == "i2":
                codes = int2_codes(codes)
            sc = np.float64(ta[f"{key}_{kv}_scale"][slot, g])
            vals = fp8_e4m3_value(codes) if key == "f8" else codes.astype(np.float64)
            dst[t0:t1] = vals * sc
    return K, V


def block_f32(w, entry: int, g: int, kv: str, host=None) -> np.ndarray:
    """The values of one stored (page, kv head) block of K (kv = "k") or V as
    f32: a hot block (tier 0) widened exactly, a cold slot as f32(code *
    scale), one rounding of the exact product (FP8: e4m3(code) * scale), a
    1-bit slot as decode_1bit gives it.
    This is what a demotion reads when it moves a page down the cascade."""
    host = host or HostView(w)
    tier, slot = entry_class(entry)
    if tier == 0:
        (ka, kind), (va, _) = host.pools()
        return widen_bits((ka if kv == "k" else va)[slot, g], kind).astype(np.float32)
    ta = host.tier_arrays()
    if tier == 5:
        signs = ta[f"b1_{kv}"][slot, g]
        n = signs.size * 8
        vals = decode_1bit(signs, ta[f"b1_{kv}_scale"][slot, g], ta[f"b1_{kv}_out"][slot, g], n)
        return vals.reshape(w.page_tokens, w.head_dim)
    key = {1: "i8", 2: "i4", 3: "f8", 4: "i2"}[tier]
    codes = ta[f"{key}_{kv}"][slot, g]
    vals = fp8_e4m3_value(codes) if key == "f8" else (
        int4_codes(codes) if key == "i4" else int2_codes(codes) if key == "i2" else codes
    ).astype(np.float64)
    return (vals * np.float64(ta[f"{key}_{kv}_scale"][slot, g])).astype(np.float32)


def row_info(w):
    """For each query row: (sequence, visible key count)."""
    qs = w.query_start
    seqs = np.zeros(w.total_q, dtype=np.int64)
    vis = np.zeros(w.total_q, dtype=np.int64)
    for s in range(w.num_seqs):
        n_q = int(w.query_lens[s])
        ctx = int(w.context_lens[s])
        for t in range(n_q):
            seqs[qs[s] + t] = s
            vis[qs[s] + t] = max(0, ctx - n_q + t + 1)
    return seqs, vis


def reference(w, rows=None, heads=None, host=None, page_tokens=None):
    """Oracle out / lse for the chosen query rows and heads.

    Returns (out [len(rows)][len(heads)][d] f64, lse [len(rows)][len(heads)]).
    rows defaults to every query row, heads to every head.  GQA/MQA: query
    head h reads kv head h // (num_heads // num_kv_heads).

    Positional policy: with w.rope_theta > 0 each query row is rotated by its
    own position (its last visible key); with w.alibi_slopes (one per query
    head) each score gains -slope_h * (position - key).
    """
    host = host or HostView(w)
    theta = float(getattr(w, "rope_theta", 0.0) or 0.0)
    slopes = getattr(w, "alibi_slopes", None)
    rows = np.arange(w.total_q) if rows is None else np.asarray(rows)
    heads = np.arange(w.num_heads) if heads is None else np.asarray(heads)
    G = w.num_heads // w.num_kv_heads
    seqs, vis = row_info(w)
    qh = widen(w.q)  # [total_q][H][D]
    out = np.zeros((rows.size, heads.size, w.head_dim))
    lse = np.zeros((rows.size, heads.size))
    for s in sorted(set(int(seqs[r]) for r in rows)):
        sel = [i for i, r in enumerate(rows) if seqs[r] == s]
        n_keys = int(max(vis[rows[i]] for i in sel))
        for g in sorted(set(int(h) // G for h in heads)):
            K, V = logical_kv(w, s, g, n_tokens=n_keys, host=host)
            hsel = [j for j, h in enumerate(heads) if int(h) // G == g]
            qq = np.stack([qh[rows[i], heads[j]] for i in sel for j in hsel])
            vv = np.array([vis[rows[i]] for i in sel for j in hsel])
            if theta:
                qq = rope(qq, vv - 1, theta)
            sl = None
            if slopes is not None:
                sl = np.array([float(slopes[heads[j]]) for i in sel for j in hsel])
            o, l = attend(qq, K, V, vv, w.scale, page_tokens=page_tokens, slope=sl)
            k = 0
            for i in sel:
                for j in hsel:
                    out[i, j] = o[k]
                    lse[i, j] = l[k]
                    k += 1
    return out, lse
