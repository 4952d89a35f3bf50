"""ctypes binding of libatlas.so.

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI (include/atlas.h).  Torch tensors provide device
memory and the current HIP stream.  There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# ATLAS_LIBRARY selects another build of the same library (the host
# sanitizer build of build.py --sanitize); there is no fallback.
LIB_PATH = os.environ.get("ATLAS_LIBRARY") or os.path.join(HERE, "libatlas.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EDEVICE, ECAPACITY = 0, 1, 2, 3, 4, 5
F32, BF16, F16 = 0, 1, 2
TIER_SHIFT = 30
DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_NAME_CODE = {"f32": F32, "bf16": BF16, "f16": F16}

_p = ctypes.c_void_p
_i32 = ctypes.c_int32


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("q_dtype", _i32),
        ("kv_dtype", _i32),
        ("num_seqs", _i32),
        ("num_heads", _i32),
        ("num_kv_heads", _i32),
        ("head_dim", _i32),
        ("page_tokens", _i32),
        ("max_pages_per_seq", _i32),
        ("num_blocks", _i32),
        ("max_context_len", _i32),
        ("max_query_len", _i32),
        ("total_q", _i32),
        ("split_tokens", _i32),
        ("scale", ctypes.c_float),
        ("q", _p),
        ("k_pool", _p),
        ("v_pool", _p),
        ("page_table", _p),
        ("context_lens", _p),
        ("query_start", _p),
        ("out", _p),
        ("lse", _p),
        ("workspace", _p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", _p),
        ("profile_events", _p * 2),
        ("alibi_slopes", _p),
        ("rope_theta", ctypes.c_float),
        ("reserved", _i32),
    ]


class TierPools(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_int8", _i32),
        ("num_int4", _i32),
        ("reserved", _i32),
        ("int8_k", _p),
        ("int8_v", _p),
        ("int8_k_scale", _p),
        ("int8_v_scale", _p),
        ("int4_k", _p),
        ("int4_v", _p),
        ("int4_k_scale", _p),
        ("int4_v_scale", _p),
        ("num_fp8", _i32),
        ("reserved2", _i32),
        ("fp8_k", _p),
        ("fp8_v", _p),
        ("fp8_k_scale", _p),
        ("fp8_v_scale", _p),
        ("num_int2", _i32),
        ("reserved3", _i32),
        ("int2_k", _p),
        ("int2_v", _p),
        ("int2_k_scale", _p),
        ("int2_v_scale", _p),
        ("num_1bit", _i32),
        ("outliers_1bit", _i32),
        ("bit_k", _p),
        ("bit_v", _p),
        ("bit_k_scale", _p),
        ("bit_v_scale", _p),
        ("bit_k_out", _p),
        ("bit_v_out", _p),
    ]


class RegenSpec(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("layer", ctypes.c_uint32),
        ("seed", ctypes.c_uint64),
        ("regen_pages", _p),
        ("max_regen_pages", _i32),
        ("reserved", _i32),
    ]


EXPORTS = [
    "atlas_abi_version", "atlas_status_string", "atlas_last_error", "atlas_workspace_size",
    "atlas_paged_attention", "atlas_paged_attention_noalloc", "atlas_paged_attention_tiered",
    "atlas_paged_attention_regen",
    "atlas_fold_partials", "atlas_gather_pages", "atlas_regenerate_pages",
    "atlas_dequant_pages", "atlas_validate_tables", "atlas_read_probe", "atlas_issue_probe",
    "atlas_write_kv", "atlas_demote_pages", "atlas_promote_pages",
    "atlas_residency_create", "atlas_residency_destroy", "atlas_residency_add_seq",
    "atlas_residency_remove_seq", "atlas_residency_append", "atlas_residency_plan",
    "atlas_residency_tables", "atlas_residency_tables_transient", "atlas_residency_get_stats",
    "atlas_residency_budget_create", "atlas_residency_budget_destroy",
    "atlas_residency_budget_used", "atlas_residency_refuse_admissions",
]

_lib = None


class ResidencyConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32 if n == "struct_size" else _i32) for n in (
        "struct_size", "mode", "page_tokens", "max_seqs", "max_pages_per_seq", "hot_blocks",
        "recent_tokens", "sink_tokens", "admit_per_plan", "fp8_pages", "int8_pages",
        "num_fp8", "num_int8", "num_int4", "int4_pages", "num_int2", "int2_pages", "num_1bit",
        "transient_blocks")] + [("budget", ctypes.c_void_p)]


class ResidencyStats(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32)] + [(n, _i32) for n in (
        "sequences", "hot_used", "fp8_used", "int8_used", "int4_used", "int2_used",
        "regenerated_pages")] + [(n, ctypes.c_int64) for n in (
        "appended_tokens", "demotions", "transcodes", "admissions", "evictions",
        "capacity_failures", "archive_used", "reconstructions", "refused_admissions")]


class ResidencyJobs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("capacity", _i32), ("n_demote", _i32),
                ("n_admit", _i32), ("demote_src", _p), ("demote_dst", _p),
                ("admit_page", _p), ("admit_block", _p), ("n_promote", _i32),
                ("reserved", _i32), ("promote_src", _p), ("promote_dst", _p)]


class AtlasError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed with status {status}: {detail}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libatlas.so (built in-tree by kv_cache_runtime_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python kv_cache_runtime_amd/build.py)")
    L = ctypes.CDLL(path)
    L.atlas_abi_version.restype = ctypes.c_uint32
    L.atlas_abi_version.argtypes = []
    L.atlas_status_string.restype = ctypes.c_char_p
    L.atlas_status_string.argtypes = [_i32]
    L.atlas_last_error.restype = ctypes.c_char_p
    L.atlas_last_error.argtypes = []
    L.atlas_workspace_size.restype = _i32
    L.atlas_workspace_size.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(RegenSpec),
                                       ctypes.POINTER(ctypes.c_size_t)]
    L.atlas_paged_attention.restype = _i32
    L.atlas_paged_attention.argtypes = [ctypes.POINTER(AttnArgs)]
    L.atlas_paged_attention_noalloc.restype = _i32
    L.atlas_paged_attention_noalloc.argtypes = [ctypes.POINTER(AttnArgs)]
    L.atlas_paged_attention_tiered.restype = _i32
    L.atlas_paged_attention_tiered.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(TierPools)]
    L.atlas_paged_attention_regen.restype = _i32
    L.atlas_paged_attention_regen.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(RegenSpec)]
    L.atlas_fold_partials.restype = _i32
    L.atlas_fold_partials.argtypes = [_p, _p, _i32, _i32, _i32, _p, _p, _p]
    L.atlas_gather_pages.restype = _i32
    L.atlas_gather_pages.argtypes = [ctypes.POINTER(AttnArgs), _i32, _i32, _p, _p]
    L.atlas_regenerate_pages.restype = _i32
    L.atlas_regenerate_pages.argtypes = [ctypes.c_uint64, ctypes.c_uint32, _i32, _i32, _i32, _i32,
                                         ctypes.c_float, _p, _p, _i32, _i32, _p, _p, _p, _p]
    L.atlas_dequant_pages.restype = _i32
    L.atlas_dequant_pages.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(TierPools), _p,
                                      _i32, _p, _p]
    L.atlas_validate_tables.restype = _i32
    L.atlas_validate_tables.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(TierPools),
                                        ctypes.POINTER(RegenSpec), _i32, _p, _p]
    L.atlas_write_kv.restype = _i32
    L.atlas_write_kv.argtypes = [ctypes.POINTER(AttnArgs), _p, _p]
    L.atlas_demote_pages.restype = _i32
    L.atlas_demote_pages.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(TierPools), _p, _p,
                                     _i32, _p]
    L.atlas_promote_pages.restype = _i32
    L.atlas_promote_pages.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(TierPools), _p, _p,
                                      _i32, _p, _p]
    L.atlas_read_probe.restype = _i32
    L.atlas_read_probe.argtypes = [_p, ctypes.c_size_t, _p, _i32, _p]
    L.atlas_issue_probe.restype = _i32
    L.atlas_issue_probe.argtypes = [_i32, _i32, _i32, _p, _p, _p]
    L.atlas_residency_create.restype = _i32
    L.atlas_residency_create.argtypes = [ctypes.POINTER(ResidencyConfig), ctypes.POINTER(_p)]
    L.atlas_residency_destroy.restype = _i32
    L.atlas_residency_destroy.argtypes = [_p]
    for name in ("atlas_residency_add_seq", "atlas_residency_remove_seq"):
        getattr(L, name).restype = _i32
        getattr(L, name).argtypes = [_p, _i32]
    L.atlas_residency_append.restype = _i32
    L.atlas_residency_append.argtypes = [_p, _i32, _i32]
    L.atlas_residency_plan.restype = _i32
    L.atlas_residency_plan.argtypes = [_p, ctypes.POINTER(ResidencyJobs)]
    L.atlas_residency_tables.restype = _i32
    L.atlas_residency_tables.argtypes = [_p, _p, _i32, _p, _p, _p]
    L.atlas_residency_tables_transient.restype = _i32
    L.atlas_residency_tables_transient.argtypes = [_p, _p, _i32, _p, _p, _p,
                                                   ctypes.POINTER(ResidencyJobs)]
    L.atlas_residency_budget_create.restype = _i32
    L.atlas_residency_budget_create.argtypes = [ctypes.c_int64, ctypes.POINTER(_p)]
    L.atlas_residency_budget_destroy.restype = _i32
    L.atlas_residency_budget_destroy.argtypes = [_p]
    L.atlas_residency_budget_used.restype = _i32
    L.atlas_residency_budget_used.argtypes = [_p, ctypes.POINTER(ctypes.c_int64)]
    L.atlas_residency_refuse_admissions.restype = _i32
    L.atlas_residency_refuse_admissions.argtypes = [_p, ctypes.POINTER(ResidencyJobs), _p]
    L.atlas_residency_get_stats.restype = _i32
    L.atlas_residency_get_stats.argtypes = [_p, ctypes.POINTER(ResidencyStats)]
    if L.atlas_abi_version() != 4:
        raise RuntimeError("libatlas ABI version mismatch")
    _lib = L
    return L


def _check(status: int, what: str):
    if status != OK:
        detail = _lib.atlas_last_error().decode()
        raise AtlasError(status, what, detail)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return ctypes.c_void_p(t.data_ptr()) if t.numel() else None
    return ctypes.c_void_p(int(t))


def _stream(stream):
    if stream is None:
        if torch.cuda.is_available():
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return None
    return ctypes.c_void_p(int(stream))


def make_args(*, q, k_pool, v_pool, page_table, context_lens, num_heads, num_kv_heads,
              head_dim, page_tokens, max_context_len, scale, out, lse, query_start=None,
              max_query_len=1, total_q=None, num_blocks=None, kv_dtype=None, q_dtype=None,
              workspace=None, workspace_bytes=0, split_tokens=0, stream=None,
              alibi_slopes=None, rope_theta=0.0) -> AttnArgs:
    """Fill an atlas_attn_args from tensors (device pointers) and host ints."""
    a = AttnArgs()
    a.struct_size = ctypes.sizeof(AttnArgs)
    a.q_dtype = q_dtype if q_dtype is not None else DTYPE_CODE[q.dtype]
    a.kv_dtype = kv_dtype if kv_dtype is not None else DTYPE_CODE[k_pool.dtype]
    a.num_seqs = int(context_lens.numel())
    a.num_heads = int(num_heads)
    a.num_kv_heads = int(num_kv_heads)
    a.head_dim = int(head_dim)
    a.page_tokens = int(page_tokens)
    a.max_pages_per_seq = int(page_table.shape[-1])
    a.num_blocks = int(num_blocks if num_blocks is not None else k_pool.shape[0])
    a.max_context_len = int(max_context_len)
    a.max_query_len = int(max_query_len)
    a.total_q = int(total_q if total_q is not None else q.shape[0])
    a.split_tokens = int(split_tokens)
    a.scale = float(scale)
    a.q = _ptr(q)
    a.k_pool = _ptr(k_pool)
    a.v_pool = _ptr(v_pool)
    a.page_table = _ptr(page_table)
    a.context_lens = _ptr(context_lens)
    a.query_start = _ptr(query_start)
    a.out = _ptr(out)
    a.lse = _ptr(lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes)
    a.stream = _stream(stream)
    a.alibi_slopes = _ptr(alibi_slopes)
    a.rope_theta = float(rope_theta)
    # the struct holds raw pointers only: keep the tensors alive with it, so
    # that a temporary passed here is not recycled before the call runs
    a.tensors = [t for t in (q, k_pool, v_pool, page_table, context_lens, out, lse,
                             query_start, workspace, alibi_slopes)
                 if isinstance(t, torch.Tensor)]
    return a


def make_regen(seed, layer, regen_pages, max_regen_pages) -> RegenSpec:
    r = RegenSpec()
    r.tensors = [regen_pages] if isinstance(regen_pages, torch.Tensor) else []
    r.struct_size = ctypes.sizeof(RegenSpec)
    r.layer = int(layer)
    r.seed = int(seed) & (2**64 - 1)
    r.regen_pages = _ptr(regen_pages)
    r.max_regen_pages = int(max_regen_pages)
    return r


def make_tiers(t: dict) -> TierPools:
    p = TierPools()
    p.tensors = [v for v in t.values() if isinstance(v, torch.Tensor)]
    p.struct_size = ctypes.sizeof(TierPools)
    p.num_int8 = int(t["i8_k"].shape[0])
    p.num_int4 = int(t["i4_k"].shape[0])
    p.int8_k, p.int8_v = _ptr(t["i8_k"]), _ptr(t["i8_v"])
    p.int8_k_scale, p.int8_v_scale = _ptr(t["i8_k_scale"]), _ptr(t["i8_v_scale"])
    p.int4_k, p.int4_v = _ptr(t["i4_k"]), _ptr(t["i4_v"])
    p.int4_k_scale, p.int4_v_scale = _ptr(t["i4_k_scale"]), _ptr(t["i4_v_scale"])
    if "f8_k" in t:
        p.num_fp8 = int(t["f8_k"].shape[0])
        p.fp8_k, p.fp8_v = _ptr(t["f8_k"]), _ptr(t["f8_v"])
        p.fp8_k_scale, p.fp8_v_scale = _ptr(t["f8_k_scale"]), _ptr(t["f8_v_scale"])
    if "i2_k" in t:
        p.num_int2 = int(t["i2_k"].shape[0])
        p.int2_k, p.int2_v = _ptr(t["i2_k"]), _ptr(t["i2_v"])
        p.int2_k_scale, p.int2_v_scale = _ptr(t["i2_k_scale"]), _ptr(t["i2_v_scale"])
    if "b1_k" in t:  # 1-bit archive: signs, scales and [.., outliers] entries
        p.num_1bit = int(t["b1_k"].shape[0])
        p.outliers_1bit = int(t["b1_k_out"].shape[-1])
        p.bit_k, p.bit_v = _ptr(t["b1_k"]), _ptr(t["b1_v"])
        p.bit_k_scale, p.bit_v_scale = _ptr(t["b1_k_scale"]), _ptr(t["b1_v_scale"])
        p.bit_k_out, p.bit_v_out = _ptr(t["b1_k_out"]), _ptr(t["b1_v_out"])
    return p


# ---------------------------------------------------------------------------
# Thin wrappers with the C names
# ---------------------------------------------------------------------------

def atlas_abi_version() -> int:
    return int(load().atlas_abi_version())


def atlas_status_string(status: int) -> str:
    return load().atlas_status_string(int(status)).decode()


def atlas_last_error() -> str:
    return load().atlas_last_error().decode()


def atlas_workspace_size(args: AttnArgs, regen: RegenSpec | None = None) -> int:
    L = load()
    n = ctypes.c_size_t(0)
    _check(L.atlas_workspace_size(ctypes.byref(args),
                                  ctypes.byref(regen) if regen is not None else None,
                                  ctypes.byref(n)), "atlas_workspace_size")
    return int(n.value)


def atlas_paged_attention(args: AttnArgs):
    _check(load().atlas_paged_attention(ctypes.byref(args)), "atlas_paged_attention")


def atlas_paged_attention_noalloc(args: AttnArgs):
    """atlas_paged_attention with the library's built-in device scratch in
    place of args.workspace (for callers that cannot allocate)."""
    _check(load().atlas_paged_attention_noalloc(ctypes.byref(args)),
           "atlas_paged_attention_noalloc")


def atlas_paged_attention_tiered(args: AttnArgs, pools: TierPools):
    _check(load().atlas_paged_attention_tiered(ctypes.byref(args), ctypes.byref(pools)),
           "atlas_paged_attention_tiered")


def atlas_paged_attention_regen(args: AttnArgs, regen: RegenSpec):
    _check(load().atlas_paged_attention_regen(ctypes.byref(args), ctypes.byref(regen)),
           "atlas_paged_attention_regen")


def atlas_fold_partials(part_out, part_lse, out, lse, stream=None):
    """part_out [splits][rows][D], part_lse [splits][rows] -> out [rows][D], lse [rows]."""
    splits, rows, d = part_out.shape
    _check(load().atlas_fold_partials(_ptr(part_out), _ptr(part_lse), splits, rows, d,
                                      _ptr(out), _ptr(lse), _stream(stream)),
           "atlas_fold_partials")


def atlas_gather_pages(args: AttnArgs, seq: int, num_tokens: int, k_out, v_out):
    _check(load().atlas_gather_pages(ctypes.byref(args), int(seq), int(num_tokens),
                                     _ptr(k_out), _ptr(v_out)), "atlas_gather_pages")


def atlas_regenerate_pages(seed, layer, num_kv_heads, head_dim, page_tokens, kv_dtype,
                           logical_pages, dst_blocks, num_blocks, k_pool, v_pool, stream=None,
                           rope_theta: float = 0.0, nonfinite=None):
    """nonfinite: optional device int32 tensor [n], the non-finite values
    stored per page (-1: rejected block id)."""
    n = int(logical_pages.numel())
    _check(load().atlas_regenerate_pages(int(seed) & (2**64 - 1), int(layer), int(num_kv_heads),
                                         int(head_dim), int(page_tokens), int(kv_dtype),
                                         float(rope_theta), _ptr(logical_pages), _ptr(dst_blocks), n,
                                         int(num_blocks), _ptr(k_pool), _ptr(v_pool),
                                         _stream(stream), _ptr(nonfinite)),
           "atlas_regenerate_pages")


def atlas_dequant_pages(args: AttnArgs, pools: TierPools, entries, k_out, v_out):
    _check(load().atlas_dequant_pages(ctypes.byref(args), ctypes.byref(pools), _ptr(entries),
                                      int(entries.numel()), _ptr(k_out), _ptr(v_out)),
           "atlas_dequant_pages")


def atlas_validate_tables(args: AttnArgs, pools=None, regen=None, check_values: bool = False,
                          report_dev=None):
    """Counts of invalid entries / lengths / non-finite values / scales (a
    list of 4 ints); waits for the stream.  report_dev: device uint32-sized
    buffer of 4 elements (allocated here if None)."""
    if report_dev is None:
        report_dev = torch.zeros(4, dtype=torch.int32, device="cuda")
    host = (ctypes.c_uint32 * 4)()
    _check(load().atlas_validate_tables(ctypes.byref(args),
                                        ctypes.byref(pools) if pools is not None else None,
                                        ctypes.byref(regen) if regen is not None else None,
                                        1 if check_values else 0, _ptr(report_dev), host),
           "atlas_validate_tables")
    return [int(x) for x in host]


def atlas_write_kv(args: AttnArgs, k_new, v_new):
    """Write each query row's K/V rows into the page of its own position."""
    _check(load().atlas_write_kv(ctypes.byref(args), _ptr(k_new), _ptr(v_new)), "atlas_write_kv")


def atlas_demote_pages(args: AttnArgs, pools: TierPools, src_slots, dst_entries, rejected=None):
    """Encode hot blocks src_slots[i] into cold entries dst_entries[i]."""
    _check(load().atlas_demote_pages(ctypes.byref(args), ctypes.byref(pools), _ptr(src_slots),
                                     _ptr(dst_entries), int(src_slots.numel()), _ptr(rejected)),
           "atlas_demote_pages")


def atlas_promote_pages(args: AttnArgs, pools: TierPools, src_entries, dst_blocks,
                        rejected=None, nonfinite=None):
    """Reconstruct the pages of src_entries[i] into hot blocks dst_blocks[i]."""
    _check(load().atlas_promote_pages(ctypes.byref(args), ctypes.byref(pools), _ptr(src_entries),
                                      _ptr(dst_blocks), int(src_entries.numel()), _ptr(rejected),
                                      _ptr(nonfinite)),
           "atlas_promote_pages")


def atlas_read_probe(src, out, blocks: int, stream=None):
    """Streaming read of the whole tensor `src` (measurement helper)."""
    _check(load().atlas_read_probe(_ptr(src), int(src.numel() * src.element_size()), _ptr(out),
                                   int(blocks), _stream(stream)), "atlas_read_probe")


def atlas_issue_probe(mix: int, waves_per_simd: int, iters: int, clocks, sink, stream=None):
    """One launch of the issue-rate probe (measurement helper); clocks: 2
    int64 on the device, sink: 1024 float32 on the device."""
    _check(load().atlas_issue_probe(int(mix), int(waves_per_simd), int(iters), _ptr(clocks),
                                    _ptr(sink), _stream(stream)), "atlas_issue_probe")


# ---------------------------------------------------------------------------
# Convenience: run a synth.Paged problem end to end
# ---------------------------------------------------------------------------

class Problem:
    """Device-side tensors and argument structs for one paged problem.

    Allocates the outputs and the workspace once (torch), so repeated calls
    time only the library.
    """

    def __init__(self, w, split_tokens: int = 0, stream=None):
        dev = w.q.device
        self.w = w
        self.table = torch.from_numpy(w.page_table).to(dev)
        self.ctx = torch.from_numpy(w.context_lens).to(dev)
        self.qstart = None if w.is_decode else torch.from_numpy(w.query_start).to(dev)
        self.out = torch.empty((w.total_q, w.num_heads, w.head_dim), device=dev,
                               dtype=torch.float32)
        self.lse = torch.empty((w.total_q, w.num_heads), device=dev, dtype=torch.float32)
        self.alibi = None
        if getattr(w, "alibi_slopes", None) is not None:
            self.alibi = torch.from_numpy(np.ascontiguousarray(w.alibi_slopes,
                                                               dtype=np.float32)).to(dev)
        self.kind = "plain"
        self.tiers = None
        self.regen = None
        if w.tiers is not None:
            self.kind = "tiered"
            self.tiers = make_tiers(w.tiers)
        elif w.regen is not None:
            self.kind = "regen"
            self.regen_pages = torch.from_numpy(w.regen["regen_pages"]).to(dev)
            self.regen = make_regen(w.regen["seed"], w.regen["layer"], self.regen_pages,
                                    int(w.regen["regen_pages"].max()))
        self.args = make_args(
            q=w.q, k_pool=w.k_pool, v_pool=w.v_pool, page_table=self.table,
            context_lens=self.ctx, num_heads=w.num_heads, num_kv_heads=w.num_kv_heads,
            head_dim=w.head_dim, page_tokens=w.page_tokens, max_context_len=w.max_context_len,
            scale=w.scale, out=self.out, lse=self.lse, query_start=self.qstart,
            max_query_len=w.max_query_len, total_q=w.total_q,
            kv_dtype=_NAME_CODE[w.kv_dtype], q_dtype=_NAME_CODE[w.q_dtype],
            split_tokens=split_tokens, stream=stream, alibi_slopes=self.alibi,
            rope_theta=getattr(w, "rope_theta", 0.0))
        ws = atlas_workspace_size(self.args, self.regen)
        self.workspace = torch.empty(max(ws, 1), device=dev, dtype=torch.uint8)
        self.args.workspace = _ptr(self.workspace)
        self.args.workspace_bytes = ws

    def fill_resident_from_regenerator(self):
        """Write the regenerator's values into the resident pool pages of a
        regenerated problem (CFR-Atlas: admitting regenerated pages into the
        resident cache)."""
        w = self.w
        logical, blocks = [], []
        for s in range(w.num_seqs):
            for p in range(int(w.regen["regen_pages"][s]), w.pages_of(s)):
                logical.append(p)
                blocks.append(int(w.page_table[s, p]))
        if not logical:
            return
        dev = w.q.device
        lp = torch.tensor(logical, dtype=torch.int32, device=dev)
        bl = torch.tensor(blocks, dtype=torch.int32, device=dev)
        atlas_regenerate_pages(w.regen["seed"], w.regen["layer"], w.num_kv_heads, w.head_dim,
                               w.page_tokens, _NAME_CODE[w.kv_dtype], lp, bl, w.num_blocks,
                               w.k_pool, w.v_pool, rope_theta=getattr(w, "rope_theta", 0.0))

    def validate(self, check_values: bool = False):
        return atlas_validate_tables(self.args, self.tiers, self.regen, check_values)

    def run_noalloc(self):
        """The same call through atlas_paged_attention_noalloc (plain pages
        only): the library's built-in scratch instead of self.workspace."""
        assert self.kind == "plain"
        atlas_paged_attention_noalloc(self.args)
        return self.out, self.lse

    def run(self):
        if self.kind == "tiered":
            atlas_paged_attention_tiered(self.args, self.tiers)
        elif self.kind == "regen":
            atlas_paged_attention_regen(self.args, self.regen)
        else:
            atlas_paged_attention(self.args)
        return self.out, self.lse
