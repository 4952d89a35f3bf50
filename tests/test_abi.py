"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, its structs match the C layout, and host-side argument
validation rejects bad calls before anything is launched."""

import ctypes
import os
import re
import subprocess

import pytest

from kv_cache_runtime_amd import atlas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "atlas.h")


def _declared():
    """Functions declared by every header under include/."""
    inc = os.path.join(ROOT, "include")
    names = set()
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(atlas_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = atlas.load()
    declared = _declared()
    assert len(declared) >= 11
    for name in declared:
        assert hasattr(L, name), name
    assert set(atlas.EXPORTS) == set(declared)
    nm = subprocess.run(["nm", "-D", "--defined-only", atlas.LIB_PATH], capture_output=True,
                        text=True).stdout
    exported = set(re.findall(r"\bT (atlas_\w+)", nm))
    assert exported == set(declared)


def test_struct_layouts_match_c(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "atlas.h"\n'
        'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(atlas_attn_args),'
        ' sizeof(atlas_tier_pools), sizeof(atlas_regen_spec),'
        ' offsetof(atlas_attn_args, q), offsetof(atlas_attn_args, stream),'
        ' offsetof(atlas_regen_spec, regen_pages)); return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    A = atlas.AttnArgs
    assert got == [ctypes.sizeof(A), ctypes.sizeof(atlas.TierPools),
                   ctypes.sizeof(atlas.RegenSpec), A.q.offset, A.stream.offset,
                   atlas.RegenSpec.regen_pages.offset]


def test_abi_version_and_status_strings():
    assert atlas.atlas_abi_version() == 4
    assert atlas.atlas_status_string(0) == "ok"
    assert atlas.atlas_status_string(3).startswith("workspace")
    assert atlas.atlas_status_string(99) == "unknown status"


FAKE = 0x10000  # never dereferenced: validation fails or succeeds on the host


def _args(**kw):
    a = atlas.AttnArgs()
    a.struct_size = ctypes.sizeof(atlas.AttnArgs)
    vals = dict(q_dtype=atlas.BF16, kv_dtype=atlas.BF16, num_seqs=4, num_heads=32,
                num_kv_heads=8, head_dim=128, page_tokens=16, max_pages_per_seq=64,
                num_blocks=256, max_context_len=1000, max_query_len=1, total_q=4,
                split_tokens=0, scale=0.088)
    vals.update(kw)
    for k, v in vals.items():
        setattr(a, k, v)
    for f in ("q", "k_pool", "v_pool", "page_table", "context_lens", "out", "lse"):
        if f not in kw:
            setattr(a, f, FAKE)
    return a


def _ws(a, regen=None):
    n = ctypes.c_size_t(0)
    st = atlas.load().atlas_workspace_size(ctypes.byref(a),
                                           ctypes.byref(regen) if regen else None,
                                           ctypes.byref(n))
    return st, n.value


def test_workspace_size_of_a_valid_call():
    st, n = _ws(_args())
    assert st == atlas.OK
    # max_context_len 1000 over 4 rows x 8 kv heads: splits of 256 tokens,
    # ceil(1000 / 256) = 4 splits per (row, head)
    parts = 4 * 32 * 4
    assert n == ((parts * 128 * 4 + 255) // 256 * 256) + ((parts * 4 + 255) // 256 * 256)
    st, n1 = _ws(_args(split_tokens=1024))
    assert st == atlas.OK and n1 == 0  # one split: results are written directly


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=12), atlas.EINVAL),
    (dict(q_dtype=7), atlas.EINVAL),
    (dict(num_seqs=0), atlas.EINVAL),
    (dict(num_heads=30), atlas.EINVAL),
    (dict(num_heads=48, num_kv_heads=3), atlas.EUNSUPPORTED),
    (dict(head_dim=96), atlas.EUNSUPPORTED),
    (dict(head_dim=0), atlas.EINVAL),
    (dict(page_tokens=0), atlas.EINVAL),
    (dict(page_tokens=24), atlas.EUNSUPPORTED),
    (dict(max_pages_per_seq=0), atlas.EINVAL),
    (dict(max_context_len=64 * 16 + 1), atlas.EINVAL),
    (dict(max_context_len=-1), atlas.EINVAL),
    (dict(total_q=5), atlas.EINVAL),
    (dict(scale=float("nan")), atlas.EINVAL),
    (dict(scale=float("inf")), atlas.EINVAL),
    (dict(split_tokens=100), atlas.EINVAL),
    (dict(split_tokens=-64), atlas.EINVAL),
    (dict(q=None), atlas.EINVAL),
    (dict(page_table=None), atlas.EINVAL),
    (dict(lse=None), atlas.EINVAL),
])
def test_invalid_arguments_are_rejected_before_launch(kw, status):
    a = _args(**kw)
    st, _ = _ws(a)
    assert st == status, atlas.atlas_last_error()
    assert atlas.load().atlas_paged_attention(ctypes.byref(a)) == status
    assert atlas.atlas_last_error()


def test_prefill_arguments_are_checked():
    a = _args(query_start=FAKE, total_q=100, max_query_len=0)
    assert _ws(a)[0] == atlas.EINVAL
    a = _args(query_start=FAKE, total_q=100, max_query_len=101)
    assert _ws(a)[0] == atlas.EINVAL
    a = _args(query_start=FAKE, total_q=100, max_query_len=50)
    assert _ws(a)[0] == atlas.OK


def test_missing_or_small_workspace_is_reported():
    a = _args()
    st, need = _ws(a)
    assert st == atlas.OK and need > 0
    L = atlas.load()
    assert L.atlas_paged_attention(ctypes.byref(a)) == atlas.EWORKSPACE
    a.workspace = FAKE
    a.workspace_bytes = need - 1
    assert L.atlas_paged_attention(ctypes.byref(a)) == atlas.EWORKSPACE
    a.workspace = FAKE + 8
    a.workspace_bytes = need
    assert L.atlas_paged_attention(ctypes.byref(a)) == atlas.EINVAL  # misaligned


def test_tiered_and_regen_arguments_are_checked():
    L = atlas.load()
    a = _args(kv_dtype=atlas.F16)
    pools = atlas.TierPools()
    assert L.atlas_paged_attention_tiered(ctypes.byref(a), None) == atlas.EINVAL
    assert L.atlas_paged_attention_tiered(ctypes.byref(a), ctypes.byref(pools)) == atlas.EINVAL
    pools.struct_size = ctypes.sizeof(atlas.TierPools)
    pools.num_int8 = 3  # pointers missing
    assert L.atlas_paged_attention_tiered(ctypes.byref(a), ctypes.byref(pools)) == atlas.EINVAL
    a32 = _args(kv_dtype=atlas.F32, q_dtype=atlas.F32)
    pools.num_int8 = 0
    assert L.atlas_paged_attention_tiered(ctypes.byref(a32), ctypes.byref(pools)) == \
        atlas.EUNSUPPORTED
    r = atlas.make_regen(42, 0, FAKE, 10)
    assert L.atlas_paged_attention_regen(ctypes.byref(a32), ctypes.byref(r)) == \
        atlas.EUNSUPPORTED
    r.layer = 1 << 16
    assert L.atlas_paged_attention_regen(ctypes.byref(_args()), ctypes.byref(r)) == atlas.EINVAL
    r = atlas.make_regen(42, 0, FAKE, 65)
    assert L.atlas_paged_attention_regen(ctypes.byref(_args()), ctypes.byref(r)) == atlas.EINVAL


def test_fold_and_inspection_arguments_are_checked():
    L = atlas.load()
    assert L.atlas_fold_partials(FAKE, FAKE, 0, 4, 64, FAKE, FAKE, None) == atlas.EINVAL
    assert L.atlas_fold_partials(FAKE, FAKE, 2, 4, 512, FAKE, FAKE, None) == atlas.EUNSUPPORTED
    assert L.atlas_fold_partials(None, FAKE, 2, 4, 64, FAKE, FAKE, None) == atlas.EINVAL
    a = _args()
    assert L.atlas_gather_pages(ctypes.byref(a), 4, 10, FAKE, FAKE) == atlas.EINVAL
    assert L.atlas_gather_pages(ctypes.byref(a), 0, 64 * 16 + 1, FAKE, FAKE) == atlas.EINVAL
    assert L.atlas_regenerate_pages(1, 1 << 16, 8, 128, 16, atlas.BF16, 0.0, FAKE, FAKE, 1, 1,
                                    FAKE, FAKE, None, None) == atlas.EINVAL
    assert L.atlas_regenerate_pages(1, 0, 8, 128, 16, atlas.F16, 0.0, FAKE, FAKE, 1, 1,
                                    FAKE, FAKE, None, None) == atlas.EUNSUPPORTED
    assert L.atlas_regenerate_pages(1, 0, 8, 127, 16, atlas.BF16, 0.0, FAKE, FAKE, 1, 1,
                                    FAKE, FAKE, None, None) == atlas.EINVAL
    for theta in (0.5, 1.0, -2.0, float("nan"), float("inf")):
        assert L.atlas_regenerate_pages(1, 0, 8, 128, 16, atlas.BF16, theta, FAKE, FAKE, 1, 1,
                                        FAKE, FAKE, None, None) == atlas.EINVAL


def test_validate_tables_arguments_are_checked():
    L = atlas.load()
    a = _args()
    assert L.atlas_validate_tables(ctypes.byref(a), None, None, 0, None, None) == atlas.EINVAL
    pools = atlas.TierPools()
    pools.struct_size = ctypes.sizeof(atlas.TierPools)
    r = atlas.make_regen(42, 0, FAKE, 10)
    assert L.atlas_validate_tables(ctypes.byref(a), ctypes.byref(pools), ctypes.byref(r), 0,
                                   FAKE, None) == atlas.EINVAL
    bad = _args(num_heads=30)
    assert L.atlas_validate_tables(ctypes.byref(bad), None, None, 0, FAKE, None) == atlas.EINVAL
    pools.num_int8 = 2  # scales missing, values requested
    assert L.atlas_validate_tables(ctypes.byref(_args(kv_dtype=atlas.F16)), ctypes.byref(pools),
                                   None, 1, FAKE, None) == atlas.EINVAL


def test_read_probe_arguments_are_checked():
    L = atlas.load()
    assert L.atlas_read_probe(None, 16, FAKE, 4, None) == atlas.EINVAL
    assert L.atlas_read_probe(FAKE, 24, FAKE, 4, None) == atlas.EINVAL
    assert L.atlas_read_probe(FAKE + 8, 32, FAKE, 4, None) == atlas.EINVAL
    assert L.atlas_read_probe(FAKE, 32, FAKE, 0, None) == atlas.EINVAL


def test_issue_probe_arguments_are_checked():
    L = atlas.load()
    assert L.atlas_issue_probe(0, 1, 16, None, FAKE, None) == atlas.EINVAL
    assert L.atlas_issue_probe(0, 1, 16, FAKE, None, None) == atlas.EINVAL
    assert L.atlas_issue_probe(8, 1, 16, FAKE, FAKE, None) == atlas.EINVAL
    assert L.atlas_issue_probe(-1, 1, 16, FAKE, FAKE, None) == atlas.EINVAL
    assert L.atlas_issue_probe(0, 3, 16, FAKE, FAKE, None) == atlas.EINVAL
    assert L.atlas_issue_probe(0, 2, 0, FAKE, FAKE, None) == atlas.EINVAL
    assert L.atlas_issue_probe(0, 2, (1 << 20) + 1, FAKE, FAKE, None) == atlas.EINVAL


def test_write_and_demote_arguments_are_checked():
    L = atlas.load()
    a = _args()
    assert L.atlas_write_kv(ctypes.byref(a), None, FAKE) == atlas.EINVAL
    assert L.atlas_write_kv(ctypes.byref(a), FAKE + 8, FAKE) == atlas.EINVAL   # misaligned
    assert L.atlas_write_kv(ctypes.byref(_args(num_heads=30)), FAKE, FAKE) == atlas.EINVAL
    pools = atlas.TierPools()
    pools.struct_size = ctypes.sizeof(atlas.TierPools)
    f16 = _args(kv_dtype=atlas.F16)
    assert L.atlas_demote_pages(ctypes.byref(f16), None, FAKE, FAKE, 1, None) == atlas.EINVAL
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, -1,
                                None) == atlas.EINVAL
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), None, FAKE, 1,
                                None) == atlas.EINVAL
    pools.num_int4 = 2  # int4 pointers missing
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    pools.num_int4 = 0
    pools.num_fp8 = 2  # fp8 pointers missing
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    assert "fp8" in atlas.atlas_last_error()
    pools.num_fp8 = 0
    pools.num_int2 = 2  # int2 pointers missing
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    assert "int2" in atlas.atlas_last_error()
    pools.num_int2 = 0
    pools.reserved3 = 1
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    pools.reserved3 = 0
    pools.reserved2 = 1
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    pools.reserved2 = 0
    assert L.atlas_demote_pages(ctypes.byref(_args(kv_dtype=atlas.F32, q_dtype=atlas.F32)),
                                ctypes.byref(pools), FAKE, FAKE, 1, None) == atlas.EUNSUPPORTED
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), None, None, 0,
                                None) == atlas.OK   # nothing to do
    # 1-bit archive: pointers, outlier count and the 16-bit element index
    pools.num_1bit = 2
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    assert "1-bit" in atlas.atlas_last_error()
    pools.bit_k = pools.bit_v = pools.bit_k_scale = pools.bit_v_scale = FAKE
    pools.outliers_1bit = 65
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    pools.outliers_1bit = 4  # outlier pointers missing
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    pools.bit_k_out = pools.bit_v_out = FAKE
    big = _args(kv_dtype=atlas.F16, head_dim=128, page_tokens=1024, max_pages_per_seq=4)
    assert L.atlas_demote_pages(ctypes.byref(big), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EUNSUPPORTED
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), None, None, 0,
                                None) == atlas.OK
    pools.num_1bit = -1
    assert L.atlas_demote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                None) == atlas.EINVAL
    pools.num_1bit = 0


def test_promote_arguments_are_checked():
    L = atlas.load()
    pools = atlas.TierPools()
    pools.struct_size = ctypes.sizeof(atlas.TierPools)
    f16 = _args(kv_dtype=atlas.F16)
    assert L.atlas_promote_pages(ctypes.byref(f16), None, FAKE, FAKE, 1, None, None) == atlas.EINVAL
    assert L.atlas_promote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, -1,
                                 None, None) == atlas.EINVAL
    assert L.atlas_promote_pages(ctypes.byref(f16), ctypes.byref(pools), None, FAKE, 1,
                                 None, None) == atlas.EINVAL
    assert L.atlas_promote_pages(ctypes.byref(_args(kv_dtype=atlas.F16, num_blocks=0)),
                                 ctypes.byref(pools), FAKE, FAKE, 1, None, None) == atlas.EINVAL
    pools.num_int8 = 1  # int8 pointers missing
    assert L.atlas_promote_pages(ctypes.byref(f16), ctypes.byref(pools), FAKE, FAKE, 1,
                                 None, None) == atlas.EINVAL
    pools.num_int8 = 0
    assert L.atlas_promote_pages(ctypes.byref(f16), ctypes.byref(pools), None, None, 0,
                                 None, None) == atlas.OK


def test_positional_policy_arguments_are_checked():
    L = atlas.load()
    for theta in (0.5, 1.0, -1.0, float("nan"), float("inf")):
        a = _args()
        a.rope_theta = theta
        assert L.atlas_paged_attention(ctypes.byref(a)) == atlas.EINVAL, theta
        assert "rope_theta" in atlas.atlas_last_error()
    a = _args()
    a.reserved = 1
    assert L.atlas_paged_attention(ctypes.byref(a)) == atlas.EINVAL
    # a valid policy passes the argument checks
    a = _args()
    a.rope_theta = 10000.0
    a.alibi_slopes = FAKE
    assert _ws(a)[0] == atlas.OK


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    """The no-allocation entry point refuses, before any device call, a call
    whose workspace would exceed the built-in scratch (64 MiB)."""
    a = _args(num_seqs=64, total_q=64, max_context_len=32768, max_pages_per_seq=2048,
              num_blocks=65536, split_tokens=64)
    st, need = _ws(a)
    assert st == atlas.OK and need > (64 << 20)
    st = atlas.load().atlas_paged_attention_noalloc(ctypes.byref(a))
    assert st == atlas.EWORKSPACE
    assert b"scratch" in atlas.load().atlas_last_error()


def test_workspace_size_serves_an_all_cold_tiered_call():
    """A tiered decode whose pages are all cold has no hot pool (num_blocks 0,
    NULL pools); the sizing call accepts it and gives the split-K bytes the
    tiered call needs, while the plain call still refuses it."""
    a = _args(num_blocks=0, split_tokens=64)
    a.k_pool = None
    a.v_pool = None
    st, need = _ws(a)
    assert st == atlas.OK and need > 0
    b = _args(split_tokens=64)
    assert _ws(b) == (atlas.OK, need)
    assert atlas.load().atlas_paged_attention(ctypes.byref(a)) == atlas.EINVAL
    c = _args(num_blocks=0)  # pools present, no blocks: the plain call refuses too
    assert atlas.load().atlas_paged_attention(ctypes.byref(c)) == atlas.EINVAL

