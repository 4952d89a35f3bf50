"""ctypes binding of the host residency runtime (include/atlas_residency.h).

Argument marshalling only: every decision is made by the runtime inside
libatlas.so.  Host arrays are numpy int32.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import atlas

REGEN, TIERED = 0, 1


def _arr(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class Budget:
    """A shared hot-block budget (the global budget of several layers'
    runtimes)."""

    def __init__(self, blocks: int):
        self._L = atlas.load()
        self._h = ctypes.c_void_p()
        atlas._check(self._L.atlas_residency_budget_create(int(blocks), ctypes.byref(self._h)),
                     "atlas_residency_budget_create")

    @property
    def used(self) -> int:
        v = ctypes.c_int64(0)
        atlas._check(self._L.atlas_residency_budget_used(self._h, ctypes.byref(v)),
                     "atlas_residency_budget_used")
        return v.value

    def close(self):
        if self._h:
            self._L.atlas_residency_budget_destroy(self._h)
            self._h = ctypes.c_void_p()


class Residency:
    """One runtime handle (one layer).  Fields of the config as keyword
    arguments; budget: an optional shared Budget."""

    def __init__(self, *, mode, page_tokens, max_seqs, max_pages_per_seq, hot_blocks,
                 recent_tokens=0, sink_tokens=0, admit_per_plan=0, fp8_pages=0, int8_pages=0,
                 num_fp8=0, num_int8=0, num_int4=0, int4_pages=0, num_int2=0,
                 int2_pages=0, num_1bit=0, transient_blocks=0, job_capacity=1 << 16,
                 budget: Budget | None = None):
        L = atlas.load()
        c = atlas.ResidencyConfig()
        c.struct_size = ctypes.sizeof(c)
        for k, v in dict(mode=mode, page_tokens=page_tokens, max_seqs=max_seqs,
                         max_pages_per_seq=max_pages_per_seq, hot_blocks=hot_blocks,
                         recent_tokens=recent_tokens, sink_tokens=sink_tokens,
                         admit_per_plan=admit_per_plan, fp8_pages=fp8_pages,
                         int8_pages=int8_pages, num_fp8=num_fp8, num_int8=num_int8,
                         num_int4=num_int4, int4_pages=int4_pages, num_int2=num_int2,
                         int2_pages=int2_pages, num_1bit=num_1bit,
                         transient_blocks=transient_blocks).items():
            setattr(c, k, int(v))
        c.budget = budget._h.value if budget is not None else None
        self._budget = budget  # kept alive while the runtime uses it
        self.config = c
        self._h = ctypes.c_void_p()
        atlas._check(L.atlas_residency_create(ctypes.byref(c), ctypes.byref(self._h)),
                     "atlas_residency_create")
        self._L = L
        self.max_pages = int(max_pages_per_seq)
        self._cap = int(job_capacity)
        self._bufs = [np.zeros(self._cap, dtype=np.int32) for _ in range(6)]

    def close(self):
        if self._h:
            self._L.atlas_residency_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _call(self, name, *args):
        st = getattr(self._L, name)(self._h, *args)
        if st != atlas.OK:
            raise atlas.AtlasError(st, name, self._L.atlas_last_error().decode())

    def add_seq(self, seq: int):
        self._call("atlas_residency_add_seq", int(seq))

    def remove_seq(self, seq: int):
        self._call("atlas_residency_remove_seq", int(seq))

    def append(self, seq: int, n_tokens: int):
        self._call("atlas_residency_append", int(seq), int(n_tokens))

    def _jobs(self):
        j = atlas.ResidencyJobs()
        j.struct_size = ctypes.sizeof(j)
        j.capacity = self._cap
        (j.demote_src, j.demote_dst, j.admit_page, j.admit_block, j.promote_src,
         j.promote_dst) = (_arr(b) for b in self._bufs)
        return j

    def plan(self):
        """Returns (demote_src, demote_dst, admit_page, admit_block) int32 arrays."""
        j = self._jobs()
        self._call("atlas_residency_plan", ctypes.byref(j))
        nd, na = j.n_demote, j.n_admit
        return (self._bufs[0][:nd].copy(), self._bufs[1][:nd].copy(),
                self._bufs[2][:na].copy(), self._bufs[3][:na].copy())

    def refuse_admissions(self, admit_page, admit_block, nonfinite):
        """Take back the admissions of the last plan whose nonfinite count
        (host int32, from atlas_regenerate_pages) is not 0."""
        page = np.ascontiguousarray(admit_page, dtype=np.int32)
        block = np.ascontiguousarray(admit_block, dtype=np.int32)
        counts = np.ascontiguousarray(nonfinite, dtype=np.int32)
        assert page.size == block.size == counts.size
        j = atlas.ResidencyJobs()
        j.struct_size = ctypes.sizeof(j)
        j.capacity = max(1, page.size)
        j.n_admit = page.size
        j.admit_page, j.admit_block = _arr(page), _arr(block)
        self._call("atlas_residency_refuse_admissions", ctypes.byref(j), _arr(counts))

    def tables(self, seqs):
        """Returns (page_table [n][max_pages], context_lens [n], regen_pages [n])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = seqs.size
        table = np.zeros((n, self.max_pages), dtype=np.int32)
        ctx = np.zeros(n, dtype=np.int32)
        regen = np.zeros(n, dtype=np.int32)
        self._call("atlas_residency_tables", _arr(seqs), n, _arr(table), _arr(ctx), _arr(regen))
        return table, ctx, regen

    def tables_transient(self, seqs):
        """tables() with archived pages given transient blocks; returns
        (page_table, context_lens, regen_pages, promote_src, promote_dst)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = seqs.size
        table = np.zeros((n, self.max_pages), dtype=np.int32)
        ctx = np.zeros(n, dtype=np.int32)
        regen = np.zeros(n, dtype=np.int32)
        j = self._jobs()
        self._call("atlas_residency_tables_transient", _arr(seqs), n, _arr(table), _arr(ctx),
                   _arr(regen), ctypes.byref(j))
        k = j.n_promote
        return table, ctx, regen, self._bufs[4][:k].copy(), self._bufs[5][:k].copy()

    def stats(self) -> dict:
        s = atlas.ResidencyStats()
        s.struct_size = ctypes.sizeof(s)
        self._call("atlas_residency_get_stats", ctypes.byref(s))
        return {name: getattr(s, name) for name, _ in s._fields_ if name != "struct_size"}
