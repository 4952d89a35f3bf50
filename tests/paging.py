"""Test-side page layout helpers (pure data movement, no attention arithmetic).

`relayout` takes a plain problem (synth.Paged) and returns the same logical
K/V laid out with another page size and/or another physical placement, by
copying stored bits through the page tables with numpy.
"""

import numpy as np
import torch

import synth


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def _from_bits(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(a.copy()).view(dtype)


def relayout(w, page_tokens: int, seed: int, placement: str = "permuted", spare_blocks: int = 0):
    """Same logical K/V of every sequence under a new page size and placement.

    Unused rows and blocks are filled with NaN bits.  `spare_blocks` extra
    NaN blocks are appended so block ids are not dense.
    """
    assert w.tiers is None and w.regen is None
    rng = np.random.default_rng(seed)
    S, Hkv, D, P0 = w.num_seqs, w.num_kv_heads, w.head_dim, w.page_tokens
    kb, vb = _bits(w.k_pool), _bits(w.v_pool)
    nan_bits = np.array(np.nan, dtype=np.float32).view(np.int32) if kb.dtype == np.int32 else \
        (torch.tensor(float("nan"), dtype=w.k_pool.dtype).view(torch.int16).item())
    n_pages = [-(-int(c) // page_tokens) for c in w.context_lens]
    total = sum(n_pages) + spare_blocks
    ids = rng.permutation(total) if placement == "permuted" else np.arange(total)
    shape = (total + 1, Hkv, page_tokens, D)
    k2 = np.full(shape, nan_bits, dtype=kb.dtype)
    v2 = np.full(shape, nan_bits, dtype=vb.dtype)
    table = np.full((S, max(1, max(n_pages))), total, dtype=np.int32)
    i = 0
    for s in range(S):
        ctx = int(w.context_lens[s])
        # logical rows of this sequence, all heads: [ctx][Hkv][D]
        blocks = w.page_table[s, np.arange(ctx) // P0]
        lk = kb[blocks, :, np.arange(ctx) % P0, :]
        lv = vb[blocks, :, np.arange(ctx) % P0, :]
        for p in range(n_pages[s]):
            blk = int(ids[i])
            i += 1
            table[s, p] = blk
            t0, t1 = p * page_tokens, min(ctx, (p + 1) * page_tokens)
            k2[blk, :, :t1 - t0] = lk[t0:t1].transpose(1, 0, 2)
            v2[blk, :, :t1 - t0] = lv[t0:t1].transpose(1, 0, 2)
    dev = w.q.device
    return synth.Paged(S, w.num_heads, Hkv, D, page_tokens, w.q_dtype, w.kv_dtype,
                       w.context_lens, w.query_lens, w.scale, w.q,
                       _from_bits(k2, w.k_pool.dtype).to(dev),
                       _from_bits(v2, w.v_pool.dtype).to(dev), table, name=w.name)
