"""atlas_paged_attention_noalloc (the entry point for callers that cannot
allocate): through the C ABI it must give the bits atlas_paged_attention
gives with a caller workspace, call after call, since both run the same
kernels on the same plan; here two calls in a row, the second smaller, for
split-K decode (partials in the scratch) and matrix-core prefill (the window
ring in the scratch)."""

import numpy as np
import pytest
import torch

import synth
from kv_cache_runtime_amd import atlas

pytestmark = pytest.mark.gpu


def _pair(w, split_tokens=0):
    prob = atlas.Problem(w, split_tokens=split_tokens)
    o_ref, l_ref = prob.run()
    o_ref, l_ref = o_ref.clone(), l_ref.clone()
    prob.out.fill_(float("nan"))
    prob.lse.fill_(float("nan"))
    o, l = prob.run_noalloc()
    torch.cuda.synchronize()
    a, b = o.cpu().numpy(), l.cpu().numpy()
    ra, rb = o_ref.cpu().numpy(), l_ref.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(b.view(np.uint32), rb.view(np.uint32))
    assert np.isfinite(ra).all()
    return prob


def test_noalloc_decode_then_smaller(gpu):
    big = synth.build(dict(num_seqs=16, context_lens=("uniform", 1000, 9000), num_heads=32,
                           num_kv_heads=8, head_dim=128, page_tokens=16, kv_dtype="bf16"),
                      device=gpu, seed=31, name="noalloc-decode")
    small = synth.build(dict(num_seqs=3, context_lens=[5, 700, 2000], num_heads=8,
                             num_kv_heads=2, head_dim=128, page_tokens=64, kv_dtype="f16"),
                        device=gpu, seed=32, name="noalloc-decode-small")
    p1 = _pair(big, split_tokens=256)
    assert atlas.atlas_workspace_size(p1.args, None) > 0
    _pair(small, split_tokens=128)


def test_noalloc_prefill_then_smaller(gpu):
    big = synth.build(dict(num_seqs=2, context_lens=[3000, 5000], query_lens=[700, 1200],
                           num_heads=16, num_kv_heads=2, head_dim=128, page_tokens=32,
                           kv_dtype="bf16"), device=gpu, seed=33, name="noalloc-prefill")
    small = synth.build(dict(num_seqs=1, context_lens=[900], query_lens=[300], num_heads=8,
                             num_kv_heads=8, head_dim=128, page_tokens=16, kv_dtype="f16"),
                        device=gpu, seed=34, name="noalloc-prefill-small")
    p1 = _pair(big, split_tokens=1024)  # several windows through the ring
    assert atlas.atlas_workspace_size(p1.args, None) > 0
    _pair(small)
