"""GPU checks of the two measurement helpers bench.py relies on: the streaming
read probe (its non-temporal loads must still read every word) and the
issue-rate probe (it must run every mix, report both clocks and leave the
sink alone)."""

import numpy as np
import pytest

from kv_cache_runtime_amd import atlas

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,blocks", [(4096, 1), (1 << 20, 64), ((1 << 20) + 4, 300)])
def test_read_probe_reads_every_word(gpu, words, blocks):
    import torch
    rng = np.random.default_rng(words + blocks)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(gpu)
    out = torch.zeros(blocks, dtype=torch.int32, device=gpu)
    print(f"[read probe] {words} words, {blocks} workgroups", flush=True)
    atlas.atlas_read_probe(src, out, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("waves", [1, 2])
def test_issue_probe_runs_every_mix(gpu, waves):
    import torch
    clocks = torch.zeros(2, dtype=torch.int64, device=gpu)
    sink = torch.full((1024,), 7.0, dtype=torch.float32, device=gpu)
    for mix in range(8):
        clocks.zero_()
        print(f"[issue probe] mix {mix}, {waves} waves per SIMD", flush=True)
        atlas.atlas_issue_probe(mix, waves, 16, clocks, sink)
        torch.cuda.synchronize()
        ticks, real = (int(v) for v in clocks.cpu())
        assert ticks > 0 and real > 0, (mix, ticks, real)
        ghz = ticks / real * 0.1
        assert 0.3 < ghz < 4.0, (mix, ghz)
    assert bool((sink == 7.0).all())
