"""GPU: the whole prefill step captured in a HIP graph replays bit-identically.

The step (page tables + plan, head-aware relocation, attention, importance and
top-k) is captured once; every replay, with eager library work and host
synchronisations between replays, must reproduce the eager step's outputs
bit for bit. Every entry point takes its buffers from the caller and records
only kernel launches, so nothing in the graph depends on host state.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import Dev, layer_for

pytestmark = pytest.mark.gpu


def _step(layer, dev, w, out, lse, imp, idx, n_last, k):
    layer.build_pages(dev.seg_page_indptr, dev.seg_pages, dev.cache_page_indptr, dev.cache_pages,
                      dev.seg_orig_start)
    layer.relocate(dev.k_cache, dev.k_work, dev.v_cache, dev.v_work, w.rope_theta)
    layer.attention(dev.q, dev.k_work, dev.v_work, out=out, lse=lse)
    layer.importance_topk(dev.q, dev.k_work, lse, n_last, k, importance=imp, topk_idx=idx)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("name", ["tiny_224", "qwen3_32b_varlen"])
def test_graph_replay_matches_eager(name):
    print(f"case graph replay {name}", flush=True)
    w = workloads.make(name)
    dev = Dev(w)
    layer = layer_for(w)
    T, Hq, D = w.total_q_rows, w.num_q_heads, w.head_dim
    n_last = 16
    k = [max(1, w.context_len(r) // 5) for r in range(w.num_requests)]
    bufs = dict(out=torch.empty(T, Hq, D, dtype=torch.bfloat16, device="cuda"),
                lse=torch.empty(T, Hq, dtype=torch.float32, device="cuda"),
                imp=torch.empty(int(layer.sizes["total_keys"]), dtype=torch.float32, device="cuda"),
                idx=torch.empty(sum(k), dtype=torch.int32, device="cuda"))
    _step(layer, dev, w, n_last=n_last, k=k, **bufs)
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in bufs.items()}

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(layer, dev, w, n_last=n_last, k=k, **bufs)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        _step(layer, dev, w, n_last=n_last, k=k, **bufs)

    # eager work on separate buffers between replays
    other = {n: torch.empty_like(t) for n, t in bufs.items()}
    for rep in range(3):
        for t in bufs.values():
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in bufs:
            assert torch.equal(_bits(bufs[n]), _bits(ref[n])), f"replay {rep}: {n} differs from the eager step"
        _step(layer, dev, w, n_last=n_last, k=k, **other)
        torch.cuda.synchronize()
        assert np.array_equal(other["idx"].cpu().numpy(), ref["idx"].cpu().numpy())
