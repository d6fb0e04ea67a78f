"""GPU: page tables, head-aware move lists and visible spans, bit-exact vs the oracle."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

G_, L_, R_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.RETRIEVAL, workloads.DENSE


def small_variants():
    yield workloads.tiny()
    yield workloads.tiny(window=8)
    yield workloads.make_custom("retr_mixed", Hq=4, Hkv=4, D=64, theta=1e4,
                                seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                                orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                                classes=[R_, L_, G_, R_, D_, L_, R_, G_], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                                retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])
    yield workloads.make_custom("ragged_g8", Hq=16, Hkv=2, D=128, theta=1e6,
                                seg_lens_per_req=[[256, 128, 77], [32, 300]],
                                orig_starts_per_req=[[1000, 3, None], [17, None]],
                                classes=[L_, G_, G_, L_], windows=[100, 0, 0, 1],
                                )


def check_tables(w):
    from gpu_util import build
    print(f"case {w.name}: build_pages", flush=True)
    layer, dev = build(w)
    import torch
    torch.cuda.synchronize()
    ind, ids, pos = oracle.page_tables(w)
    assert np.array_equal(layer.page_indptr.cpu().numpy(), ind)
    n = int(ind[-1])
    assert np.array_equal(layer.page_ids.cpu().numpy()[:n], ids)
    assert np.array_equal(layer.page_pos.cpu().numpy()[:n], pos)
    src, dst, delta = oracle.move_list(w)
    assert layer.num_moves == len(src)
    if len(src):
        assert np.array_equal(layer.move_src.cpu().numpy()[:len(src)], src)
        assert np.array_equal(layer.move_dst.cpu().numpy()[:len(src)], dst)
        assert np.array_equal(layer.move_delta.cpu().numpy()[:len(src)], delta)
    return layer


@pytest.mark.parametrize("w", list(small_variants()), ids=lambda w: w.name)
def test_tables_small(w):
    layer = check_tables(w)
    spans = layer.visible_spans().cpu().numpy()
    assert np.array_equal(spans, oracle.visible_spans(w))


@pytest.mark.parametrize("name", ["mistral7b_32k", "qwen3_32b_varlen", "long_64k", "sparse_ffn_8k"])
def test_tables_full_size(name):
    w = workloads.make(name, with_data=False) if name != "sparse_ffn_8k" else workloads.sparse_ffn_8k(
        with_ffn=False, with_data=False)
    layer = check_tables(w)
    if name == "mistral7b_32k":
        spans = layer.visible_spans().cpu().numpy()
        assert np.array_equal(spans, oracle.visible_spans(w))
