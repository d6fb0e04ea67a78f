"""GPU: the masked-dense comparators vs their fp64 oracle.

``masked_dense_attn`` (dense [Hkv][L][D] layout, its own kernel) and
``segpaged_attn_prefill_masked`` (the tuned attention kernel reading an
explicit mask over all-global page tables).

Same bar as the SegPaged attention (max |err| 2e-2, mean 2e-3, relative
Frobenius 1e-2 per head, LSE 1e-3) on the rows whose mask is not empty;
empty rows must give O = 0 and LSE = -inf. Cases: the prefill class mask of
small layouts (so the result also equals the SegPaged attention's), random
masks with empty rows, D = 64 and 128, an odd group size (one head per
wave), a ragged number of query rows, and the 32K layer on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import dataclasses

from gpu_util import Dev, assert_attn_close, bf16, bits, layer_for
from head_aware_paged_amd import masked_dense_attn, segkv_masked_dense_workspace_size

pytestmark = pytest.mark.gpu


def run_dense(q, k, v, mask):
    T, Hq, D = q.shape
    Hkv, L = k.shape[0], k.shape[1]
    ws = torch.empty(max(16, segkv_masked_dense_workspace_size(T, Hq, Hkv, D, L)), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    vt = np.ascontiguousarray(np.swapaxes(v, 1, 2))
    masked_dense_attn(bf16(q), bf16(k), bf16(vt), torch.from_numpy(np.ascontiguousarray(mask)).cuda(),
                      1.0 / math.sqrt(D), out, lse, ws)
    torch.cuda.synchronize()
    return bits(out), lse.cpu().numpy()


def check(name, ob, lse, O, L):
    live = np.isfinite(L)
    assert np.array_equal(np.isfinite(lse), live), name
    assert np.all(ob[~live] == 0), name
    rows = np.where(live.all(axis=1))[0]
    assert_attn_close(ob, lse, O, L, rows=rows, name=name)


@pytest.mark.parametrize("make,L", [(lambda: workloads.tiny(), 256), (lambda: workloads.tiny(window=8), 256)])
def test_class_mask(make, L):
    w = make()
    print(f"case {w.name}: masked dense, class mask", flush=True)
    K, V, mask = oracle.dense_layout(w, L)
    ob, lse = run_dense(w.q, K, V, mask)
    O, Ls = oracle.masked_dense(w.q, K, V, mask)
    check(w.name, ob, lse, O, Ls)


@pytest.mark.parametrize("T,Hq,Hkv,D,L", [(40, 8, 2, 128, 320), (33, 3, 3, 64, 128), (16, 4, 4, 64, 64),
                                          (70, 16, 2, 128, 192)])
def test_random_mask(T, Hq, Hkv, D, L):
    print(f"case random mask T={T} Hq={Hq} Hkv={Hkv} D={D} L={L}", flush=True)
    rng = np.random.Generator(np.random.PCG64(T * 1000 + L))
    q = workloads._normal_bf16(rng, (T, Hq, D))
    k = workloads._normal_bf16(rng, (Hkv, L, D))
    v = workloads._normal_bf16(rng, (Hkv, L, D))
    mask = (rng.random((Hkv, T, L)) < 0.4).astype(np.uint8)
    mask[0, T // 2] = 0          # an empty row
    if L > 64:
        mask[Hkv - 1, :, L - 64:] = 0  # a key tile no row sees
    ob, lse = run_dense(q, k, v, mask)
    O, Ls = oracle.masked_dense(q, k, v, mask)
    check(f"random T={T} D={D}", ob, lse, O, Ls)


_MISTRAL_DENSE = {}


def _mistral_dense():
    """The 32K layout in dense form (L = 33280) and the oracle on every row,
    computed once for both dense-layout tests."""
    if not _MISTRAL_DENSE:
        w = workloads.mistral_32k()
        K, V, mask = oracle.dense_layout(w, 33280)
        O, Ls = oracle.masked_dense(w.q, K, V, mask)
        _MISTRAL_DENSE.update(w=w, K=K, V=V, mask=mask, O=O, L=Ls)
    return _MISTRAL_DENSE


def test_mistral_32k_all_rows():
    print("case mistral7b_32k: masked dense (class mask), all rows", flush=True)
    m = _mistral_dense()
    ob, lse = run_dense(m["w"].q, m["K"], m["V"], m["mask"])
    assert_attn_close(ob, lse, m["O"], m["L"], name="mistral7b_32k masked dense")


def run_masked_prefill(w, mask):
    """The tuned kernel in mask mode over w's store, with every kv head global (dense tables)."""
    wg = dataclasses.replace(w, head_class=np.zeros_like(w.head_class), window=np.zeros_like(w.window),
                             retr_seg=np.full_like(w.retr_seg, -1))
    dev = Dev(w, cache=False)
    layer = layer_for(wg)
    layer.build_pages(dev.seg_page_indptr, dev.seg_pages)
    out, lse = layer.attention_masked(dev.q, dev.k_work, dev.v_work,
                                      torch.from_numpy(np.ascontiguousarray(mask)).cuda())
    torch.cuda.synchronize()
    return bits(out), lse.cpu().numpy()


def _retr_mixed1():
    R_, L_, G_ = workloads.RETRIEVAL, workloads.LOCAL, workloads.GLOBAL
    return workloads.make_custom("retr_one", Hq=8, Hkv=4, D=64, theta=1e4, seg_lens_per_req=[[64, 32, 48, 64, 27]],
                                 orig_starts_per_req=[[5, 0, 100, 3, None]], classes=[R_, L_, G_, R_],
                                 windows=[0, 40, 0, 0], retr=[(2, 0), None, None, (1, 3)])


@pytest.mark.parametrize("make,L", [(lambda: workloads.tiny(window=8), 256), (_retr_mixed1, 256)])
def test_masked_prefill_class_mask(make, L):
    w = make()
    print(f"case {w.name}: masked prefill, class mask", flush=True)
    K, V, mask = oracle.dense_layout(w, L)
    ob, lse = run_masked_prefill(w, mask)
    O, Ls = oracle.masked_dense(w.q, K, V, mask)
    assert_attn_close(ob, lse, O, Ls, name=w.name + " masked prefill")


def test_masked_prefill_random_causal_mask():
    w = workloads.make_custom("g4_d128", Hq=16, Hkv=4, D=128, theta=1e6, seg_lens_per_req=[[256, 128, 77]],
                              orig_starts_per_req=[[1000, 3, None]], classes=[workloads.GLOBAL] * 4,
                              windows=[0] * 4)
    print("case g4_d128: masked prefill, random causal mask", flush=True)
    L = 512
    K, V, mask = oracle.dense_layout(w, L)
    rng = np.random.default_rng(9)
    mask &= (rng.random(mask.shape) < 0.3).astype(np.uint8)
    bq = 384
    for t in range(w.total_q_rows):
        mask[:, t, bq + t] = 1  # every row keeps its own key
    ob, lse = run_masked_prefill(w, mask)
    O, Ls = oracle.masked_dense(w.q, K, V, mask)
    assert_attn_close(ob, lse, O, Ls, name="g4_d128 masked prefill random")


def test_masked_prefill_mistral_32k_all_rows():
    print("case mistral7b_32k: masked prefill (class mask, dense tables), all rows", flush=True)
    m = _mistral_dense()
    ob, lse = run_masked_prefill(m["w"], m["mask"])
    assert_attn_close(ob, lse, m["O"], m["L"], name="mistral7b_32k masked prefill")
