"""GPU: the elastic layer stack (every step in the library's kernels) vs its fp64 oracle.

Each deep layer must choose exactly the oracle's rows; the test first checks
that the oracle's k-th and (k+1)-th importance values are more than 1e-3
apart (relative), far beyond the 1e-4 importance bar, so the choice is
unambiguous. The final residual stream carries several bf16 rounding points
per layer (Q/K/V, attention output, residual, activation, residual), each
within one step of the oracle's, and later layers carry earlier differences
forward; the bar is relative Frobenius 1e-2 and, per element, four bf16
steps of the value (2^-5 |ref|) plus 3e-2.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits, i32, v_pages
from head_aware_paged_amd.session import ElasticStack

pytestmark = pytest.mark.gpu
G_, L_ = workloads.GLOBAL, workloads.LOCAL


def _d128(seed):
    return workloads.make_custom("stack_d128", Hq=16, Hkv=4, D=128, theta=1e6, seg_lens_per_req=[[256, 128, 77]],
                                 orig_starts_per_req=[[1000, 3, None]], classes=[G_, L_, G_, L_],
                                 windows=[0, 100, 0, 1], seed=seed)


def _same_pages(w0, w):
    """w's data laid out in w0's physical page order (the layers of a stack share one page mapping)."""
    k, v = np.empty_like(w.k_work), np.empty_like(w.v_work)
    k[w0.seg_pages] = w.k_work[w.seg_pages]
    v[w0.seg_pages] = w.v_work[w.seg_pages]
    return dataclasses.replace(w, seg_pages=w0.seg_pages, k_work=k, v_work=v)


@pytest.mark.parametrize("make,n_layers,n_shallow,hidden,inter,k,n_last,window", [
    (lambda s: workloads.tiny(seed=s), 4, 2, 256, 512, 8, 16, 16),
    (_d128, 3, 1, 512, 1024, 19, 32, 64),
])
def test_stack_vs_oracle(make, n_layers, n_shallow, hidden, inter, k, n_last, window):
    ws = [make(100 + i) for i in range(n_layers)]
    w0 = ws[0]
    ws = [w0] + [_same_pages(w0, w) for w in ws[1:]]
    print(f"case {w0.name}: elastic stack of {n_layers} ({n_shallow} shallow)", flush=True)
    h, wts = workloads.stack_inputs(w0, n_layers, hidden, inter, seed=5)
    out_ref, chosen_ref, imps = oracle.stack(list(zip(ws, wts)), h, n_shallow, window, k, n_last)
    for imp in imps[n_shallow:]:
        s = np.sort(imp)[::-1]
        assert s[k - 1] - s[k] > 1e-3 * abs(s[k - 1]), "ambiguous top-k boundary in the oracle"
    layers = []
    for w, wt in zip(ws, wts):
        d = {n: bf16(a) for n, a in wt.items()}
        d["k_pool"], d["v_pool"] = bf16(w.k_work), bf16(v_pages(w.v_work))
        layers.append(d)
    st = ElasticStack(w0.num_q_heads, w0.num_kv_heads, w0.head_dim, w0.seg_indptr, w0.seg_start, w0.seg_len,
                      w0.head_class, w0.window, w0.retr_seg, i32(w0.seg_page_indptr), i32(w0.seg_pages), layers,
                      n_shallow, window, k, n_last, w0.rope_theta)
    hid = bf16(h)
    chosen = st.forward(hid)
    torch.cuda.synchronize()
    for li in range(n_shallow, n_layers):
        assert np.array_equal(chosen[li][:k].cpu().numpy(), chosen_ref[li]), li
    got = oracle.bf16_bits_to_f64(bits(hid))
    d = np.abs(got - out_ref)
    rel = np.sqrt((d ** 2).sum() / (out_ref ** 2).sum())
    print(f"max {d.max():.3g} mean {d.mean():.3g} rel {rel:.3g}", flush=True)
    assert rel <= 1e-2, float(rel)
    assert np.all(d <= 2.0 ** -5 * np.abs(out_ref) + 3e-2), float(d.max())
