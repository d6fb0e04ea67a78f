"""GPU: token-selective SwiGLU FFN vs the fp64 oracle.

Unselected rows must be bit-identical; selected rows within ulp_bf16(ref) +
1e-3 of the oracle (which rounds the activation to bf16 at the same point).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16, bits, i32
from head_aware_paged_amd.session import SparseFFN

pytestmark = pytest.mark.gpu


def run_ffn(d, idx):
    hid = bf16(d["hidden"])
    ffn = SparseFFN(bf16(d["w_gate"]), bf16(d["w_up"]), bf16(d["w_down"]), k_max=max(1, len(idx)))
    ffn(hid, i32(idx), len(idx))
    torch.cuda.synchronize()
    return bits(hid)


def check(d, idx, got, rows=None):
    sel = np.asarray(idx)
    rows = sel if rows is None else rows
    ref = oracle.sparse_ffn(d["hidden"], rows, d["w_gate"], d["w_up"], d["w_down"])
    g = oracle.bf16_bits_to_f64(got[rows])
    err = np.abs(g - ref[rows])
    bound = oracle.ulp_bf16(ref[rows]) + 1e-3
    print(f"FFN max err {err.max():.3e}, max err/bound {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)
    rest = np.setdiff1d(np.arange(d["hidden"].shape[0]), sel)
    assert np.array_equal(got[rest], d["hidden"][rest])


@pytest.mark.parametrize("n,h,inter,k", [(300, 256, 384, 100), (64, 128, 128, 64), (200, 384, 256, 1)])
def test_small(n, h, inter, k):
    print(f"case ffn n={n} hidden={h} inter={inter} k={k}", flush=True)
    d = workloads.ffn_only(seed=k, n_tokens=n, hidden=h, inter=inter)
    idx = np.sort(np.random.default_rng(k).choice(n, size=k, replace=False)).astype(np.int32)
    got = run_ffn(d, idx)
    check(d, idx, got)


def test_full_8k_selected_rows():
    w = workloads.sparse_ffn_8k()
    print("case sparse_ffn_8k: FFN on 2048 selected rows", flush=True)
    d = dict(hidden=w.hidden, w_gate=w.w_gate, w_up=w.w_up, w_down=w.w_down)
    idx = np.sort(np.random.default_rng(1).choice(8192, size=2048, replace=False)).astype(np.int32)
    got = run_ffn(d, idx)
    rows = idx[np.random.default_rng(2).choice(2048, size=12, replace=False)]
    check(d, idx, got, rows=rows)
