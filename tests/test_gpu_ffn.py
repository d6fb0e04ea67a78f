"""GPU: token-selective SwiGLU FFN vs the fp64 oracle.

Unselected rows must be bit-identical. Selected rows: the kernel forms the
activation a_j = silu(g_j) u_j in fp32 and the oracle in fp64, and both round
it to bf16, so an activation lying next to a bf16 rounding midpoint may round
to the neighbouring value on one side only (a "flip", one bf16 step s_j). The
bound per output element i is therefore
    |out_i - ref_i| <= ulp_bf16(ref_i) + sum_{j near a midpoint} |W_down[i, j]| s_j + 1e-4,
where ulp_bf16(ref_i) covers the final bf16 store (half a step, either
binade), the sum covers every possible flip, and 1e-4 the fp32 sums of the
down projection. "Near" means within 2^-18 |a_j| + 2^-16 of the midpoint:
fp32 evaluation of the 4096-long gate/up dot products of these unit-variance
inputs moves a_j by well under 1e-5 (6.9e-6 at most in an fp32 emulation of
512 rows of the 8K case), and the window is twice that.
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


def flip_allowance(d, rows):
    """Per output element, the sum of |W_down| times the bf16 step over the
    activations that lie near a rounding midpoint."""
    pre = oracle.swiglu_activation(d["hidden"], rows, d["w_gate"], d["w_up"])
    a = oracle.round_bf16(pre)
    b = oracle.f64_to_bf16_bits(a).astype(np.int32)
    toward = np.where((b & 0x7FFF) == 0, b + 1, np.where(np.abs(pre) > np.abs(a), b + 1, b - 1))
    nbr = oracle.bf16_bits_to_f64(toward.astype(np.uint16))
    near = np.abs(pre - (a + nbr) / 2) <= 2.0 ** -18 * np.abs(pre) + 2.0 ** -16
    return (near * np.abs(nbr - a)) @ np.abs(oracle.bf16_bits_to_f64(d["w_down"])).T


def check(d, idx, got):
    sel = np.asarray(idx)
    ref = oracle.sparse_ffn(d["hidden"], sel, d["w_gate"], d["w_up"], d["w_down"])
    g = oracle.bf16_bits_to_f64(got[sel])
    err = np.abs(g - ref[sel])
    bound = oracle.ulp_bf16(ref[sel]) + flip_allowance(d, sel) + 1e-4
    print(f"FFN max err {err.max():.3e}, max err/bound {(err / bound).max():.3f}, "
          f"mean err {err.mean():.3e}", flush=True)
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


def test_full_8k_all_selected_rows():
    w = workloads.sparse_ffn_8k()
    print("case sparse_ffn_8k: FFN on 2048 selected rows", flush=True)
    d = dict(hidden=w.hidden, w_gate=w.w_gate, w_up=w.w_up, w_down=w.w_down)
    idx = np.sort(np.random.default_rng(1).choice(8192, size=2048, replace=False)).astype(np.int32)
    got = run_ffn(d, idx)
    check(d, idx, got)


def test_8k_ragged_row_count():
    """k = 1800 selected rows at 8K: the large-tile kernels' last token tile is
    partly past k (rows read as zeros, no output written for them)."""
    w = workloads.sparse_ffn_8k()
    print("case sparse_ffn_8k: FFN on 1800 selected rows", flush=True)
    d = dict(hidden=w.hidden, w_gate=w.w_gate, w_up=w.w_up, w_down=w.w_down)
    idx = np.sort(np.random.default_rng(7).choice(8192, size=1800, replace=False)).astype(np.int32)
    got = run_ffn(d, idx)
    check(d, idx, got)
