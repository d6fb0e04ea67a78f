"""GPU: attention-importance scores and top-k selection vs the fp64 oracle.

Importance: relative error <= 1e-4. Top-k: bit-exact against the oracle's
selection rule applied to the GPU's own importance vector, and against the
fp64 selection except for swaps among keys within 1e-4 (relative) of the
k-th value.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import build, i32

pytestmark = pytest.mark.gpu

G_, L_, R_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.RETRIEVAL, workloads.DENSE


def run(w, n_last, k):
    layer, dev = build(w)
    _, lse = layer.attention(dev.q, dev.k_work, dev.v_work)
    imp, idx = layer.importance_topk(dev.q, dev.k_work, lse, n_last, k)
    torch.cuda.synchronize()
    return imp.cpu().numpy(), (idx.cpu().numpy() if idx is not None else None)


def check(w, imp_gpu, idx_gpu, n_last, k):
    ref = oracle.importance(w, n_last=n_last)
    off = koff = 0
    for r, imp_r in enumerate(ref):
        n = len(imp_r)
        g = imp_gpu[off:off + n].astype(np.float64)
        rel = np.abs(g - imp_r) / np.maximum(imp_r, 1e-30)
        big = imp_r > 1e-6 * imp_r.max()
        print(f"[{w.name} r{r}] importance max rel err {rel[big].max():.3e}", flush=True)
        assert rel[big].max() <= 1e-4
        assert np.all(np.abs(g - imp_r)[~big] <= 1e-4 * imp_r.max())
        if idx_gpu is not None:
            kr = k[r]
            got = idx_gpu[koff:koff + kr]
            # 1. the selection rule on the GPU's own scores (fp32 values, exact)
            assert np.array_equal(got, oracle.topk_select(imp_gpu[off:off + n], kr))
            # 2. vs the fp64 selection: only near-ties at the threshold may swap
            exp = oracle.topk_select(imp_r, kr)
            if kr > 0 and not np.array_equal(got, exp):
                tau = np.sort(imp_r)[::-1][kr - 1]
                diff = np.setxor1d(got, exp)
                assert np.all(np.abs(imp_r[diff] - tau) <= 1e-4 * tau), diff
                print(f"[{w.name} r{r}] near-tie swaps: {len(diff) // 2}", flush=True)
            koff += kr
        off += n


def test_importance_topk_8k():
    w = workloads.sparse_ffn_8k(with_ffn=False)
    print("case sparse_ffn_8k: importance + top-k", flush=True)
    imp, idx = run(w, 64, [w.topk])
    check(w, imp, idx, 64, [w.topk])
    assert abs(imp.astype(np.float64).sum() - 32 * 64) < 1e-2


@pytest.mark.parametrize("name", ["mistral7b_32k", "qwen3_32b_varlen"])
def test_importance_topk_full_size(name):
    """The attention layouts at full size: importance over each request's last
    64 rows, top 25 % of its keys (the benchmark step's setting)."""
    w = workloads.make(name)
    print(f"case {name}: importance + top-k at full size", flush=True)
    k = [w.context_len(r) // 4 for r in range(w.num_requests)]
    imp, idx = run(w, 64, k)
    check(w, imp, idx, 64, k)


def test_zero_q_selects_lowest_indices():
    w = workloads.sparse_ffn_8k(with_ffn=False)
    w.q[:] = 0
    print("case sparse_ffn_8k: Q=0 exact ties", flush=True)
    imp, idx = run(w, 64, [w.topk])
    assert np.all(imp[:8129] == imp[0])
    assert np.array_equal(idx, np.arange(2048))


def test_mixed_classes_multi_request():
    w = workloads.make_custom("retr_mixed", Hq=8, Hkv=4, D=64, theta=1e4,
                              seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                              orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                              classes=[R_, L_, G_, R_, D_, L_, R_, G_], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                              retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])
    print("case retr_mixed: importance + top-k, 2 requests, n_last 20", flush=True)
    k = [50, 7]
    imp, idx = run(w, 20, k)
    check(w, imp, idx, 20, k)


def test_many_requests():
    """18 requests x 4 kv heads: more than 64 pairs, so the build kernel's
    importance item blocks take their multi-wave sums."""
    nreq = 18
    w = workloads.make_custom("many_req", Hq=8, Hkv=4, D=64, theta=1e4,
                              seg_lens_per_req=[[48 + 16 * (r % 4), 30 + 11 * (r % 5)] for r in range(nreq)],
                              orig_starts_per_req=[[3 * r, None] for r in range(nreq)],
                              classes=[(G_, L_, D_, L_)[(r + h) % 4] for r in range(nreq) for h in range(4)],
                              windows=[(0, 24, 0, 9)[(r + h) % 4] for r in range(nreq) for h in range(4)])
    print("case many_req: importance + top-k, 18 requests, n_last 16", flush=True)
    k = [(r * 7) % 40 for r in range(nreq)]
    imp, idx = run(w, 16, k)
    check(w, imp, idx, 16, k)


def test_requests_beyond_one_topk_launch():
    """70 requests x 2 kv heads: the selections take two top-k launches (64
    vectors per launch), the second with its own score and output offsets."""
    nreq = 70
    w = workloads.make_custom("many_req_70", Hq=4, Hkv=2, D=64, theta=1e4,
                              seg_lens_per_req=[[32 + 16 * (r % 3), 17 + 5 * (r % 7)] for r in range(nreq)],
                              orig_starts_per_req=[[5 * r, None] for r in range(nreq)],
                              classes=[(G_, L_, D_)[(r + h) % 3] for r in range(nreq) for h in range(2)],
                              windows=[(0, 20, 0)[(r + h) % 3] for r in range(nreq) for h in range(2)])
    print("case many_req_70: importance + top-k, 70 requests, n_last 8", flush=True)
    k = [(r * 5) % 30 for r in range(nreq)]
    imp, idx = run(w, 8, k)
    check(w, imp, idx, 8, k)


@pytest.mark.parametrize("n,k,levels", [(1000, 100, 7), (33280, 8320, 50), (4096, 4096, 3), (5, 1, 1),
                                        (70000, 1, 0), (2049, 2048, 2), (4097, 100, 0), (61440, 30000, 0),
                                        (61441, 5, 0), (70000, 35000, 1000), (36864, 36863, 1),
                                        (70000, 50000, 0), (36864, 30000, 0), (36000, 9000, 0)])
def test_topk_select_ties(n, k, levels):
    print(f"case topk n={n} k={k} levels={levels}", flush=True)
    x = workloads.uniform_f32(seed=n + k, n=n, levels=levels)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    from head_aware_paged_amd import segkv_topk_select
    segkv_topk_select(torch.from_numpy(x).cuda(), n, k, idx)
    torch.cuda.synchronize()
    ref = sorted(sorted(range(n), key=lambda j: (-float(x[j]), j))[:k])
    assert idx.cpu().numpy().tolist() == ref


def test_topk_select_signed_scores():
    """Negative scores and signed zeros: -0 and +0 tie, ties go to the lower index."""
    n, k = 9000, 4500
    print(f"case topk signed n={n} k={k}", flush=True)
    x = workloads.uniform_f32(seed=77, n=n, lo=-1.0, hi=1.0)
    x[::7] = np.float32(0.0)
    x[3::7] = np.float32(-0.0)
    x[5::11] = np.float32(-1e-30)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    from head_aware_paged_amd import segkv_topk_select
    segkv_topk_select(torch.from_numpy(x).cuda(), n, k, idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oracle.topk_select(x, k))


@pytest.mark.parametrize("n,k", [(33280, 8320), (1000, 999), (70000, 17)])
def test_topk_select_narrow_range(n, k):
    """Keys that share their leading 19 bits (1 + [0, 2^-12) in fp32: about
    2,048 distinct values, so many ties): the first radix passes see a single
    bin, the k-th key is resolved by the low bits, and ties go to the lower
    index."""
    print(f"case topk narrow range n={n} k={k}", flush=True)
    x = (np.float32(1.0) + workloads.uniform_f32(seed=n + 3 * k, n=n, lo=0.0, hi=2.0 ** -12)).astype(np.float32)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    from head_aware_paged_amd import segkv_topk_select
    segkv_topk_select(torch.from_numpy(x).cuda(), n, k, idx)
    torch.cuda.synchronize()
    ref = sorted(sorted(range(n), key=lambda j: (-float(x[j]), j))[:k])
    assert idx.cpu().numpy().tolist() == ref
