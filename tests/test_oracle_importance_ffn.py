"""Pins for importance, top-k and the sparse FFN oracles (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _bits_to_f64(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _small_dense(q_len=24, n_last=8, Hq=4, Hkv=2, classes=(3, 1), windows=(0, 12)):
    w = workloads.make_custom("imp", Hq=Hq, Hkv=Hkv, D=64, theta=1e4,
                              seg_lens_per_req=[[48, 32, q_len]], orig_starts_per_req=[[0, 0, None]],
                              classes=list(classes), windows=list(windows))
    w.n_last = n_last
    return w


def test_importance_sums_to_heads_times_rows():
    w = _small_dense()
    imp = oracle.importance(w)[0]
    assert abs(imp.sum() - w.num_q_heads * w.n_last) < 1e-10


def test_importance_brute_force():
    w = _small_dense(q_len=10, n_last=4)
    imp = oracle.importance(w)[0]
    Lk = w.context_len(0)
    bq = Lk - 10
    G = 2
    ref = [0.0] * Lk
    for g in range(4):
        h = g // G
        # gather K of head h token by token
        K = {}
        for s in w.segments_of(0):
            b = int(w.seg_start[s])
            for j in range(b, b + int(w.seg_len[s])):
                pid = w.seg_pages[w.seg_page_indptr[s * 2 + h] + (j - b) // 16]
                K[j] = _bits_to_f64(w.k_work[pid, (j - b) % 16]).tolist()
        for t in range(6, 10):
            q = _bits_to_f64(w.q[t, g]).tolist()
            js = oracle.visible_brute(w, 0, h, bq + t)
            s = {j: sum(a * b for a, b in zip(q, K[j])) / 8.0 for j in js}
            lse = math.log(sum(math.exp(x) for x in s.values()))
            for j in js:
                ref[j] += math.exp(s[j] - lse)
    np.testing.assert_allclose(imp, ref, rtol=1e-12, atol=1e-15)


def test_importance_zero_q_closed_form():
    # Q = 0 with dense heads: row i spreads 1/(i+1) over keys 0..i.
    w = _small_dense(classes=(3, 3), windows=(0, 0))
    w.q[:] = 0
    imp = oracle.importance(w)[0]
    Lk = w.context_len(0)
    rows = range(Lk - w.n_last, Lk)
    ref = np.array([w.num_q_heads * sum(1.0 / (i + 1) for i in rows if i >= j) for j in range(Lk)])
    np.testing.assert_allclose(imp, ref, rtol=1e-13)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for n, k, levels in [(50, 10, 4), (64, 64, 3), (33, 0, 2), (100, 37, 1000), (17, 5, 1)]:
        x = rng.integers(0, levels, n).astype(np.float64)
        ref = sorted(sorted(range(n), key=lambda j: (-x[j], j))[:k])
        assert oracle.topk_select(x, k).tolist() == ref


def test_topk_zero_q_8k_is_first_k():
    # Every key j <= 8128 gets the same importance (each of the last 64 rows sees
    # it), the largest value, so ties at the lowest indices win: 0..2047.
    w = workloads.sparse_ffn_8k(with_ffn=False, with_data=False)
    w.q[:] = 0
    imp = oracle.importance(w)[0]
    assert np.all(imp[:8129] == imp[0]) and np.all(imp[8129:] < imp[0])
    assert oracle.topk_select(imp, w.topk).tolist() == list(range(2048))


def test_ffn_dense_matches_torch():
    d = workloads.ffn_only(n_tokens=12, hidden=64, inter=96)
    n = 12
    out = oracle.sparse_ffn(d["hidden"], np.arange(n), d["w_gate"], d["w_up"], d["w_down"])
    H = torch.tensor(_bits_to_f64(d["hidden"]))
    Wg, Wu, Wd = (torch.tensor(_bits_to_f64(d[k])) for k in ("w_gate", "w_up", "w_down"))
    a = torch.nn.functional.silu(torch.nn.functional.linear(H, Wg)) * torch.nn.functional.linear(H, Wu)
    a = a.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    ref = H + torch.nn.functional.linear(a, Wd)
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-9)


def test_ffn_identity_cases():
    d = workloads.ffn_only(n_tokens=20, hidden=32, inter=48)
    idx = np.array([1, 4, 5, 19])
    zero_down = np.zeros_like(d["w_down"])
    out = oracle.sparse_ffn(d["hidden"], idx, d["w_gate"], d["w_up"], zero_down)
    np.testing.assert_array_equal(out, _bits_to_f64(d["hidden"]))
    out = oracle.sparse_ffn(d["hidden"], idx, d["w_gate"], d["w_up"], d["w_down"])
    rest = np.setdiff1d(np.arange(20), idx)
    np.testing.assert_array_equal(out[rest], _bits_to_f64(d["hidden"])[rest])
    assert np.all(out[idx] != _bits_to_f64(d["hidden"])[idx])


def test_ffn_brute_force():
    d = workloads.ffn_only(n_tokens=3, hidden=8, inter=6)
    H, Wg, Wu, Wd = (_bits_to_f64(d[k]) for k in ("hidden", "w_gate", "w_up", "w_down"))
    out = oracle.sparse_ffn(d["hidden"], [2], d["w_gate"], d["w_up"], d["w_down"])
    h = H[2]
    act = []
    for m in range(6):
        g = sum(Wg[m, c] * h[c] for c in range(8))
        u = sum(Wu[m, c] * h[c] for c in range(8))
        act.append(float(oracle.round_bf16(g / (1 + math.exp(-g)) * u)))
    ref = [h[c] + sum(Wd[c, m] * act[m] for m in range(6)) for c in range(8)]
    np.testing.assert_allclose(out[2], ref, rtol=1e-13, atol=1e-15)
