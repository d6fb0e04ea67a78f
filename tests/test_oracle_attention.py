"""Pins for the oracle's attention (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

G_, L_, R_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.RETRIEVAL, workloads.DENSE


def _bits_to_f64(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _gather_by_token(w, r, h):
    """Independent of the oracle: walk every token, find its segment and page."""
    Lk = w.context_len(r)
    K = np.zeros((Lk, w.head_dim))
    V = np.zeros((Lk, w.head_dim))
    for j in range(Lk):
        for s in w.segments_of(r):
            b = int(w.seg_start[s])
            if b <= j < b + int(w.seg_len[s]):
                pid = w.seg_pages[w.seg_page_indptr[s * w.num_kv_heads + h] + (j - b) // 16]
                K[j] = _bits_to_f64(w.k_work[pid, (j - b) % 16])
                V[j] = _bits_to_f64(w.v_work[pid, (j - b) % 16])
    return K, V


def _retr_variant():
    return workloads.make_custom("tiny_retr", Hq=4, Hkv=4, D=64, theta=1e4,
                                 seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                                 orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                                 classes=[R_, L_, G_, R_, D_, L_, R_, G_], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                                 retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])


@pytest.mark.parametrize("make", [workloads.tiny, lambda: workloads.tiny(window=8), _retr_variant])
def test_vectorised_matches_brute_force(make):
    w = make()
    O1, L1 = oracle.attention(w)
    O2, L2 = oracle.attention_brute(w)
    assert np.max(np.abs(O1 - O2)) < 1e-12
    assert np.max(np.abs(L1 - L2)) < 1e-12


def _all_global(Hq=8, Hkv=4, q_len=32, seed=0):
    return workloads.make_custom("all_global", Hq=Hq, Hkv=Hkv, D=64, theta=1e4,
                                 seg_lens_per_req=[[64, 48, q_len]], orig_starts_per_req=[[7, 0, None]],
                                 classes=[G_] * Hkv, windows=[0] * Hkv, seed=seed)


@pytest.mark.parametrize("Hq,Hkv,q_len", [(8, 4, 32), (4, 4, 27), (8, 2, 5)])
def test_all_global_equals_causal_sdpa(Hq, Hkv, q_len):
    # All-global heads are ordinary causal attention with the query block
    # aligned to the bottom-right of the key range: torch SDPA in fp64 with an
    # explicit additive mask, GQA by repeating each kv head over its group.
    w = _all_global(Hq, Hkv, q_len)
    O, L = oracle.attention(w)
    Lk = w.context_len(0)
    bq = Lk - q_len
    kv = [_gather_by_token(w, 0, h) for h in range(Hkv)]
    K = torch.tensor(np.stack([k for k, _ in kv]))           # [Hkv, Lk, D]
    V = torch.tensor(np.stack([v for _, v in kv]))
    G = Hq // Hkv
    K = K.repeat_interleave(G, dim=0)
    V = V.repeat_interleave(G, dim=0)
    Q = torch.tensor(_bits_to_f64(w.q)).permute(1, 0, 2)      # [Hq, Lq, D]
    i = torch.arange(q_len)[:, None] + bq
    j = torch.arange(Lk)[None, :]
    mask = torch.where(j <= i, 0.0, float("-inf")).to(torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
    np.testing.assert_allclose(O, ref.permute(1, 0, 2).numpy(), atol=1e-12)
    S = (Q @ K.transpose(1, 2)) / math.sqrt(64) + mask
    np.testing.assert_allclose(L, torch.logsumexp(S, dim=-1).T.numpy(), atol=1e-12)


def test_wide_local_window_equals_global():
    a = workloads.make_custom("a", Hq=4, Hkv=2, D=64, theta=1e4, seg_lens_per_req=[[64, 64, 32]],
                              orig_starts_per_req=[[0, 0, None]], classes=[L_, L_], windows=[160, 10 ** 6])
    b = workloads.make_custom("b", Hq=4, Hkv=2, D=64, theta=1e4, seg_lens_per_req=[[64, 64, 32]],
                              orig_starts_per_req=[[0, 0, None]], classes=[G_, G_], windows=[0, 0])
    Oa, La = oracle.attention(a)
    Ob, Lb = oracle.attention(b)
    np.testing.assert_array_equal(Oa, Ob)
    np.testing.assert_array_equal(La, Lb)


def test_retrieval_of_every_reused_segment_equals_global():
    a = workloads.make_custom("a", Hq=2, Hkv=1, D=64, theta=1e4, seg_lens_per_req=[[48, 64, 20]],
                              orig_starts_per_req=[[0, 0, None]], classes=[R_], windows=[0], retr=[(1, 0)])
    b = workloads.make_custom("b", Hq=2, Hkv=1, D=64, theta=1e4, seg_lens_per_req=[[48, 64, 20]],
                              orig_starts_per_req=[[0, 0, None]], classes=[D_], windows=[0])
    Oa, La = oracle.attention(a)
    Ob, Lb = oracle.attention(b)
    np.testing.assert_array_equal(Oa, Ob)
    np.testing.assert_array_equal(La, Lb)


def test_constant_v_and_zero_q():
    w = _retr_variant()
    c_bits = np.uint16(0x3FC0)  # bf16 1.5
    wc = workloads.make_custom("c", Hq=4, Hkv=4, D=64, theta=1e4,
                               seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                               orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                               classes=[R_, L_, G_, R_, D_, L_, R_, G_], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                               retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])
    wc.v_work[:] = c_bits
    O, _ = oracle.attention(wc)
    np.testing.assert_allclose(O, 1.5, rtol=0, atol=1e-14)
    # Q = 0: every visible score is 0, so O is the mean of the visible V rows and LSE = ln #V
    w.q[:] = 0
    O, L = oracle.attention(w)
    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            row = int(w.cu_q[r]) + t
            for g in range(4):
                js = oracle.visible_brute(w, r, g, bq + t)
                _, V = _gather_by_token(w, r, g)
                np.testing.assert_allclose(O[row, g], V[js].mean(axis=0), atol=1e-13)
                assert abs(L[row, g] - math.log(len(js))) < 1e-13
