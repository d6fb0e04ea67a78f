"""CPU: the decode-attention oracle pinned to things other than itself.

1. The vectorised form equals the pure-Python loop form (visible keys from
   the per-index predicate, not the interval routine).
2. The decode row of a request equals the prefill oracle's last row of a
   copy of the layout whose query segment is one token longer, the extra
   token being the new one (q, k, v taken from that copy's store).
3. Closed form: with q = 0 and every value vector equal, O is that vector and
   LSE = ln(number of visible keys including the new one).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads

G_, L_, R_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.RETRIEVAL, workloads.DENSE


def _retr_mixed():
    return workloads.make_custom("retr_mixed", Hq=8, Hkv=4, D=64, theta=1e4,
                                 seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                                 orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                                 classes=[R_, L_, G_, R_, D_, L_, R_, G_], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                                 retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])


@pytest.mark.parametrize("make", [lambda: workloads.tiny(window=8), _retr_mixed])
def test_vectorised_matches_brute_force(make):
    w = make()
    q, k, v = workloads.decode_inputs(w, seed=3)
    O1, L1 = oracle.decode(w, q, k, v)
    O2, L2 = oracle.decode_brute(w, q, k, v)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)
    assert np.allclose(L1, L2, rtol=0, atol=1e-12)


def _token_bits(w, pool, r, h, pos):
    """bf16 bits of the stored token at absolute position pos of (r, h)."""
    for s in w.segments_of(r):
        b, n = int(w.seg_start[s]), int(w.seg_len[s])
        if b <= pos < b + n:
            t = pos - b
            page = w.seg_pages[w.seg_page_indptr[s * w.num_kv_heads + h] + t // w.page_size]
            return pool[page, t % w.page_size]
    raise AssertionError(pos)


@pytest.mark.parametrize("make", [lambda: workloads.tiny(window=8), _retr_mixed])
def test_decode_equals_prefill_of_one_longer_segment(make):
    w2 = make()
    R, Hkv = w2.num_requests, w2.num_kv_heads
    # w1: the same store with every query segment one token shorter
    seg_len = w2.seg_len.copy()
    last_rows = []
    keep = []
    for r in range(R):
        sq = w2.query_segment(r)
        assert seg_len[sq] >= 2
        seg_len[sq] -= 1
        t0, t1 = int(w2.cu_q[r]), int(w2.cu_q[r + 1])
        keep.extend(range(t0, t1 - 1))
        last_rows.append(t1 - 1)
    cu_q = np.concatenate([[0], np.cumsum([int(w2.cu_q[r + 1] - w2.cu_q[r]) - 1 for r in range(R)])]).astype(np.int32)
    w1 = dataclasses.replace(w2, seg_len=seg_len, cu_q=cu_q, q=w2.q[np.asarray(keep)])
    q_new = w2.q[np.asarray(last_rows)]
    k_new = np.stack([np.stack([_token_bits(w2, w2.k_work, r, h, w1.context_len(r)) for h in range(Hkv)])
                      for r in range(R)])
    v_new = np.stack([np.stack([_token_bits(w2, w2.v_work, r, h, w1.context_len(r)) for h in range(Hkv)])
                      for r in range(R)])
    O, L = oracle.decode(w1, q_new, k_new, v_new)
    O2, L2 = oracle.attention(w2, rows=last_rows)
    assert np.allclose(O, O2[last_rows], rtol=0, atol=1e-12)
    assert np.allclose(L, L2[last_rows], rtol=0, atol=1e-12)


def test_zero_q_constant_v():
    w = _retr_mixed()
    q, k, v = workloads.decode_inputs(w, seed=5)
    q[:] = 0
    one = np.uint16(0x3F80)  # 1.0 in bf16
    v[:] = one
    w = dataclasses.replace(w, v_work=np.full_like(w.v_work, one))
    O, L = oracle.decode(w, q, k, v)
    assert np.all(O == 1.0)
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.num_requests):
        for g in range(w.num_q_heads):
            n = len(oracle.visible_brute(w, r, g // G, w.context_len(r))) + 1
            assert abs(L[r, g] - np.log(n)) < 1e-12
