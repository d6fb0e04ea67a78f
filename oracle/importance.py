"""Attention-importance token scores and top-k selection, fp64.

Pages: RedKnot README "About" (Elastic Sparsity: token-selective FFN driven by
attention importance); paooo.com "RedKnot的主要功能" and "RedKnot的核心优势"
(the top-k tokens by attention score take the dense FFN, the rest the identity
residual).

Definition taken (the pages give no formula): the importance of key j in
request r is the column sum of the softmax probabilities over the last
``n_last`` query rows and over every query head,
    imp_j = sum_g sum_i exp(s_{g,i,j} - lse_{g,i})   (0 where j is not visible).
Top-k orders keys by (-imp_j, j), so ties go to the lower index, and returns
the first k indices in ascending index order.
"""
import math

import numpy as np

from .attention import _mask_from_intervals, attention
from .bf16 import bf16_bits_to_f64
from .store import gather_kv


def importance(w, n_last=None, k_pool=None, v_pool=None, q=None):
    """List over requests of fp64 importance vectors [Lk]."""
    n_last = w.n_last if n_last is None else n_last
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    qb = w.q if q is None else q
    rows = []
    for r in range(w.num_requests):
        t1 = int(w.cu_q[r + 1])
        rows.extend(range(max(int(w.cu_q[r]), t1 - n_last), t1))
    _, L = attention(w, k_pool, v_pool, rows=rows, q=qb)
    out = []
    for r in range(w.num_requests):
        t0, t1 = int(w.cu_q[r]), int(w.cu_q[r + 1])
        ts = np.arange(max(t0, t1 - n_last), t1) - t0
        bq = int(w.seg_start[w.query_segment(r)])
        Lk = w.context_len(r)
        imp = np.zeros(Lk)
        for h in range(Hkv):
            K, _ = gather_kv(w, r, h, k_pool, v_pool)
            mask = _mask_from_intervals(w, r, h, bq + ts, Lk)
            for g in range(h * G, (h + 1) * G):
                Q = bf16_bits_to_f64(qb[t0 + ts, g, :])
                S = scale * (Q @ K.T)
                P = np.where(mask, np.exp(S - L[t0 + ts, g][:, None]), 0.0)
                imp += P.sum(axis=0)
        out.append(imp)
    return out


def topk_select(scores, k):
    """First k keys by (-score, index), returned in ascending index order."""
    scores = np.asarray(scores, dtype=np.float64)
    idx = np.arange(scores.shape[0])
    order = np.lexsort((idx, -scores))
    return np.sort(order[:k]).astype(np.int32)
