"""Per-head masked softmax attention over the visible sets, fp64.

Pages: paooo.com "RedKnot的技术原理" (paged per-head storage with a fused
varlen kernel, no attn_mask is ever built) and "如何使用RedKnot" (EXECUTE:
global heads attend over the full recomputed range, local heads over the
reused paged KV); RedKnot README "About" (per-class visible windows).

The oracle *does* build explicit masks: it is the plain definition
    s_j = scale * q . k_j               for j in V(h, i)
    o   = sum_j softmax(s)_j v_j,  lse = log sum_j exp(s_j)   (natural log)
with query head g reading kv head g // G (G = Hq / Hkv, contiguous groups) and
scale = 1 / sqrt(D) (readings; the pages state neither). Rows are never empty:
a row always sees its own position.
"""
import math

import numpy as np

from .bf16 import bf16_bits_to_f64
from .store import gather_kv
from .visibility import visible_brute, visible_intervals


def _mask_from_intervals(w, r, h, positions, Lk):
    j = np.arange(Lk)
    mask = np.zeros((len(positions), Lk), dtype=bool)
    for a, i in enumerate(positions):
        for lo, hi in visible_intervals(w, r, h, int(i)):
            mask[a, lo:hi] = True
    return mask


def attention(w, k_pool=None, v_pool=None, rows=None, q=None, chunk=128, with_scores=False):
    """Vectorised oracle.

    Returns (O [T_q, Hq, D] fp64, LSE [T_q, Hq] fp64). ``rows`` optionally
    restricts the evaluation to a list of global query-row indices (other rows
    are NaN). ``q`` overrides the query tensor (uint16 bf16 bits).
    """
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    qb = w.q if q is None else q
    T = w.total_q_rows
    O = np.full((T, Hq, D), np.nan)
    L = np.full((T, Hq), np.nan)
    want = np.zeros(T, bool)
    if rows is None:
        want[:] = True
    else:
        want[np.asarray(rows, dtype=np.int64)] = True
    for r in range(w.num_requests):
        t0, t1 = int(w.cu_q[r]), int(w.cu_q[r + 1])
        sel = np.nonzero(want[t0:t1])[0]
        if len(sel) == 0:
            continue
        bq = int(w.seg_start[w.query_segment(r)])
        Lk = w.context_len(r)
        for h in range(Hkv):
            K, V = gather_kv(w, r, h, k_pool, v_pool)
            for c0 in range(0, len(sel), chunk):
                ts = sel[c0:c0 + chunk]
                mask = _mask_from_intervals(w, r, h, bq + ts, Lk)
                for g in range(h * G, (h + 1) * G):
                    Q = bf16_bits_to_f64(qb[t0 + ts, g, :])
                    S = scale * (Q @ K.T)
                    S = np.where(mask, S, -np.inf)
                    m = S.max(axis=1, keepdims=True)
                    p = np.exp(S - m)
                    l = p.sum(axis=1, keepdims=True)
                    O[t0 + ts, g, :] = (p @ V) / l
                    L[t0 + ts, g] = (m + np.log(l))[:, 0]
    return O, L


def attention_brute(w, k_pool=None, v_pool=None, rows=None):
    """Pure-Python loop form of the same definition (small inputs only)."""
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    T = w.total_q_rows
    O = np.full((T, Hq, D), np.nan)
    L = np.full((T, Hq), np.nan)
    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        kv = [gather_kv(w, r, h, k_pool, v_pool) for h in range(Hkv)]
        kv = [(K.tolist(), V.tolist()) for K, V in kv]
        for t in range(int(w.cu_q[r + 1]) - int(w.cu_q[r])):
            row = int(w.cu_q[r]) + t
            if rows is not None and row not in rows:
                continue
            i = bq + t
            for g in range(Hq):
                h = g // G
                K, V = kv[h]
                q = bf16_bits_to_f64(w.q[row, g, :]).tolist()
                js = visible_brute(w, r, h, i)
                s = [scale * sum(a * b for a, b in zip(q, K[j])) for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = sum(e)
                for d in range(D):
                    O[row, g, d] = sum(e[a] * V[j][d] for a, j in enumerate(js)) / l
                L[row, g] = m + math.log(l)
    return O, L
