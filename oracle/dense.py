"""Masked-dense attention, the comparator of the paged head-aware layout, fp64 — TEST INFRASTRUCTURE.

Pages: paooo.com "RedKnot的核心优势" and "RedKnot的技术原理" (the fused
variable-length kernel avoids the dense layout plus mask of a general
attention call, and the pages quote that path's cost as several times
higher). The comparator is that general call: every kv head's keys laid out
densely, one boolean mask per (kv head, query row, key), softmax over the
keys the mask keeps.

Readings:
  * one request; the dense layout holds positions 0..L-1 of each kv head
    (K as [Hkv][L][D]), L rounded up to a multiple of 64 with masked padding;
  * mask[h][t][j] = 1 iff key j is visible to query row t of kv head h; the
    head-aware visible set of the prefill gives the mask that makes the two
    paths compute the same attention;
  * a row whose mask is empty has O = 0 and LSE = -inf;
  * softmax scale 1/sqrt(D); query head g reads kv head g // G.
"""
import math

import numpy as np

from .bf16 import bf16_bits_to_f64
from .store import gather_kv
from .visibility import visible_intervals


def dense_layout(w, L):
    """Dense K [Hkv, L, D] and V [Hkv, L, D] (bf16 bits) of request 0 from its working store,
    zero past the context, and the prefill visibility mask [Hkv, T_q, L] (uint8)."""
    Hkv, D = w.num_kv_heads, w.head_dim
    Lk = w.context_len(0)
    assert w.num_requests == 1 and L >= Lk
    K = np.zeros((Hkv, L, D), np.uint16)
    V = np.zeros((Hkv, L, D), np.uint16)
    mask = np.zeros((Hkv, w.total_q_rows, L), np.uint8)
    bq = int(w.seg_start[w.query_segment(0)])
    for h in range(Hkv):
        for s in w.segments_of(0):
            b, n = int(w.seg_start[s]), int(w.seg_len[s])
            run = w.seg_pages[w.seg_page_indptr[s * Hkv + h]:w.seg_page_indptr[s * Hkv + h + 1]]
            K[h, b:b + n] = w.k_work[run].reshape(-1, D)[:n]
            V[h, b:b + n] = w.v_work[run].reshape(-1, D)[:n]
        for t in range(w.total_q_rows):
            for lo, hi in visible_intervals(w, 0, h, bq + t):
                mask[h, t, lo:hi] = 1
    return K, V, mask


def masked_dense(q_bits, k_bits, v_bits, mask):
    """q [T, Hq, D], k/v [Hkv, L, D] (bf16 bits), mask [Hkv, T, L] -> (O [T, Hq, D], LSE [T, Hq]) fp64."""
    T, Hq, D = q_bits.shape
    Hkv = k_bits.shape[0]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    O = np.zeros((T, Hq, D))
    L = np.full((T, Hq), -np.inf)
    for h in range(Hkv):
        K, V = bf16_bits_to_f64(k_bits[h]), bf16_bits_to_f64(v_bits[h])
        keep = mask[h].astype(bool)
        for g in range(h * G, (h + 1) * G):
            S = np.where(keep, scale * (bf16_bits_to_f64(q_bits[:, g]) @ K.T), -np.inf)
            m = S.max(axis=1)
            live = np.isfinite(m)
            P = np.exp(S[live] - m[live, None])
            l = P.sum(axis=1)
            O[live, g] = (P @ V) / l[:, None]
            L[live, g] = m[live] + np.log(l)
    return O, L
