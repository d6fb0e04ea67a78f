"""Decode-phase attention: one new query row per request, fp64 — TEST INFRASTRUCTURE.

Pages: arXiv abstract mirror (abstract: RedKnot serves long-context
generation); paooo.com "如何使用RedKnot" (EXECUTE attends over the visible
state that SELECTVISIBLESTATE chose for each head) and RedKnot README "About"
(per-head page tables and per-class visible windows). The pages describe the
prefill only; the decode step is the next step of the same requests.

Readings (the pages give no formula):
  * the new token of request r sits at position i = L_k(r), right after its
    query segment, and belongs to that segment;
  * its kv head h sees the keys the class rule of the prefill gives position
    i (see ``visibility``): GLOBAL and DENSE every key j <= i, LOCAL(W) the
    query segment and the W-token window ending at i, RETRIEVAL(S) the query
    segment and the two reused segments in full; the set always holds the new
    token itself;
  * the new token's key and value (RoPE already applied at i) are inputs,
    ``k_new``/``v_new``; every other key comes from the working store,
    positions [0, L_k);
  * softmax scale 1/sqrt(D), query head g reads kv head g // G, as in the
    prefill oracle.
"""
import math

import numpy as np

from .bf16 import bf16_bits_to_f64
from .store import gather_kv
from .visibility import visible_brute, visible_intervals


def decode(w, q_new, k_new, v_new, k_pool=None, v_pool=None):
    """Vectorised form. q_new [R, Hq, D], k_new/v_new [R, Hkv, D] (uint16 bf16 bits).

    Returns (O [R, Hq, D], LSE [R, Hq]) in fp64, LSE in natural log.
    """
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    R = w.num_requests
    O = np.zeros((R, Hq, D))
    L = np.zeros((R, Hq))
    for r in range(R):
        i = w.context_len(r)  # the new token's position; keys [0, i) are stored
        for h in range(Hkv):
            K, V = gather_kv(w, r, h, k_pool, v_pool)
            K = np.vstack([K, bf16_bits_to_f64(k_new[r, h])[None, :]])  # row i = the new token
            V = np.vstack([V, bf16_bits_to_f64(v_new[r, h])[None, :]])
            mask = np.zeros(i + 1, dtype=bool)
            for lo, hi in visible_intervals(w, r, h, i):
                mask[lo:hi] = True
            for g in range(h * G, (h + 1) * G):
                q = bf16_bits_to_f64(q_new[r, g])
                s = np.where(mask, scale * (K @ q), -np.inf)
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                O[r, g] = (p @ V) / l
                L[r, g] = m + math.log(l)
    return O, L


def decode_brute(w, q_new, k_new, v_new, k_pool=None, v_pool=None):
    """Pure-Python loop form of the same definition (small inputs only): the
    visible stored keys come from the per-index predicate, then the new token."""
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    R = w.num_requests
    O = np.zeros((R, Hq, D))
    L = np.zeros((R, Hq))
    for r in range(R):
        i = w.context_len(r)
        for g in range(Hq):
            h = g // G
            K, V = gather_kv(w, r, h, k_pool, v_pool)
            keys = [K[j].tolist() for j in visible_brute(w, r, h, i)] + [bf16_bits_to_f64(k_new[r, h]).tolist()]
            vals = [V[j].tolist() for j in visible_brute(w, r, h, i)] + [bf16_bits_to_f64(v_new[r, h]).tolist()]
            q = bf16_bits_to_f64(q_new[r, g]).tolist()
            s = [scale * sum(a * b for a, b in zip(q, k)) for k in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            l = sum(e)
            for d in range(D):
                O[r, g, d] = sum(e[a] * vals[a][d] for a in range(len(e))) / l
            L[r, g] = m + math.log(l)
    return O, L
