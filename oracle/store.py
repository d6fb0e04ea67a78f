"""Reading the paged stores back into logical token order (fp64).

The working store holds one run of 16-token pages per (segment, kv head); page
q of segment s for kv head h is physical page
``seg_pages[seg_page_indptr[s * Hkv + h] + q]`` and holds tokens
``b_s + 16 q ... b_s + 16 q + 15``. The offline cache uses the same scheme with
``cache_page_indptr``/``cache_pages`` for reused segments only. (Pages: RedKnot
README, "About": per-head page table + segmented KV store; paooo.com,
"如何使用RedKnot": BUILDSTATE pages segment KV per head into the pools.)
"""
import numpy as np

from .bf16 import bf16_bits_to_f64


def _seg_tokens(pool, indptr, pages, s, h, Hkv, n):
    run = pages[indptr[s * Hkv + h]:indptr[s * Hkv + h + 1]]
    return pool[run].reshape(-1, pool.shape[-1])[:n]


def gather_kv(w, r, h, k_pool=None, v_pool=None):
    """K, V of request r, kv head h over positions [0, Lk), as fp64 [Lk, D]."""
    k_pool = w.k_work if k_pool is None else k_pool
    v_pool = w.v_work if v_pool is None else v_pool
    Hkv = w.num_kv_heads
    ks, vs = [], []
    for s in w.segments_of(r):
        n = int(w.seg_len[s])
        ks.append(_seg_tokens(k_pool, w.seg_page_indptr, w.seg_pages, s, h, Hkv, n))
        vs.append(_seg_tokens(v_pool, w.seg_page_indptr, w.seg_pages, s, h, Hkv, n))
    return bf16_bits_to_f64(np.concatenate(ks)), bf16_bits_to_f64(np.concatenate(vs))
