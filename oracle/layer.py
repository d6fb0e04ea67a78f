"""One attention layer's EXECUTE glue around the attention, fp64 — TEST INFRASTRUCTURE.

Pages: paooo.com "如何使用RedKnot" (EXECUTE recomputes the query segment and
runs the layer over the visible state that SELECTVISIBLESTATE chose), RedKnot
README "About" (the query segment's KV is produced online and appended to the
per-head paged store next to the reused segments). The pages give no formula
for the projections; the readings below are the plain transformer layer.

Readings:
  * no normalisation layer in this glue; weights are [out_features, in_features];
  * the fused projection W_qkv stacks, in this order, the Hq query heads, the
    Hkv key heads and the Hkv value heads, D rows each;
  * row t of request r (rows cu_q[r]..cu_q[r+1]) sits at position
    p = b_q(r) + (t - cu_q[r]); Q and K are rotated at p with the rotate-half
    RoPE of ``rope.py``; V is not rotated;
  * the declared rounding points are the bf16 tensors handed on: Q, and the K
    and V written into the query segment's working pages (page t // 16, slot
    t % 16 of the segment's page run for that kv head), then the attention
    output, then the updated residual stream;
  * the output projection adds onto the residual stream:
    hidden_t <- hidden_t + W_o . attn_t, with attn_t the [Hq * D] row.
"""
import dataclasses

import numpy as np

from .attention import attention
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits
from .rope import rope


def row_positions(w):
    """Position of every query row, [T_q] (row t of request r at b_q(r) + t - cu_q[r])."""
    pos = np.empty(w.total_q_rows, dtype=np.int64)
    for r in range(w.num_requests):
        t0, t1 = int(w.cu_q[r]), int(w.cu_q[r + 1])
        pos[t0:t1] = int(w.seg_start[w.query_segment(r)]) + np.arange(t1 - t0)
    return pos


def qkv_rope(w, hidden_bits, w_qkv_bits):
    """Projection and RoPE of the query rows, before rounding.

    hidden_bits [T_q, Hd], w_qkv_bits [(Hq + 2 Hkv) D, Hd] (bf16 bits).
    Returns fp64 (Q [T_q, Hq, D], K [T_q, Hkv, D], V [T_q, Hkv, D]).
    """
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    X = bf16_bits_to_f64(hidden_bits)
    Y = X @ bf16_bits_to_f64(w_qkv_bits).T                 # [T_q, (Hq + 2 Hkv) D]
    pos = row_positions(w)
    q = Y[:, :Hq * D].reshape(-1, Hq, D)
    k = Y[:, Hq * D:(Hq + Hkv) * D].reshape(-1, Hkv, D)
    v = Y[:, (Hq + Hkv) * D:].reshape(-1, Hkv, D)
    return rope(q, pos[:, None], w.rope_theta), rope(k, pos[:, None], w.rope_theta), v


def append_query_kv(w, k_bits, v_bits, k_pool=None, v_pool=None):
    """Copies of the working pools ([pages, P, D], token-major) with the query
    rows' K/V bits ([T_q, Hkv, D]) written into their segment's pages."""
    k_pool = (w.k_work if k_pool is None else k_pool).copy()
    v_pool = (w.v_work if v_pool is None else v_pool).copy()
    P, Hkv = w.page_size, w.num_kv_heads
    for r in range(w.num_requests):
        s = w.query_segment(r)
        for tl in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            t = int(w.cu_q[r]) + tl
            for h in range(Hkv):
                page = w.seg_pages[w.seg_page_indptr[s * Hkv + h] + tl // P]
                k_pool[page, tl % P] = k_bits[t, h]
                v_pool[page, tl % P] = v_bits[t, h]
    return k_pool, v_pool


def out_proj_residual(hidden_bits, attn_bits, w_o_bits):
    """hidden + attn . W_o^T in fp64 (before the final bf16 store).
    hidden_bits [n, Hd], attn_bits [n, F], w_o_bits [Hd, F]."""
    return bf16_bits_to_f64(hidden_bits) + bf16_bits_to_f64(attn_bits) @ bf16_bits_to_f64(w_o_bits).T


def layer(w, hidden_bits, w_qkv_bits, w_o_bits):
    """The whole glue: projection + RoPE + append -> attention -> output projection.

    Returns (hidden_out fp64 [T_q, Hd] before its bf16 store, and the bf16
    bits of the intermediate tensors as a dict: q, k, v, attn)."""
    q, k, v = qkv_rope(w, hidden_bits, w_qkv_bits)
    qb, kb, vb = f64_to_bf16_bits(q), f64_to_bf16_bits(k), f64_to_bf16_bits(v)
    k_pool, v_pool = append_query_kv(w, kb, vb)
    w2 = dataclasses.replace(w, q=qb, k_work=k_pool, v_work=v_pool)
    O, _ = attention(w2)
    ab = f64_to_bf16_bits(O).reshape(O.shape[0], -1)
    return out_proj_residual(hidden_bits, ab, w_o_bits), dict(q=qb, k=kb, v=vb, attn=ab)
