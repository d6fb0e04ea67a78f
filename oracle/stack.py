"""Layer-wise elastic policy over a synthetic stack of layers, fp64 — TEST INFRASTRUCTURE.

Pages: RedKnot README "About" (Elastic Sparsity: how much attention and FFN
work a layer keeps depends on its depth) and paooo.com "RedKnot的主要功能"
(the dense FFN runs only on the tokens with the highest attention scores).

Readings:
  * one request; every layer has its own weights and its own cached K/V of
    the reused segments, over the same segment layout;
  * a shallow layer (index < n_shallow) treats every kv head as LOCAL with
    the shallow window and runs the dense FFN on every query row;
  * a deep layer uses the layout's own class map and runs the FFN only on the
    k query rows of highest importance: importance over the last n_last query
    rows (``importance.py``) restricted to the query segment's keys (the key
    of query row t is position b_q + t), top k by (-importance, index);
  * a layer is: hidden <- bf16(hidden + W_o . attn(QKV(hidden))) (``layer.py``),
    then hidden <- bf16(FFN on the chosen rows) (``ffn.py``).
"""
import dataclasses

import numpy as np

from .bf16 import f64_to_bf16_bits
from .ffn import sparse_ffn
from .importance import importance, topk_select
from .layer import append_query_kv, layer


def shallow_layout(w, window):
    """The layout with every kv head LOCAL(window)."""
    return dataclasses.replace(w, head_class=np.full_like(w.head_class, 1), window=np.full_like(w.window, window),
                               retr_seg=np.full_like(w.retr_seg, -1))


def stack(layers, hidden_bits, n_shallow, shallow_window, k, n_last):
    """layers: list of (w, weights) with w a one-request workload holding that
    layer's pools and weights = dict(w_qkv, w_o, w_gate, w_up, w_down) of bf16 bits.
    Returns (final hidden fp64 before its last bf16 store, per-layer chosen rows,
    per-layer query-row importance (None for shallow layers))."""
    h = hidden_bits
    chosen, imps = [], []
    out = None
    for li, (w, wt) in enumerate(layers):
        lw = shallow_layout(w, shallow_window) if li < n_shallow else w
        o, mid = layer(lw, h, wt["w_qkv"], wt["w_o"])
        h = f64_to_bf16_bits(o)
        T = lw.total_q_rows
        if li < n_shallow:
            idx, imp_q = np.arange(T, dtype=np.int32), None
        else:
            kp, vp = append_query_kv(lw, mid["k"], mid["v"])
            imp = importance(dataclasses.replace(lw, q=mid["q"], k_work=kp, v_work=vp), n_last=n_last)[0]
            bq = int(lw.seg_start[lw.query_segment(0)])
            imp_q = imp[bq:bq + T]
            idx = topk_select(imp_q, k)
        out = sparse_ffn(h, idx, wt["w_gate"], wt["w_up"], wt["w_down"])
        h = f64_to_bf16_bits(out)
        chosen.append(idx)
        imps.append(imp_q)
    return out, chosen, imps
