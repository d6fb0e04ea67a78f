"""Buffer-owning convenience wrapper around the segkv C ABI.

A ``SegPagedLayer`` holds one layer's layout (segments + head-class map), the
device buffers the C calls write (page tables, move list, attention plan,
split-KV workspace) and forwards to the binding. Buffers are torch tensors:
PyTorch supplies device memory and streams; every computation happens in
libsegkv's HIP kernels. The four calls mirror the adapter interface the RedKnot
pages describe (paooo.com, "如何使用RedKnot"): ``build_pages`` is
SELECTVISIBLESTATE, ``relocate`` the BUILDSTATE relocation, ``attention`` and
``importance_topk``/``sparse_ffn`` the EXECUTE steps.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import (HostMeta, dims, rope_relocate, segkv_build_pages, segkv_decode_workspace_size,
               segkv_out_proj_residual, segkv_plan_sizes, segkv_qkv_rope_append, segkv_qkv_workspace_size,
               segkv_topk_select, segkv_visible_spans, segpaged_attn_decode, segpaged_attn_prefill, segpaged_attn_prefill_masked,
               sparse_ffn_swiglu,
               sparse_ffn_workspace_size, token_importance_topk)


class SegPagedLayer:
    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, seg_indptr, seg_start, seg_len,
                 head_class, window, retr_seg, page_size: int = 16, device: str = "cuda"):
        self.meta = HostMeta(seg_indptr, seg_start, seg_len, head_class, window, retr_seg)
        R = len(self.meta.seg_indptr) - 1
        self.dims = dims(R, num_q_heads, num_kv_heads, head_dim, page_size, len(self.meta.seg_start))
        self.sizes = segkv_plan_sizes(self.dims, self.meta)
        self.device = device
        self.dmeta = self.meta.to_device(device)
        q_len = [int(self.meta.seg_len[self.meta.seg_indptr[r + 1] - 1]) for r in range(R)]
        self.cu_q_host = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
        self.cu_q = torch.from_numpy(self.cu_q_host).to(device)
        i32 = dict(dtype=torch.int32, device=device)
        n_tab = max(1, self.sizes["table_entries"])
        self.page_indptr = torch.zeros(R * num_kv_heads + 1, **i32)
        self.page_ids = torch.zeros(n_tab, **i32)
        self.page_pos = torch.zeros(n_tab, **i32)
        n_mv = max(1, self.sizes["move_entries"])
        self.move_src = torch.zeros(n_mv, **i32)
        self.move_dst = torch.zeros(n_mv, **i32)
        self.move_delta = torch.zeros(n_mv, **i32)
        self.plan = torch.zeros(self.sizes["plan_bytes"], dtype=torch.uint8, device=device)
        ws = self.sizes["attn_workspace_bytes"]
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device) if ws > 0 else None
        self.imp_workspace = torch.empty(max(self.sizes["importance_workspace_bytes"], 16), dtype=torch.uint8,
                                         device=device)
        self.scale = 1.0 / math.sqrt(head_dim)

    @property
    def num_moves(self) -> int:
        return int(self.sizes["move_entries"])

    def build_pages(self, seg_page_indptr, seg_pages, cache_page_indptr=None, cache_pages=None,
                    seg_orig_start=None, stream=None):
        with_moves = cache_pages is not None
        segkv_build_pages(self.dims, self.meta, self.dmeta, self.cu_q, seg_page_indptr, seg_pages,
                          self.page_indptr, self.page_ids, self.page_pos, self.plan,
                          cache_page_indptr, cache_pages, seg_orig_start,
                          self.move_src if with_moves else None, self.move_dst if with_moves else None,
                          self.move_delta if with_moves else None, stream=stream)

    def visible_spans(self, stream=None):
        spans = torch.empty(int(self.sizes["total_q_rows"]), self.dims.num_kv_heads, 3, 2, dtype=torch.int32,
                            device=self.device)
        segkv_visible_spans(self.dims, self.meta, self.dmeta, self.cu_q, spans, stream=stream)
        return spans

    def relocate(self, k_cache, k_work, v_cache, v_work, rope_theta: float, stream=None):
        """Move the head-aware move list's pages from the cache pool to the working pool."""
        rope_relocate(k_cache, k_work, v_cache, v_work, self.move_src, self.move_dst, self.move_delta,
                      self.num_moves, self.dims.page_size, self.dims.head_dim, rope_theta, stream=stream)

    def attention(self, q, k_pool, v_pool, out=None, lse=None, want_lse=True, stream=None):
        """k_pool: [pages][page_size][head_dim] bf16; v_pool: [pages][head_dim][page_size] bf16 (d-major)."""
        T, Hq = int(self.sizes["total_q_rows"]), self.dims.num_q_heads
        if out is None:
            out = torch.empty(T, Hq, self.dims.head_dim, dtype=torch.bfloat16, device=self.device)
        if lse is None and want_lse:
            lse = torch.empty(T, Hq, dtype=torch.float32, device=self.device)
        segpaged_attn_prefill(self.dims, self.meta, q, k_pool, v_pool, self.page_ids, self.page_pos, self.plan,
                              self.scale, out, lse, self.workspace, stream=stream)
        return out, lse

    def attention_masked(self, q, k_pool, v_pool, mask, out=None, lse=None, want_lse=True, stream=None):
        """Attention with visibility from an explicit mask [Hkv][T_q][L] (uint8) over this
        layer's page tables (all-global tables: the dense layout)."""
        T, Hq, D = int(self.cu_q_host[-1]), self.dims.num_q_heads, self.dims.head_dim
        if out is None:
            out = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=self.device)
        if lse is None and want_lse:
            lse = torch.empty(T, Hq, dtype=torch.float32, device=self.device)
        segpaged_attn_prefill_masked(self.dims, self.meta, q, k_pool, v_pool, self.page_ids, self.page_pos,
                                     self.plan, self.scale, mask, out, lse, self.workspace, stream=stream)
        return out, lse

    def decode(self, q_new, k_new, v_new, k_pool, v_pool, out=None, lse=None, want_lse=True, stream=None):
        """One new query row per request at position L_k(r) over the same page tables.
        q_new: [R][Hq][D]; k_new, v_new: [R][Hkv][D] bf16."""
        R, Hq, D = self.dims.num_requests, self.dims.num_q_heads, self.dims.head_dim
        if out is None:
            out = torch.empty(R, Hq, D, dtype=torch.bfloat16, device=self.device)
        if lse is None and want_lse:
            lse = torch.empty(R, Hq, dtype=torch.float32, device=self.device)
        if not hasattr(self, "dec_workspace"):
            nbytes = segkv_decode_workspace_size(self.dims, self.meta)
            self.dec_workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        segpaged_attn_decode(self.dims, self.meta, self.dmeta, q_new, k_new, v_new, k_pool, v_pool,
                             self.page_indptr, self.page_ids, self.page_pos, self.scale, out, lse,
                             self.dec_workspace, stream=stream)
        return out, lse

    def qkv_rope_append(self, hidden, w_qkv, rope_theta: float, seg_page_indptr, seg_pages, k_pool, v_pool,
                        q_out=None, stream=None):
        """Query rows' fused QKV projection + RoPE; K/V written into the query
        segment's working pages. hidden: [T_q][hidden]; returns Q [T_q][Hq][D]."""
        Hq, D = self.dims.num_q_heads, self.dims.head_dim
        if q_out is None:
            q_out = torch.empty(int(self.cu_q_host[-1]), Hq, D, dtype=torch.bfloat16, device=self.device)
        if not hasattr(self, "qkv_workspace"):
            nbytes = segkv_qkv_workspace_size(self.dims, self.meta)
            self.qkv_workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        segkv_qkv_rope_append(self.dims, self.meta, self.dmeta, self.cu_q, seg_page_indptr, seg_pages, hidden,
                              w_qkv, rope_theta, q_out, k_pool, v_pool, self.qkv_workspace, stream=stream)
        return q_out

    @staticmethod
    def out_proj_residual(attn, w_o, hidden, stream=None):
        """hidden += W_o . attn per row, in place (attn: [T_q][Hq][D] or [T_q][Hq*D])."""
        segkv_out_proj_residual(attn, w_o, hidden, stream=stream)
        return hidden

    def importance_topk(self, q, k_pool, lse, n_last: int, k: Optional[Sequence[int]], importance=None,
                        topk_idx=None, stream=None):
        if importance is None:
            importance = torch.empty(int(self.sizes["total_keys"]), dtype=torch.float32, device=self.device)
        if k is not None and topk_idx is None:
            topk_idx = torch.empty(max(1, int(sum(k))), dtype=torch.int32, device=self.device)
        token_importance_topk(self.dims, self.meta, self.dmeta, self.cu_q, q, k_pool, self.page_indptr,
                              self.page_ids, self.page_pos, self.plan, lse, self.scale, n_last, k, importance,
                              topk_idx if k is not None else None, workspace=self.imp_workspace, stream=stream)
        return importance, topk_idx


class SparseFFN:
    """Sparse SwiGLU FFN with its activation workspace sized for at most k_max rows."""

    def __init__(self, w_gate, w_up, w_down, k_max: int):
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        nbytes = sparse_ffn_workspace_size(k_max, w_gate.shape[0])
        self.workspace = torch.empty(max(16, nbytes), dtype=torch.uint8, device=w_gate.device)

    def __call__(self, hidden, idx, k: int, stream=None):
        sparse_ffn_swiglu(hidden, idx, k, self.w_gate, self.w_up, self.w_down, self.workspace, stream=stream)
        return hidden


class ElasticStack:
    """A stack of attention + FFN layers over one segment layout (one request)
    under the layer-wise elastic policy (RedKnot README "About": Elastic
    Sparsity): layers below ``n_shallow`` treat every kv head as LOCAL(window)
    and run the dense FFN on every query row; deeper layers use the layout's
    class map and run the FFN on the ``k`` query rows of highest attention
    importance over the last ``n_last`` rows. Each layer brings its weights
    and its own working pools: dict(w_qkv, w_o, w_gate, w_up, w_down, k_pool,
    v_pool) of device tensors; every layer's pools use the one page mapping
    (seg_page_indptr, seg_pages)."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, seg_indptr, seg_start, seg_len,
                 head_class, window, retr_seg, seg_page_indptr, seg_pages, layers, n_shallow: int,
                 shallow_window: int, k: int, n_last: int, rope_theta: float, device: str = "cuda"):
        if len(seg_indptr) != 2:
            raise ValueError("the elastic stack runs one request")
        hc = np.asarray(head_class)
        self.deep = SegPagedLayer(num_q_heads, num_kv_heads, head_dim, seg_indptr, seg_start, seg_len, hc, window,
                                  retr_seg, device=device)
        self.shallow = SegPagedLayer(num_q_heads, num_kv_heads, head_dim, seg_indptr, seg_start, seg_len,
                                     np.full_like(hc, 1), np.full(len(hc), shallow_window, np.int32),
                                     np.full(len(hc) * 2, -1, np.int32), device=device)
        self.spi, self.spg = seg_page_indptr, seg_pages
        for lay in (self.deep, self.shallow):
            lay.build_pages(seg_page_indptr, seg_pages)
        self.layers, self.n_shallow, self.k, self.n_last, self.theta = layers, n_shallow, k, n_last, rope_theta
        self.T = int(self.deep.cu_q_host[-1])
        self.bq = int(np.asarray(seg_start)[-1])
        self.all_rows = torch.arange(self.T, dtype=torch.int32, device=device)
        self.idx = [torch.empty(max(1, k), dtype=torch.int32, device=device) for _ in layers]
        self.imp = torch.empty(int(self.deep.sizes["total_keys"]), dtype=torch.float32, device=device)
        inter = layers[0]["w_gate"].shape[0]
        self.ffn_ws = torch.empty(max(16, sparse_ffn_workspace_size(self.T, inter)), dtype=torch.uint8,
                                  device=device)

    def forward(self, hidden, stream=None):
        """hidden: [T_q][hidden] bf16, updated in place. Returns the rows each layer's FFN took."""
        chosen = []
        for li, L in enumerate(self.layers):
            lay = self.shallow if li < self.n_shallow else self.deep
            q = lay.qkv_rope_append(hidden, L["w_qkv"], self.theta, self.spi, self.spg, L["k_pool"], L["v_pool"],
                                    stream=stream)
            out, lse = lay.attention(q, L["k_pool"], L["v_pool"], stream=stream)
            lay.out_proj_residual(out, L["w_o"], hidden, stream=stream)
            if li < self.n_shallow:
                idx, k = self.all_rows, self.T
            else:
                lay.importance_topk(q, L["k_pool"], lse, self.n_last, None, importance=self.imp, stream=stream)
                idx, k = self.idx[li], self.k
                segkv_topk_select(self.imp[self.bq:self.bq + self.T], self.T, k, idx, stream=stream)
            sparse_ffn_swiglu(hidden, idx, k, L["w_gate"], L["w_up"], L["w_down"], self.ffn_ws, stream=stream)
            chosen.append(idx)
        return chosen
