"""Python binding of libsegkv (SegPagedAttention prefill on MI355X / gfx950).

Argument marshalling only: every function forwards to the C entry point of the
same name in ``libsegkv.so`` (declared in ``include/segkv.h``), passing raw
device pointers of torch tensors, host pointers of numpy metadata arrays and
the current HIP stream. No computation happens here, and there is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsegkv.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libsegkv_debug.so")

SEGKV_OK = 0
SEGKV_ERR_DEVICE_CHECK = -7
GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3

EXPORTS = [
    "segkv_status_string", "segkv_last_error", "segkv_plan_sizes", "segkv_build_pages",
    "segkv_visible_spans", "rope_relocate", "segpaged_attn_prefill", "segpaged_attn_prefill_masked",
    "segpaged_attn_prefill_noalloc",
    "token_importance_topk",
    "segkv_decode_workspace_size", "segpaged_attn_decode",
    "segkv_topk_select", "sparse_ffn_workspace_size", "sparse_ffn_swiglu",
    "segkv_qkv_workspace_size", "segkv_qkv_rope_append", "segkv_out_proj_residual",
    "segkv_masked_dense_workspace_size", "masked_dense_attn",
]


class SegkvError(RuntimeError):
    def __init__(self, fn: str, code: int, status: str, detail: str):
        super().__init__(f"{fn} -> {status} ({code}): {detail}")
        self.code = code
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_requests", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_segments", ctypes.c_int32)]


class Meta(ctypes.Structure):
    _fields_ = [("seg_indptr", ctypes.c_void_p), ("seg_start", ctypes.c_void_p),
                ("seg_len", ctypes.c_void_p), ("head_class", ctypes.c_void_p),
                ("window", ctypes.c_void_p), ("retr_seg", ctypes.c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [("table_entries", ctypes.c_int64), ("move_entries", ctypes.c_int64),
                ("total_q_rows", ctypes.c_int64), ("total_keys", ctypes.c_int64),
                ("plan_bytes", ctypes.c_size_t), ("attn_workspace_bytes", ctypes.c_size_t),
                ("importance_workspace_bytes", ctypes.c_size_t)]


_lib = None


def _configure(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare every entry point's argument and result types."""
    P, I32, I64, F32, F64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    sig = {
        "segkv_status_string": ([I32], ctypes.c_char_p),
        "segkv_last_error": ([], ctypes.c_char_p),
        "segkv_plan_sizes": ([P, P, P], I32),
        "segkv_build_pages": ([P, P, P, P, P, P, P, P, P, I64, P, P, P, P, P, P, I64, P, SZ, P], I32),
        "segkv_visible_spans": ([P, P, P, P, P, P], I32),
        "rope_relocate": ([P, P, P, P, I64, I64, P, P, P, I32, I32, I32, F64, P], I32),
        "segpaged_attn_prefill": ([P, P, P, P, P, I64, P, P, P, SZ, F32, P, P, P, SZ, P], I32),
        "segpaged_attn_prefill_masked": ([P, P, P, P, P, I64, P, P, P, SZ, F32, P, I64, P, P, P, SZ, P], I32),
        "segpaged_attn_prefill_noalloc": ([P, P, P, P, P, I64, P, P, P, SZ, F32, P, P, P], I32),
        "segkv_decode_workspace_size": ([P, P, P], I32),
        "segpaged_attn_decode": ([P, P, P, P, P, P, P, P, I64, P, P, P, F32, P, P, P, SZ, P], I32),
        "token_importance_topk": ([P, P, P, P, P, P, I64, P, P, P, P, SZ, P, F32, I32, P, P, P, P, SZ, P], I32),
        "segkv_topk_select": ([P, I32, I32, P, P], I32),
        "sparse_ffn_workspace_size": ([I32, I32], SZ),
        "sparse_ffn_swiglu": ([P, I32, I32, I32, P, I32, P, P, P, P, SZ, P], I32),
        "segkv_qkv_workspace_size": ([P, P, P], I32),
        "segkv_qkv_rope_append": ([P, P, P, P, P, P, I64, P, I32, P, F64, P, P, P, P, SZ, P], I32),
        "segkv_out_proj_residual": ([P, I32, I32, P, P, I32, P], I32),
        "segkv_masked_dense_workspace_size": ([I32, I32, I32, I32, I32, P], I32),
        "masked_dense_attn": ([P, P, P, P, I32, I32, I32, I32, I32, F32, P, P, P, SZ, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsegkv.so (built in-tree by ``__graft_entry__.build()``; the
    SEGKV_LIB environment variable names another build of the same library,
    such as the sanitizer build of its host code)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("SEGKV_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"libsegkv.so not found at {path}; build it with __graft_entry__.build()")
    _lib = _configure(ctypes.CDLL(path))
    return _lib


def load_debug() -> ctypes.CDLL:
    """The SEGKV_DEBUG build (device-side bounds checks, synchronous entry
    points) as a separate library handle; the binding functions keep using
    load()."""
    if not os.path.exists(DEBUG_LIB_PATH):
        raise ImportError(f"libsegkv_debug.so not found at {DEBUG_LIB_PATH}; build it with __graft_entry__.build()")
    return _configure(ctypes.CDLL(DEBUG_LIB_PATH))


def _check(fn: str, code: int):
    if code != SEGKV_OK:
        lib = load()
        raise SegkvError(fn, code, lib.segkv_status_string(code).decode(), lib.segkv_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Raw pointer of a torch tensor / numpy array (None stays NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class HostMeta:
    """Host copies of the layout metadata (contiguous numpy arrays kept alive)."""

    def __init__(self, seg_indptr, seg_start, seg_len, head_class, window, retr_seg):
        self.seg_indptr = np.ascontiguousarray(seg_indptr, np.int32)
        self.seg_start = np.ascontiguousarray(seg_start, np.int32)
        self.seg_len = np.ascontiguousarray(seg_len, np.int32)
        self.head_class = np.ascontiguousarray(head_class, np.int8)
        self.window = np.ascontiguousarray(window, np.int32)
        self.retr_seg = np.ascontiguousarray(retr_seg, np.int32)

    def struct(self) -> Meta:
        return Meta(*(a.ctypes.data for a in (self.seg_indptr, self.seg_start, self.seg_len, self.head_class,
                                               self.window, self.retr_seg)))

    def to_device(self, device="cuda") -> "DeviceMeta":
        import torch
        return DeviceMeta(*(torch.from_numpy(a).to(device) for a in (
            self.seg_indptr, self.seg_start, self.seg_len, self.head_class, self.window, self.retr_seg)))


class DeviceMeta:
    """Device copies of the layout metadata (torch tensors)."""

    def __init__(self, seg_indptr, seg_start, seg_len, head_class, window, retr_seg):
        self.tensors = (seg_indptr, seg_start, seg_len, head_class, window, retr_seg)

    def struct(self) -> Meta:
        return Meta(*(t.data_ptr() for t in self.tensors))


def dims(num_requests, num_q_heads, num_kv_heads, head_dim, page_size, num_segments) -> Dims:
    return Dims(num_requests, num_q_heads, num_kv_heads, head_dim, page_size, num_segments)


def segkv_plan_sizes(d: Dims, meta: HostMeta) -> dict:
    lib = load()
    s = Sizes()
    ms = meta.struct()
    _check("segkv_plan_sizes", lib.segkv_plan_sizes(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in Sizes._fields_}


def segkv_build_pages(d: Dims, meta: HostMeta, dmeta: DeviceMeta, cu_q, seg_page_indptr, seg_pages,
                      page_indptr, page_ids, page_pos, plan, cache_page_indptr=None, cache_pages=None,
                      seg_orig_start=None, move_src=None, move_dst=None, move_delta=None, stream=None):
    lib = load()
    ms, dm = meta.struct(), dmeta.struct()
    _check("segkv_build_pages", lib.segkv_build_pages(
        ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), _ptr(cu_q), _ptr(seg_page_indptr), _ptr(seg_pages),
        _ptr(page_indptr), _ptr(page_ids), _ptr(page_pos), page_ids.numel(), _ptr(cache_page_indptr),
        _ptr(cache_pages), _ptr(seg_orig_start), _ptr(move_src), _ptr(move_dst), _ptr(move_delta),
        0 if move_src is None else move_src.numel(), _ptr(plan), plan.numel() * plan.element_size(),
        _stream(stream)))


def segkv_visible_spans(d: Dims, meta: HostMeta, dmeta: DeviceMeta, cu_q, spans, stream=None):
    lib = load()
    ms, dm = meta.struct(), dmeta.struct()
    _check("segkv_visible_spans", lib.segkv_visible_spans(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm),
                                                          _ptr(cu_q), _ptr(spans), _stream(stream)))


def rope_relocate(k_src, k_dst, v_src, v_dst, src_page, dst_page, delta, n_moves: int, page_size: int,
                  head_dim: int, rope_theta: float, stream=None):
    lib = load()
    _check("rope_relocate", lib.rope_relocate(
        _ptr(k_src), _ptr(k_dst), _ptr(v_src), _ptr(v_dst), k_src.shape[0], k_dst.shape[0], _ptr(src_page),
        _ptr(dst_page), _ptr(delta), n_moves, page_size, head_dim, float(rope_theta), _stream(stream)))


def segpaged_attn_prefill(d: Dims, meta: HostMeta, q, k_pool, v_pool, page_ids, page_pos, plan,
                          softmax_scale: float, out, lse=None, workspace=None, stream=None):
    lib = load()
    ms = meta.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("segpaged_attn_prefill", lib.segpaged_attn_prefill(
        ctypes.byref(d), ctypes.byref(ms), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(page_ids),
        _ptr(page_pos), _ptr(plan), plan.numel() * plan.element_size(), float(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def segpaged_attn_prefill_noalloc(d: Dims, meta: HostMeta, q, k_pool, v_pool, page_ids, page_pos, plan,
                                  softmax_scale: float, out, lse=None, stream=None):
    lib = load()
    ms = meta.struct()
    _check("segpaged_attn_prefill_noalloc", lib.segpaged_attn_prefill_noalloc(
        ctypes.byref(d), ctypes.byref(ms), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(page_ids),
        _ptr(page_pos), _ptr(plan), plan.numel() * plan.element_size(), float(softmax_scale), _ptr(out),
        _ptr(lse), _stream(stream)))


def segkv_decode_workspace_size(d: Dims, meta: HostMeta) -> int:
    lib = load()
    ms = meta.struct()
    n = ctypes.c_size_t(0)
    _check("segkv_decode_workspace_size", lib.segkv_decode_workspace_size(ctypes.byref(d), ctypes.byref(ms),
                                                                          ctypes.byref(n)))
    return int(n.value)


def segpaged_attn_decode(d: Dims, meta: HostMeta, dmeta: DeviceMeta, q_new, k_new, v_new, k_pool, v_pool,
                         page_indptr, page_ids, page_pos, softmax_scale: float, out, lse=None, workspace=None,
                         stream=None):
    lib = load()
    ms, dm = meta.struct(), dmeta.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("segpaged_attn_decode", lib.segpaged_attn_decode(
        ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
        _ptr(v_pool), k_pool.shape[0], _ptr(page_indptr), _ptr(page_ids), _ptr(page_pos), float(softmax_scale),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def token_importance_topk(d: Dims, meta: HostMeta, dmeta: DeviceMeta, cu_q, q, k_pool, page_indptr, page_ids,
                          page_pos, plan, lse, softmax_scale: float, n_last: int, k: Optional[Sequence[int]],
                          importance, topk_idx=None, workspace=None, stream=None):
    lib = load()
    ms, dm = meta.struct(), dmeta.struct()
    k_arr = None if k is None else np.ascontiguousarray(k, np.int32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("token_importance_topk", lib.token_importance_topk(
        ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), _ptr(cu_q), _ptr(q), _ptr(k_pool), k_pool.shape[0],
        _ptr(page_indptr), _ptr(page_ids), _ptr(page_pos), _ptr(plan), plan.numel() * plan.element_size(),
        _ptr(lse), float(softmax_scale), int(n_last),
        _ptr(k_arr), _ptr(importance), _ptr(topk_idx), _ptr(workspace), ws_bytes, _stream(stream)))


def segkv_topk_select(scores, n: int, k: int, idx, stream=None):
    lib = load()
    _check("segkv_topk_select", lib.segkv_topk_select(_ptr(scores), n, k, _ptr(idx), _stream(stream)))


def sparse_ffn_workspace_size(k: int, inter: int) -> int:
    return load().sparse_ffn_workspace_size(k, inter)


def sparse_ffn_swiglu(hidden, idx, k: int, w_gate, w_up, w_down, workspace, stream=None):
    lib = load()
    n_rows, hidden_size = hidden.shape
    inter = w_gate.shape[0]
    _check("sparse_ffn_swiglu", lib.sparse_ffn_swiglu(
        _ptr(hidden), n_rows, hidden_size, inter, _ptr(idx), k, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def segkv_qkv_workspace_size(d: Dims, meta: HostMeta) -> int:
    lib = load()
    ms = meta.struct()
    n = ctypes.c_size_t(0)
    _check("segkv_qkv_workspace_size", lib.segkv_qkv_workspace_size(ctypes.byref(d), ctypes.byref(ms),
                                                                    ctypes.byref(n)))
    return int(n.value)


def segkv_qkv_rope_append(d: Dims, meta: HostMeta, dmeta: DeviceMeta, cu_q, seg_page_indptr, seg_pages, hidden,
                          w_qkv, rope_theta: float, q_out, k_pool, v_pool, workspace, stream=None):
    lib = load()
    ms, dm = meta.struct(), dmeta.struct()
    _check("segkv_qkv_rope_append", lib.segkv_qkv_rope_append(
        ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), _ptr(cu_q), _ptr(seg_page_indptr), _ptr(seg_pages),
        k_pool.shape[0], _ptr(hidden), hidden.shape[1], _ptr(w_qkv), float(rope_theta), _ptr(q_out), _ptr(k_pool),
        _ptr(v_pool), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def segkv_out_proj_residual(attn, w_o, hidden, stream=None):
    """attn [n, F] (or [n, Hq, D]), w_o [Hd, F], hidden [n, Hd] updated in place."""
    lib = load()
    n, hd = hidden.shape
    _check("segkv_out_proj_residual", lib.segkv_out_proj_residual(
        _ptr(attn), n, w_o.shape[1], _ptr(w_o), _ptr(hidden), hd, _stream(stream)))


def segkv_masked_dense_workspace_size(T: int, Hq: int, Hkv: int, D: int, L: int) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check("segkv_masked_dense_workspace_size", lib.segkv_masked_dense_workspace_size(T, Hq, Hkv, D, L,
                                                                                      ctypes.byref(n)))
    return int(n.value)


def masked_dense_attn(q, k, v_t, mask, softmax_scale: float, out, lse=None, workspace=None, stream=None):
    """q [T][Hq][D], k [Hkv][L][D], v_t [Hkv][D][L], mask [Hkv][T][L] (uint8)."""
    lib = load()
    T, Hq, D = q.shape
    Hkv, L = k.shape[0], k.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("masked_dense_attn", lib.masked_dense_attn(
        _ptr(q), _ptr(k), _ptr(v_t), _ptr(mask), T, Hq, Hkv, D, L, float(softmax_scale), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def segpaged_attn_prefill_masked(d: Dims, meta: HostMeta, q, k_pool, v_pool, page_ids, page_pos, plan,
                                 softmax_scale: float, mask, out, lse=None, workspace=None, stream=None):
    """mask: [Hkv][T_q][mask_L] uint8 device tensor."""
    lib = load()
    ms = meta.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("segpaged_attn_prefill_masked", lib.segpaged_attn_prefill_masked(
        ctypes.byref(d), ctypes.byref(ms), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(page_ids),
        _ptr(page_pos), _ptr(plan), plan.numel() * plan.element_size(), float(softmax_scale), _ptr(mask),
        mask.shape[-1], _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))
