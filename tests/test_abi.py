"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import head_aware_paged_amd as hk
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "segkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hk.LIB_PATH), reason="libsegkv.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(segkv_\w+|rope_relocate|segpaged_attn_\w+|token_importance_topk|"
                                 r"sparse_ffn_\w+|masked_dense_attn)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = hk.load()
    names = _declared()
    assert set(names) == set(hk.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = hk.load()
    assert lib.segkv_status_string(0) == b"SEGKV_OK"
    for code, name in [(-1, b"SEGKV_ERR_INVALID_ARG"), (-2, b"SEGKV_ERR_UNSUPPORTED"), (-3, b"SEGKV_ERR_CAPACITY"),
                       (-4, b"SEGKV_ERR_ALIGNMENT"), (-5, b"SEGKV_ERR_WORKSPACE"), (-6, b"SEGKV_ERR_HIP"),
                       (-7, b"SEGKV_ERR_DEVICE_CHECK")]:
        assert lib.segkv_status_string(code) == name


def _layout(**over):
    base = dict(R=1, Hq=8, Hkv=4, D=64, P=16,
                seg_indptr=[0, 4], seg_start=[0, 64, 128, 192], seg_len=[64, 64, 64, 32],
                head_class=[0, 1, 1, 3], window=[0, 32, 32, 0], retr_seg=[-1] * 8)
    base.update(over)
    d = hk.dims(base["R"], base["Hq"], base["Hkv"], base["D"], base["P"], len(base["seg_start"]))
    m = hk.HostMeta(base["seg_indptr"], base["seg_start"], base["seg_len"], base["head_class"], base["window"],
                    base["retr_seg"])
    return d, m


def _code(**over):
    d, m = _layout(**over)
    try:
        hk.segkv_plan_sizes(d, m)
        return 0
    except hk.SegkvError as e:
        return e.code


def test_valid_layout_sizes():
    d, m = _layout()
    s = hk.segkv_plan_sizes(d, m)
    assert s["table_entries"] == 14 + 4 + 4 + 14
    assert s["move_entries"] == 12 + 2 + 2 + 12
    assert s["total_q_rows"] == 32 and s["total_keys"] == 224
    assert s["plan_bytes"] > 0


@pytest.mark.parametrize("over,code", [
    (dict(Hq=6), -1),                                   # Hq % Hkv != 0
    (dict(D=96), -2),                                   # unsupported head_dim
    (dict(P=32), -2),                                   # unsupported page size
    (dict(Hq=12, Hkv=4), -2),                           # group 3 does not divide 256
    (dict(R=0), -1),
    (dict(head_class=[0, 7, 1, 3]), -1),                # unknown class
    (dict(window=[0, 0, 32, 0]), -1),                   # LOCAL with window 0
    (dict(seg_start=[0, 64, 120, 192]), -1),            # not contiguous / not page-aligned
    (dict(seg_len=[64, 0, 64, 32]), -1),                # empty segment
    (dict(seg_len=[60, 64, 64, 32], seg_start=[0, 60, 124, 188]), -1),  # unaligned start
    (dict(seg_indptr=[0, 3]), -1),                      # indptr does not end at S
    (dict(head_class=[2, 1, 1, 3], retr_seg=[0, 0] + [-1] * 6), -1),  # retrieval: same segment twice
    (dict(head_class=[2, 1, 1, 3], retr_seg=[0, 3] + [-1] * 6), -1),  # retrieval: query segment
    (dict(head_class=[2, 1, 1, 3], retr_seg=[0, 2] + [-1] * 6), 0),   # valid retrieval
])
def test_layout_validation(over, code):
    assert _code(**over) == code


def test_call_level_validation_returns_before_launch():
    lib = hk.load()
    # rope_relocate: bad shapes are rejected synchronously
    assert lib.rope_relocate(None, None, None, None, 1, 1, None, None, None, -1, 16, 128, 1e4, None) == -1
    assert lib.rope_relocate(None, None, None, None, 1, 1, None, None, None, 4, 32, 128, 1e4, None) == -2
    assert lib.rope_relocate(None, None, None, None, 1, 1, None, None, None, 4, 16, 80, 1e4, None) == -2
    assert lib.rope_relocate(None, None, None, None, 1, 1, None, None, None, 4, 16, 128, 1e4, None) == -1
    assert lib.rope_relocate(16, 16, None, None, 1, 1, 16, 16, 16, 0, 16, 128, 1e4, None) == 0  # no moves: no-op
    assert lib.rope_relocate(8, 16, None, None, 1, 1, 16, 16, 16, 4, 16, 128, 1e4, None) == -4  # misaligned
    assert lib.rope_relocate(16, 16, 16, None, 1, 1, 16, 16, 16, 4, 16, 128, 1e4, None) == -1  # v half given
    # top-k / ffn
    assert lib.segkv_topk_select(None, 10, 11, None, None) == -1
    assert lib.segkv_topk_select(None, 10, 0, None, None) == 0
    assert lib.sparse_ffn_swiglu(None, 8, 100, 256, None, 4, None, None, None, None, 0, None) == -2
    assert lib.sparse_ffn_swiglu(None, 8, 128, 256, None, 9, None, None, None, None, 0, None) == -1
    assert lib.sparse_ffn_workspace_size(4, 256) == 4 * 256 * 2
    assert b"k <= n" in lib.segkv_last_error() or lib.segkv_last_error() != b""


def test_attention_validation():
    lib = hk.load()
    d, m = _layout()
    ms = m.struct()
    s = hk.segkv_plan_sizes(d, m)
    args = lambda **kw: [ctypes.byref(kw.get("d", d)), ctypes.byref(ms), kw.get("q", 16), 16, 16, 10, 16, 16,
                         16, kw.get("plan_bytes", s["plan_bytes"]), kw.get("scale", 0.125), 16, None, None,
                         kw.get("ws", s["attn_workspace_bytes"]), None]
    assert lib.segpaged_attn_prefill(*args(q=None)) == -1
    assert lib.segpaged_attn_prefill(*args(q=8)) == -4
    assert lib.segpaged_attn_prefill(*args(scale=-1.0)) == -1
    assert lib.segpaged_attn_prefill(*args(plan_bytes=8)) == -5
    bad = hk.dims(1, 8, 4, 64, 16, 3)   # num_segments disagrees with seg_indptr
    assert lib.segpaged_attn_prefill(*args(d=bad)) == -1
    # the no-alloc entry validates like the workspace entry, before any device call
    nargs = lambda **kw: args(**kw)[:-3] + [None]
    assert lib.segpaged_attn_prefill_noalloc(*nargs(q=None)) == -1
    assert lib.segpaged_attn_prefill_noalloc(*nargs(q=8)) == -4
    assert lib.segpaged_attn_prefill_noalloc(*nargs(plan_bytes=8)) == -5
    # build_pages: capacity below the exact table size
    dm = hk.Meta(16, 16, 16, 16, 16, 16)
    rc = lib.segkv_build_pages(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), 16, 16, 16, 16, 16, 16,
                               s["table_entries"] - 1, None, None, None, None, None, None, 0, 16,
                               s["plan_bytes"], None)
    assert rc == -3
    rc = lib.segkv_build_pages(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), 16, 16, 16, 16, 16, 16,
                               s["table_entries"], None, None, None, 16, None, None, 0, 16, s["plan_bytes"], None)
    assert rc == -1  # moves requested without cache pointers


def test_importance_validation():
    """token_importance_topk validates its workspace and limits on the host, before any launch."""
    lib = hk.load()
    d, m = _layout()
    ms = m.struct()
    s = hk.segkv_plan_sizes(d, m)
    dm = hk.Meta(16, 16, 16, 16, 16, 16)
    k = (ctypes.c_int32 * 1)(10)
    args = lambda **kw: [ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), 16, 16, 16, 10, 16, 16, 16, 16,
                         kw.get("plan_bytes", s["plan_bytes"]), 16, 0.125, kw.get("n_last", 16), k, 16,
                         kw.get("idx", None), kw.get("ws", 16), kw.get("ws_bytes", s["importance_workspace_bytes"]),
                         None]
    assert s["importance_workspace_bytes"] == d.num_kv_heads * s["total_keys"] * 4
    assert lib.token_importance_topk(*args(ws=None)) == -5
    assert lib.token_importance_topk(*args(ws_bytes=s["importance_workspace_bytes"] - 4)) == -5
    assert lib.token_importance_topk(*args(ws=8)) == -4
    assert lib.token_importance_topk(*args(n_last=0)) == -1
    assert lib.token_importance_topk(*args(n_last=4096)) == -2
    assert lib.token_importance_topk(*args(plan_bytes=8)) == -5


def test_glue_decode_comparator_validation():
    """Host-side checks of the layer glue, decode and comparator entry points (nothing launched)."""
    lib = hk.load()
    d, m = _layout()
    ms = m.struct()
    dm = hk.Meta(16, 16, 16, 16, 16, 16)
    n = ctypes.c_size_t(0)
    assert lib.segkv_qkv_workspace_size(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value > 0
    ws = n.value

    def qkv(hidden_size=256, theta=1e4, ws_bytes=ws, hidden=16, pool_pages=10):
        return lib.segkv_qkv_rope_append(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(dm), 16, 16, 16,
                                         pool_pages, hidden, hidden_size, 16, theta, 16, 16, 16, 16, ws_bytes, None)
    assert qkv(hidden_size=100) == -2          # not a multiple of 64
    assert qkv(theta=0.0) == -1
    assert qkv(ws_bytes=ws - 1) == -5
    assert qkv(hidden=8) == -4                 # misaligned
    assert qkv(hidden=None) == -1
    assert qkv(pool_pages=0) == -1
    # output projection
    assert lib.segkv_out_proj_residual(16, 4, 100, 16, 16, 128, None) == -2
    assert lib.segkv_out_proj_residual(16, 4, 64, 16, 16, 100, None) == -2
    assert lib.segkv_out_proj_residual(16, 0, 64, 16, 16, 128, None) == 0   # no rows: no-op
    assert lib.segkv_out_proj_residual(8, 4, 64, 16, 16, 128, None) == -4
    # decode: workspace size and a group size above 16
    assert lib.segkv_decode_workspace_size(ctypes.byref(d), ctypes.byref(ms), ctypes.byref(n)) == 0
    big = hk.dims(1, 68, 4, 64, 16, 4)
    assert lib.segkv_decode_workspace_size(ctypes.byref(big), ctypes.byref(ms), ctypes.byref(n)) != 0
    # standalone masked dense
    assert lib.segkv_masked_dense_workspace_size(32, 8, 4, 64, 100, ctypes.byref(n)) == -2   # L % 64
    assert lib.segkv_masked_dense_workspace_size(32, 8, 3, 64, 128, ctypes.byref(n)) == -1   # Hq % Hkv
    assert lib.segkv_masked_dense_workspace_size(32, 8, 4, 80, 128, ctypes.byref(n)) == -2   # head_dim
    assert lib.segkv_masked_dense_workspace_size(32, 8, 4, 64, 128, ctypes.byref(n)) == 0
    dws = n.value
    assert lib.masked_dense_attn(16, 16, 16, 16, 32, 8, 4, 64, 128, ctypes.c_float(0.125), 16, None, 16,
                                 dws - 1, None) == -5
    assert lib.masked_dense_attn(16, 16, 16, 8, 32, 8, 4, 64, 128, ctypes.c_float(0.125), 16, None, 16,
                                 dws, None) == -4
    assert lib.masked_dense_attn(16, 16, 16, 16, 32, 8, 4, 64, 128, ctypes.c_float(-1.0), 16, None, 16,
                                 dws, None) == -1
    # masked prefill: the mask must cover every request's last page
    s = hk.segkv_plan_sizes(d, m)
    margs = lambda mask, mask_L: [ctypes.byref(d), ctypes.byref(ms), 16, 16, 16, 10, 16, 16, 16, s["plan_bytes"],
                                  ctypes.c_float(0.125), mask, mask_L, 16, None, 16, s["attn_workspace_bytes"], None]
    assert lib.segpaged_attn_prefill_masked(*margs(None, 256)) == -1
    assert lib.segpaged_attn_prefill_masked(*margs(16, 200)) == -1     # not a multiple of 16
    assert lib.segpaged_attn_prefill_masked(*margs(16, 16)) == -1      # too short
    assert lib.segpaged_attn_prefill_masked(*margs(8, 256)) == -4      # misaligned mask
