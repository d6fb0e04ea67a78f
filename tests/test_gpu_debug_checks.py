"""GPU: the SEGKV_DEBUG build (libsegkv_debug.so) reports out-of-range page ids
as SEGKV_ERR_DEVICE_CHECK; the release build, given the same inputs, skips the
move or reads the page as missing (zero) and returns SEGKV_OK. Every planted
error is an id the kernels already bound-check, so no access leaves its
buffer in either build. A clean call after a reported one succeeds (the flag
is cleared), and clean debug results equal the release results bit for bit."""
import contextlib

import numpy as np
import pytest
import torch

import head_aware_paged_amd as hk
import workloads
from gpu_util import bits, build

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def using(lib):
    """Route the binding's calls to another build of the library."""
    old = hk._lib
    hk._lib = lib
    try:
        yield
    finally:
        hk._lib = old


def relocate(lib, src_page, dst_page):
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    k_src = torch.randn(4, 16, 128, generator=g, device="cuda").to(torch.bfloat16)
    v_src = torch.randn(4, 128, 16, generator=g, device="cuda").to(torch.bfloat16)
    k_dst = torch.zeros(4, 16, 128, dtype=torch.bfloat16, device="cuda")
    v_dst = torch.zeros(4, 128, 16, dtype=torch.bfloat16, device="cuda")
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    with using(lib):
        try:
            hk.rope_relocate(k_src, k_dst, v_src, v_dst, i32(src_page), i32(dst_page), i32([5] * len(src_page)),
                             len(src_page), 16, 128, 1e6)
            code = 0
        except hk.SegkvError as e:
            code = e.code
    torch.cuda.synchronize()
    return code, bits(k_dst), bits(v_dst)


def test_relocate_out_of_range_move():
    print("case relocate: move 2 has destination page 9 of a 4-page pool", flush=True)
    dbg, rel = hk.load_debug(), hk.load()
    c_rel, k_rel, v_rel = relocate(rel, [0, 1, 2], [3, 0, 9])
    c_dbg, k_dbg, v_dbg = relocate(dbg, [0, 1, 2], [3, 0, 9])
    assert c_rel == 0 and c_dbg == hk.SEGKV_ERR_DEVICE_CHECK
    assert b"rope_relocate" in dbg.segkv_last_error()
    assert dbg.segkv_status_string(c_dbg) == b"SEGKV_ERR_DEVICE_CHECK"
    # the valid moves are done identically by both builds; page 9 is skipped
    assert np.array_equal(k_rel, k_dbg) and np.array_equal(v_rel, v_dbg)
    assert np.all(k_rel[1:3] == 0) and np.any(k_rel[0] != 0) and np.any(k_rel[3] != 0)
    # the flag was cleared: a clean call succeeds
    assert relocate(dbg, [0, 1], [3, 0])[0] == 0


def attend(lib, layer, dev):
    with using(lib):
        try:
            out, lse = layer.attention(dev.q, dev.k_work, dev.v_work)
            code = 0
        except hk.SegkvError as e:
            return e.code, None
    torch.cuda.synchronize()
    return code, bits(out)


def test_attention_table_entry_out_of_range():
    w = workloads.tiny()
    print("case tiny_224: a page-table entry set past the pool", flush=True)
    dbg, rel = hk.load_debug(), hk.load()
    layer, dev = build(w)
    c_rel, ref = attend(rel, layer, dev)
    c_dbg, got = attend(dbg, layer, dev)
    assert c_rel == 0 and c_dbg == 0 and np.array_equal(ref, got)  # clean tables: same bits, no report
    bad = layer.page_ids.clone()
    layer.page_ids[5] = dev.k_work.shape[0] + 7
    assert attend(rel, layer, dev)[0] == 0  # release: the entry reads as a missing page
    c_dbg, _ = attend(dbg, layer, dev)
    assert c_dbg == hk.SEGKV_ERR_DEVICE_CHECK and b"segpaged_attn_prefill" in dbg.segkv_last_error()
    layer.page_ids.copy_(bad)
    assert attend(dbg, layer, dev)[0] == 0
