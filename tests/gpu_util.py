"""Shared helpers for the GPU tests: move workloads to the device and compare."""
import math

import numpy as np
import torch

import oracle
from head_aware_paged_amd.session import SegPagedLayer

DEV = "cuda"


def bf16(u16) -> torch.Tensor:
    a = np.ascontiguousarray(u16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)


def v_pages(u16) -> np.ndarray:
    """A V pool [pages][P][D] (token-major, as the workloads hold it) in the
    library's d-major page layout [pages][D][P]."""
    return np.ascontiguousarray(np.swapaxes(u16, 1, 2))


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def layer_for(w) -> SegPagedLayer:
    return SegPagedLayer(w.num_q_heads, w.num_kv_heads, w.head_dim, w.seg_indptr, w.seg_start, w.seg_len,
                         w.head_class, w.window, w.retr_seg, page_size=w.page_size, device=DEV)


class Dev:
    """Device copies of a workload's tensors and layout arrays."""

    def __init__(self, w, cache=True):
        self.q = bf16(w.q)
        self.k_work = bf16(w.k_work)
        self.v_work = bf16(v_pages(w.v_work))
        self.seg_page_indptr = i32(w.seg_page_indptr)
        self.seg_pages = i32(w.seg_pages)
        if cache and w.k_cache.shape[0] > 0:
            self.k_cache = bf16(w.k_cache)
            self.v_cache = bf16(v_pages(w.v_cache))
            self.cache_page_indptr = i32(w.cache_page_indptr)
            self.cache_pages = i32(w.cache_pages)
            self.seg_orig_start = i32(w.seg_orig_start)
        else:
            self.k_cache = self.v_cache = self.cache_page_indptr = self.cache_pages = self.seg_orig_start = None


def build(w, dev=None, moves=True):
    dev = dev or Dev(w)
    layer = layer_for(w)
    if moves and dev.cache_pages is not None:
        layer.build_pages(dev.seg_page_indptr, dev.seg_pages, dev.cache_page_indptr, dev.cache_pages,
                          dev.seg_orig_start)
    else:
        layer.build_pages(dev.seg_page_indptr, dev.seg_pages)
    return layer, dev


def bf16_to_f64(u16):
    return oracle.bf16_bits_to_f64(u16)


def attn_errors(out_bits, lse_gpu, O_ref, L_ref, rows=None):
    """Error statistics of GPU attention against the fp64 oracle on the given rows."""
    O = bf16_to_f64(out_bits)
    if rows is not None:
        O, O_ref, lse_gpu, L_ref = O[rows], O_ref[rows], lse_gpu[rows], L_ref[rows]
    d = np.abs(O - O_ref)
    # relative Frobenius error per query head
    num = np.sqrt((d ** 2).sum(axis=(0, 2)))
    den = np.sqrt((O_ref ** 2).sum(axis=(0, 2)))
    return dict(max_abs=float(d.max()), mean_abs=float(d.mean()),
                lse_abs=float(np.abs(lse_gpu.astype(np.float64) - L_ref).max()),
                rel_fro=float((num / np.maximum(den, 1e-30)).max()))


def assert_attn_close(out_bits, lse_gpu, O_ref, L_ref, rows=None, name=""):
    e = attn_errors(out_bits, lse_gpu, O_ref, L_ref, rows)
    print(f"[{name}] {e}", flush=True)
    assert e["max_abs"] <= 2e-2 and e["mean_abs"] <= 2e-3, e
    assert e["lse_abs"] <= 1e-3, e
    assert e["rel_fro"] <= 1e-2, e
    return e


def sample_rows(w, per_request=12, seed=0):
    """Query rows spread over every request: first, last, m-tile edges and random ones."""
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(w.num_requests):
        a, b = int(w.cu_q[r]), int(w.cu_q[r + 1])
        n = b - a
        pick = {0, n - 1, min(n - 1, 31), min(n - 1, 32), n // 2}
        pick.update(int(x) for x in rng.integers(0, n, size=max(0, per_request - len(pick))))
        rows.extend(a + t for t in sorted(pick))
    return sorted(set(rows))
