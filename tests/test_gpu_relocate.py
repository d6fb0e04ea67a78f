"""GPU: RoPE relocation + page gather vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Dev, bf16, bits, build, i32, v_pages

pytestmark = pytest.mark.gpu


def full_moves(w):
    """Every reused (segment, head) page: cache page -> working page, delta = b_s - o_s."""
    src, dst, delta = [], [], []
    Hkv = w.num_kv_heads
    for r in range(w.num_requests):
        for s in w.segments_of(r)[:-1]:
            for h in range(Hkv):
                a, b = w.cache_page_indptr[s * Hkv + h], w.cache_page_indptr[s * Hkv + h + 1]
                c, d = w.seg_page_indptr[s * Hkv + h], w.seg_page_indptr[s * Hkv + h + 1]
                src.extend(w.cache_pages[a:b])
                dst.extend(w.seg_pages[c:d])
                delta.extend([int(w.seg_start[s] - w.seg_orig_start[s])] * (b - a))
    return np.array(src, np.int32), np.array(dst, np.int32), np.array(delta, np.int32)


def check_k(w, k_out_bits, src, dst, delta):
    """Bound: |gpu - ref64| <= ulp_bf16(ref64) + 2^-20 max(|x_j|, |x_{j+D/2}|)."""
    D = w.head_dim
    x = oracle.bf16_bits_to_f64(w.k_cache[src])                  # [n, 16, D]
    ref = oracle.relocate(x, delta[:, None], w.rope_theta)
    got = oracle.bf16_bits_to_f64(k_out_bits[dst])
    pairmax = np.maximum(np.abs(x[..., :D // 2]), np.abs(x[..., D // 2:]))
    pairmax = np.concatenate([pairmax, pairmax], axis=-1)
    bound = oracle.ulp_bf16(ref) + 2.0 ** -20 * pairmax
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err - bound).max())
    frac = float(np.mean(k_out_bits[dst] == oracle.f64_to_bf16_bits(ref)))
    print(f"[{w.name}] bit-equal to RNE(ref64): {frac:.6f}", flush=True)
    assert frac > 0.999
    zero = delta == 0
    if zero.any():
        assert np.array_equal(k_out_bits[dst[zero]], w.k_cache[src[zero]])


@pytest.mark.parametrize("make", [workloads.tiny, workloads.mistral_32k, workloads.long_64k],
                         ids=["tiny_224", "mistral7b_32k", "long_64k"])
def test_full_relocation(make):
    w = make(fill_reused_work=False)
    print(f"case {w.name}: full relocation", flush=True)
    src, dst, delta = full_moves(w)
    dev = Dev(w)
    k_out = dev.k_work.clone()
    v_out = dev.v_work.clone()
    from head_aware_paged_amd import rope_relocate
    rope_relocate(dev.k_cache, k_out, dev.v_cache, v_out, i32(src), i32(dst), i32(delta), len(src), 16,
                  w.head_dim, w.rope_theta)
    torch.cuda.synchronize()
    kb, vb = bits(k_out), bits(v_out)
    check_k(w, kb, src, dst, delta)
    # V pages move verbatim (in the d-major page layout the pools use)
    assert np.array_equal(vb[dst], v_pages(w.v_cache[src]))
    untouched = np.setdiff1d(np.arange(w.k_work.shape[0]), dst)
    assert np.array_equal(kb[untouched], w.k_work[untouched])
    assert np.array_equal(vb[untouched], v_pages(w.v_work[untouched]))


def test_head_aware_moves_and_k_only():
    w = workloads.mistral_32k(fill_reused_work=False)
    print("case mistral7b_32k: head-aware move list, K only", flush=True)
    layer, dev = build(w)
    k_out = dev.k_work.clone()
    layer.relocate(dev.k_cache, k_out, None, None, w.rope_theta)
    torch.cuda.synchronize()
    src, dst, delta = oracle.move_list(w)
    kb = bits(k_out)
    check_k(w, kb, src, dst, delta)
    untouched = np.setdiff1d(np.arange(w.k_work.shape[0]), dst)
    assert np.array_equal(kb[untouched], w.k_work[untouched])


def test_in_place_and_out_of_range_moves():
    w = workloads.tiny()
    print("case tiny_224: in-place relocation, invalid ids skipped", flush=True)
    k = bf16(w.k_cache)
    n = w.k_cache.shape[0]
    src = np.arange(n, dtype=np.int32)
    delta = np.full(n, 37, np.int32)
    src_bad = src.copy()
    src_bad[3] = n + 5           # out of range: skipped
    dst = src_bad.copy()
    dst[3] = 3
    from head_aware_paged_amd import rope_relocate
    rope_relocate(k, k, None, None, i32(src_bad), i32(dst), i32(delta), n, 16, w.head_dim, w.rope_theta)
    torch.cuda.synchronize()
    kb = bits(k)
    ok = np.arange(n) != 3
    check_k(w, kb, src[ok], src[ok], delta[ok])
    assert np.array_equal(kb[3], w.k_cache[3])
