"""CPU: the masked-dense comparator's oracle pinned to things other than itself.

1. With the prefill visibility as the mask, it equals the (separately pinned)
   SegPaged attention oracle on the same layout.
2. With the causal mask of an all-global layout it equals torch's fp64
   scaled-dot-product attention (is_causal over the last T rows).
3. Pure-Python loops on a tiny case with a random mask, including a row whose
   mask is empty (O = 0, LSE = -inf).
"""
import math

import numpy as np
import torch

import oracle
import workloads

G_, L_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.DENSE


def test_class_mask_equals_segpaged_attention():
    w = workloads.tiny(window=8)
    K, V, mask = oracle.dense_layout(w, 256)
    O, L = oracle.masked_dense(w.q, K, V, mask)
    O2, L2 = oracle.attention(w)
    assert np.allclose(O, O2, rtol=0, atol=1e-12) and np.allclose(L, L2, rtol=0, atol=1e-12)


def test_causal_mask_equals_sdpa():
    w = workloads.make_custom("all_global", Hq=4, Hkv=2, D=64, theta=1e4, seg_lens_per_req=[[64, 48]],
                              orig_starts_per_req=[[0, None]], classes=[G_, G_], windows=[0, 0], seed=2)
    K, V, mask = oracle.dense_layout(w, 128)
    O, L = oracle.masked_dense(w.q, K, V, mask)
    q = torch.from_numpy(oracle.bf16_bits_to_f64(w.q)).permute(1, 0, 2)            # [Hq, T, D]
    k = torch.from_numpy(oracle.bf16_bits_to_f64(K[:, :112])).repeat_interleave(2, 0)  # [Hq, 112, D]
    v = torch.from_numpy(oracle.bf16_bits_to_f64(V[:, :112])).repeat_interleave(2, 0)
    causal = torch.ones(48, 112, dtype=torch.bool).tril(diagonal=64)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=causal)
    assert np.allclose(O, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_brute_force_random_mask():
    rng = np.random.default_rng(3)
    T, Hq, Hkv, D, L = 5, 4, 2, 8, 64
    q = oracle.f64_to_bf16_bits(rng.standard_normal((T, Hq, D)))
    k = oracle.f64_to_bf16_bits(rng.standard_normal((Hkv, L, D)))
    v = oracle.f64_to_bf16_bits(rng.standard_normal((Hkv, L, D)))
    mask = (rng.random((Hkv, T, L)) < 0.3).astype(np.uint8)
    mask[1, 2] = 0  # an empty row for kv head 1
    O, Ls = oracle.masked_dense(q, k, v, mask)
    Q, Kf, Vf = (oracle.bf16_bits_to_f64(x).tolist() for x in (q, k, v))
    for t in range(T):
        for g in range(Hq):
            h = g // 2
            keys = [j for j in range(L) if mask[h, t, j]]
            if not keys:
                assert np.all(O[t, g] == 0) and Ls[t, g] == -np.inf
                continue
            s = [sum(a * b for a, b in zip(Q[t][g], Kf[h][j])) / math.sqrt(D) for j in keys]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            for d in range(D):
                assert math.isclose(O[t, g, d], sum(e[i] * Vf[h][j][d] for i, j in enumerate(keys)) / sum(e),
                                    rel_tol=1e-12, abs_tol=1e-12)
            assert math.isclose(Ls[t, g], mx + math.log(sum(e)), rel_tol=1e-12)
