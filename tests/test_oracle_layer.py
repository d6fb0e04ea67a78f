"""CPU: the layer-glue oracle (projection + RoPE + append, output projection)
pinned to things other than itself.

1. One-hot projection rows: Q/K/V equal the rotation (``oracle.rope``, pinned
   on its own) of the hidden features the rows pick, in the stacking order
   Q heads, K heads, V heads; V is not rotated.
2. RoPE is a rotation that depends on relative position only: with every row
   of a request holding the same hidden vector, q(p) . k(p) equals the
   unrotated q . k for every row, and q(p + 1) . k(p) is the same for every p;
   a row at position 0 is not rotated at all.
3. The append puts row t's K/V where the store reader (``oracle.gather_kv``)
   finds position b_q + t, and leaves every other page untouched.
4. Output projection: W_o = identity gives hidden + attn exactly; W_o = 0
   gives hidden.
5. The chain with the query rows of W_qkv zero: attention is uniform over the
   visible keys, so the layer output is hidden + the bf16 mean of the
   visible V rows (identity W_o).
6. Projection = pure-Python dot products on a tiny case.
"""
import math

import numpy as np

import oracle
import workloads

G_, L_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.DENSE


def _layout(seg_lens=((32, 48, 21), (16, 7)), D=64):
    return workloads.make_custom("glue", Hq=4, Hkv=2, D=D, theta=1e4,
                                 seg_lens_per_req=[list(x) for x in seg_lens],
                                 orig_starts_per_req=[[0] * (len(x) - 1) + [None] for x in seg_lens],
                                 classes=[G_, L_, D_, L_], windows=[0, 20, 0, 9], seed=4)


def _bits(x):
    return oracle.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_one_hot_rows_pick_features():
    w = _layout()
    Hq, Hkv, D, Hd = 4, 2, 64, 512
    hidden, _, _ = workloads.layer_inputs(w, Hd, seed=1)
    rng = np.random.default_rng(0)
    sel = rng.permutation(Hd)[:(Hq + 2 * Hkv) * D]
    W = np.zeros(((Hq + 2 * Hkv) * D, Hd))
    W[np.arange(len(sel)), sel] = 1.0
    q, k, v = oracle.qkv_rope(w, hidden, _bits(W))
    X = oracle.bf16_bits_to_f64(hidden)[:, sel]
    pos = oracle.row_positions(w)[:, None]
    assert np.array_equal(q, oracle.rope(X[:, :Hq * D].reshape(-1, Hq, D), pos, 1e4))
    assert np.array_equal(k, oracle.rope(X[:, Hq * D:(Hq + Hkv) * D].reshape(-1, Hkv, D), pos, 1e4))
    assert np.array_equal(v, X[:, (Hq + Hkv) * D:].reshape(-1, Hkv, D))


def test_rotation_relative_position():
    w = _layout(seg_lens=((16, 40),))  # one request, query rows at positions 16..55
    Hd = 128
    hidden, w_qkv, _ = workloads.layer_inputs(w, Hd, seed=2)
    hidden[:] = hidden[0]  # every row holds the same vector
    q, k, _ = oracle.qkv_rope(w, hidden, w_qkv)
    Y = oracle.bf16_bits_to_f64(hidden[:1]) @ oracle.bf16_bits_to_f64(w_qkv).T
    q0, k0 = Y[0, :4 * 64].reshape(4, 64), Y[0, 4 * 64:6 * 64].reshape(2, 64)
    for g in range(4):
        h = g // 2
        same = np.einsum("td,td->t", q[:, g], k[:, h])
        assert np.allclose(same, q0[g] @ k0[h], rtol=1e-12, atol=1e-12)
        nxt = np.einsum("td,td->t", q[1:, g], k[:-1, h])
        assert np.allclose(nxt, nxt[0], rtol=1e-12, atol=1e-12)
        assert abs(nxt[0] - same[0]) > 1e-6  # the rotation is not the identity
    # norms of the rotated pairs (j, j + D/2) are those of the unrotated pairs
    assert np.allclose(np.hypot(q[..., :32], q[..., 32:]), np.hypot(q0[..., :32], q0[..., 32:]), rtol=1e-12)
    # a request with no reused segment: its first row is at position 0, unrotated
    w0 = _layout(seg_lens=((24,),))
    h0, wq0, _ = workloads.layer_inputs(w0, Hd, seed=3)
    q, k, v = oracle.qkv_rope(w0, h0, wq0)
    Y = oracle.bf16_bits_to_f64(h0[:1]) @ oracle.bf16_bits_to_f64(wq0).T
    assert np.array_equal(q[0].ravel(), Y[0, :4 * 64]) and np.array_equal(k[0].ravel(), Y[0, 4 * 64:6 * 64])


def test_append_lands_where_the_store_reads():
    w = _layout()
    hidden, w_qkv, _ = workloads.layer_inputs(w, 128, seed=5)
    _, k, v = oracle.qkv_rope(w, hidden, w_qkv)
    kb, vb = _bits(k), _bits(v)
    kp, vp = oracle.append_query_kv(w, kb, vb)
    touched = set()
    for r in range(w.num_requests):
        s = w.query_segment(r)
        bq, n = int(w.seg_start[s]), int(w.seg_len[s])
        t0 = int(w.cu_q[r])
        for h in range(w.num_kv_heads):
            K, V = oracle.gather_kv(w, r, h, kp, vp)
            assert np.array_equal(K[bq:bq + n], oracle.bf16_bits_to_f64(kb[t0:t0 + n, h]))
            assert np.array_equal(V[bq:bq + n], oracle.bf16_bits_to_f64(vb[t0:t0 + n, h]))
            K0, V0 = oracle.gather_kv(w, r, h)
            assert np.array_equal(K[:bq], K0[:bq]) and np.array_equal(V[:bq], V0[:bq])
            a, b = w.seg_page_indptr[s * w.num_kv_heads + h], w.seg_page_indptr[s * w.num_kv_heads + h + 1]
            touched.update(int(x) for x in w.seg_pages[a:b])
    rest = np.setdiff1d(np.arange(w.k_work.shape[0]), np.array(sorted(touched)))
    assert np.array_equal(kp[rest], w.k_work[rest]) and np.array_equal(vp[rest], w.v_work[rest])


def test_out_proj_identity_and_zero():
    rng = np.random.default_rng(1)
    hidden, attn = _bits(rng.standard_normal((9, 256))), _bits(rng.standard_normal((9, 256)))
    out = oracle.out_proj_residual(hidden, attn, _bits(np.eye(256)))
    assert np.array_equal(out, oracle.bf16_bits_to_f64(hidden) + oracle.bf16_bits_to_f64(attn))
    out = oracle.out_proj_residual(hidden, attn, np.zeros((256, 256), np.uint16))
    assert np.array_equal(out, oracle.bf16_bits_to_f64(hidden))


def test_chain_with_zero_queries_averages_visible_values():
    w = _layout()
    Hq, Hkv, D = 4, 2, 64
    Hd = Hq * D
    hidden, w_qkv, _ = workloads.layer_inputs(w, Hd, seed=6)
    w_qkv[:Hq * D] = 0
    out, mid = oracle.layer(w, hidden, w_qkv, _bits(np.eye(Hd)))
    kp, vp = oracle.append_query_kv(w, mid["k"], mid["v"])
    X = oracle.bf16_bits_to_f64(hidden)
    for r in range(w.num_requests):
        for tl in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            t = int(w.cu_q[r]) + tl
            i = int(w.seg_start[w.query_segment(r)]) + tl
            for g in range(Hq):
                _, V = oracle.gather_kv(w, r, g // 2, kp, vp)
                vis = oracle.visible_brute(w, r, g // 2, i)
                mean = oracle.round_bf16(V[vis].mean(axis=0))
                assert np.allclose(out[t, g * D:(g + 1) * D], X[t, g * D:(g + 1) * D] + mean, rtol=0, atol=1e-12)


def test_projection_brute_force():
    w = _layout(seg_lens=((16, 5),))
    Hd = 64
    hidden, w_qkv, _ = workloads.layer_inputs(w, Hd, seed=7)
    # rotation angle 0 needs position 0: compare V (unrotated) and |pairs| of Q, K
    q, k, v = oracle.qkv_rope(w, hidden, w_qkv)
    X = oracle.bf16_bits_to_f64(hidden).tolist()
    W = oracle.bf16_bits_to_f64(w_qkv).tolist()
    for t in range(5):
        y = [sum(a * b for a, b in zip(X[t], W[f])) for f in range(len(W))]
        for h in range(2):
            for d in range(64):
                assert math.isclose(v[t, h, d], y[(4 + 2 + h) * 64 + d], rel_tol=1e-12, abs_tol=1e-12)
        for g in range(4):
            for j in range(32):
                a, b = y[g * 64 + j], y[g * 64 + 32 + j]
                assert math.isclose(math.hypot(q[t, g, j], q[t, g, 32 + j]), math.hypot(a, b), rel_tol=1e-12)
