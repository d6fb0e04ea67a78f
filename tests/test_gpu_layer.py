"""GPU: the layer glue around the attention vs the fp64 oracle.

Projection + RoPE + append: Q, K and V are bf16 roundings of fp32-accumulated
dot products over hidden_size terms, rotated in fp32 with cos/sin rounded
from fp64. Summing hidden_size <= 4096 products of unit-variance sums in
fp32 leaves an absolute error of order sqrt(4096) 2^-24 = 2^-18, far under
half a bf16 step of a unit-size value (2^-9), so each GPU value is the
correctly rounded oracle value or, when the oracle value lies within that
error of a rounding boundary, its neighbour: |gpu - ref| <= 2^-8 |ref| +
2^-16 per element, and at least 99.9 % exactly equal to bf16(ref). Every pool page outside the query segments is unchanged.

Output projection: the same bound on hidden + W_o . attn.

Whole chain (projection -> page tables -> attention -> output projection):
the attention sees Q/K/V that differ from the oracle's by at most one bf16
step at rare elements, so the bar is the attention's: max |err| 3e-2 and mean
3e-3 on the output rows (unit-variance values), relative Frobenius 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Dev, bf16, bits, build, layer_for
from test_gpu_attention import SMALL_NAMES, small

pytestmark = pytest.mark.gpu


def _check_rounded(name, got_bits, ref):
    got = oracle.bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -16), (name, float(err.max()))
    exact = np.mean(got_bits == oracle.f64_to_bf16_bits(ref))
    assert exact >= 0.999, (name, exact)


def _qkv_case(w, hidden_size, seed):
    print(f"case {w.name}: qkv_rope_append hidden={hidden_size}", flush=True)
    hidden, w_qkv, _ = workloads.layer_inputs(w, hidden_size, seed=seed)
    dev = Dev(w, cache=False)
    layer = layer_for(w)
    q = layer.qkv_rope_append(bf16(hidden), bf16(w_qkv), w.rope_theta, dev.seg_page_indptr, dev.seg_pages,
                              dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    qr, kr, vr = oracle.qkv_rope(w, hidden, w_qkv)
    _check_rounded(w.name + " Q", bits(q), qr)
    kp, vp = bits(dev.k_work), np.swapaxes(bits(dev.v_work), 1, 2)
    Hkv = w.num_kv_heads
    got_k, got_v, ref_k, ref_v = [], [], [], []
    written = np.zeros(kp.shape[:2], dtype=bool)  # (page, slot) that a query row owns
    for r in range(w.num_requests):
        s = w.query_segment(r)
        for tl in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            t = int(w.cu_q[r]) + tl
            for h in range(Hkv):
                page = w.seg_pages[w.seg_page_indptr[s * Hkv + h] + tl // 16]
                written[page, tl % 16] = True
                got_k.append(kp[page, tl % 16])
                got_v.append(vp[page, tl % 16])
                ref_k.append(kr[t, h])
                ref_v.append(vr[t, h])
    _check_rounded(w.name + " K", np.stack(got_k), np.stack(ref_k))
    _check_rounded(w.name + " V", np.stack(got_v), np.stack(ref_v))
    # every other slot of the pools (reused segments, page tails): unchanged
    assert np.array_equal(kp[~written], w.k_work[~written])
    assert np.array_equal(vp[~written], w.v_work[~written])
    return layer, dev


@pytest.mark.parametrize("name", SMALL_NAMES)
def test_qkv_small(name):
    _qkv_case(small(name), 320, seed=1)


def test_qkv_mistral_32k():
    _qkv_case(workloads.mistral_32k(), 4096, seed=2)


def test_qkv_many_rows():
    # 48 feature tiles x 11 token tiles of 128 rows: the launch takes the 128-row token tile
    G_, L_ = workloads.GLOBAL, workloads.LOCAL
    w = workloads.make_custom("rows_1400", Hq=32, Hkv=8, D=128, theta=1e6, seg_lens_per_req=[[64, 1400]],
                              orig_starts_per_req=[[7, None]], classes=[G_] + [L_] * 7, windows=[0] + [300] * 7)
    _qkv_case(w, 256, seed=4)


# the last two take the 128-row token tile (>= 512 work-groups), the others the 64-row one
@pytest.mark.parametrize("n_rows,in_f,hd", [(1, 64, 128), (77, 256, 384), (300, 1024, 512), (512, 4096, 4096),
                                            (2048, 128, 4096), (2050, 64, 4096)])
def test_out_proj(n_rows, in_f, hd):
    print(f"case out_proj n={n_rows} in={in_f} hidden={hd}", flush=True)
    rng = np.random.Generator(np.random.PCG64(n_rows))
    hidden = workloads._normal_bf16(rng, (n_rows, hd))
    attn = workloads._normal_bf16(rng, (n_rows, in_f))
    w_o = workloads._normal_bf16(rng, (hd, in_f), std=in_f ** -0.5)
    h = bf16(hidden)
    from head_aware_paged_amd.session import SegPagedLayer
    SegPagedLayer.out_proj_residual(bf16(attn), bf16(w_o), h)
    torch.cuda.synchronize()
    _check_rounded("out_proj", bits(h), oracle.out_proj_residual(hidden, attn, w_o))


def test_out_proj_operands_beyond_32bit_offsets():
    """An attention input of more than 2^31 bytes (262,208 rows x 4,096 bf16):
    past the 32-bit offsets of a buffer load, so the output projection takes
    its general kernel; 16 sampled rows (both ends, the middle) against the
    oracle, and every row outside the input left finite."""
    n, in_f, hd = 262_208, 4096, 128
    assert n * in_f * 2 > 2 ** 31
    print(f"case out_proj n={n} in={in_f} hidden={hd} (> 2^31-byte input)", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    attn = torch.randn(n, in_f, generator=gen, device="cuda").to(torch.bfloat16)
    hidden = torch.randn(n, hd, generator=gen, device="cuda").to(torch.bfloat16)
    w_o = (torch.randn(hd, in_f, generator=gen, device="cuda") * in_f ** -0.5).to(torch.bfloat16)
    rows = np.array([0, 1, 63, 64, 1000, 65535, 131071, 131072, 200003, 262143, 262144, 262145, 262200, 262205,
                     262206, 262207])
    ri = torch.from_numpy(rows).cuda()
    h0 = bits(hidden[ri])
    a0 = bits(attn[ri])
    from head_aware_paged_amd.session import SegPagedLayer
    SegPagedLayer.out_proj_residual(attn, w_o, hidden)
    torch.cuda.synchronize()
    got = bits(hidden[ri])
    _check_rounded("out_proj > 2^31 B", got, oracle.out_proj_residual(h0, a0, bits(w_o)))
    assert bool(torch.isfinite(hidden.float()).all())


@pytest.mark.parametrize("name", ["tiny_224", "retr_mixed", "mha_g1", "mistral_32k"])
def test_layer_chain(name):
    w = workloads.mistral_32k() if name == "mistral_32k" else small(name)
    hidden_size = 4096 if name == "mistral_32k" else 256
    print(f"case {w.name}: layer chain hidden={hidden_size}", flush=True)
    hidden, w_qkv, w_o = workloads.layer_inputs(w, hidden_size, seed=3)
    layer, dev = build(w)
    q = layer.qkv_rope_append(bf16(hidden), bf16(w_qkv), w.rope_theta, dev.seg_page_indptr, dev.seg_pages,
                              dev.k_work, dev.v_work)
    out, _ = layer.attention(q, dev.k_work, dev.v_work)
    h = bf16(hidden)
    layer.out_proj_residual(out, bf16(w_o), h)
    torch.cuda.synchronize()
    ref, _ = oracle.layer(w, hidden, w_qkv, w_o)
    got = oracle.bf16_bits_to_f64(bits(h))
    d = np.abs(got - ref)
    rel = np.sqrt((d ** 2).sum() / (ref ** 2).sum())
    assert d.max() <= 3e-2 and d.mean() <= 3e-3 and rel <= 1e-2, (float(d.max()), float(d.mean()), float(rel))
