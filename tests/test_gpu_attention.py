"""GPU: SegPagedAttention prefill vs the fp64 oracle, plus visibility probes.

Tolerances: max |O - O_ref| <= 2e-2 and mean <= 2e-3 on the bf16 output (fp32
accumulate); LSE within 1e-3; per-head relative Frobenius error <= 1e-2 (at
32K+ contexts |O| is ~0.01, so the absolute bounds alone would be weak).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Dev, assert_attn_close, bf16, bits, build, v_pages

pytestmark = pytest.mark.gpu

G_, L_, R_, D_ = workloads.GLOBAL, workloads.LOCAL, workloads.RETRIEVAL, workloads.DENSE


def small_variants():
    yield workloads.tiny()
    yield workloads.tiny(window=8)
    yield workloads.make_custom("retr_mixed", Hq=4, Hkv=4, D=64, theta=1e4,
                                seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                                orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                                classes=[R_, L_, G_, R_, D_, L_, R_, G_], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                                retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])
    yield workloads.make_custom("ragged_g8", Hq=16, Hkv=2, D=128, theta=1e6,
                                seg_lens_per_req=[[256, 128, 77], [32, 300]],
                                orig_starts_per_req=[[1000, 3, None], [17, None]],
                                classes=[L_, G_, G_, L_], windows=[100, 0, 0, 1])
    yield workloads.make_custom("g4_d128_q512", Hq=16, Hkv=4, D=128, theta=1e6,
                                seg_lens_per_req=[[2048, 2048, 512]], orig_starts_per_req=[[0, 0, None]],
                                classes=[G_, L_, R_, D_], windows=[0, 1024, 0, 0], retr=[None, None, (1, 0), None])
    yield workloads.make_custom("mha_g1", Hq=3, Hkv=3, D=64, theta=1e4,
                                seg_lens_per_req=[[160, 200]], orig_starts_per_req=[[0, None]],
                                classes=[G_, L_, D_], windows=[0, 64, 0])
    # 18 requests x 4 kv heads: more than 64 (request, kv head) pairs and m-tiles,
    # so the planning sums take their multi-wave path
    nreq = 18
    yield workloads.make_custom("many_req", Hq=8, Hkv=4, D=64, theta=1e4,
                                seg_lens_per_req=[[48 + 16 * (r % 4), 30 + 11 * (r % 5)] for r in range(nreq)],
                                orig_starts_per_req=[[3 * r, None] for r in range(nreq)],
                                classes=[(G_, L_, D_, L_)[(r + h) % 4] for r in range(nreq) for h in range(4)],
                                windows=[(0, 24, 0, 9)[(r + h) % 4] for r in range(nreq) for h in range(4)])


SMALL_NAMES = [w.name for w in small_variants()]


def small(name):
    """A fresh copy of a small variant (tests mutate their inputs)."""
    return next(w for w in small_variants() if w.name == name)


def run_attn(w, dev=None, layer=None):
    if layer is None:
        layer, dev = build(w, dev)
    out, lse = layer.attention(dev.q, dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    return bits(out), lse.cpu().numpy(), layer, dev


@pytest.mark.parametrize("name", SMALL_NAMES)
def test_small_vs_oracle(name):
    w = small(name)
    print(f"case {w.name}: attention", flush=True)
    ob, lse, layer, dev = run_attn(w)
    O, L = oracle.attention(w)
    assert_attn_close(ob, lse, O, L, name=w.name)
    # deterministic: a second run is bit-identical
    out2, lse2 = layer.attention(dev.q, dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out2), ob) and np.array_equal(lse2.cpu().numpy(), lse)


@pytest.mark.parametrize("name", SMALL_NAMES[:4])
def test_zero_q_counts_visible_keys(name):
    w = small(name)
    # Q = 0: every visible score is 0, so exp(LSE) is exactly the visible-key count.
    print(f"case {w.name}: Q=0 count probe", flush=True)
    w.q[:] = 0
    _, lse, _, _ = run_attn(w)
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            row = int(w.cu_q[r]) + t
            for g in range(w.num_q_heads):
                n = oracle.visible_count(w, r, g // G, bq + t)
                assert int(round(float(np.exp(np.float64(lse[row, g]))))) == n, (row, g)


@pytest.mark.parametrize("name", SMALL_NAMES[:4])
def test_constant_v(name):
    w = small(name)
    print(f"case {w.name}: constant V", flush=True)
    w.v_work[:] = np.uint16(0x3FC0)   # 1.5
    ob, _, _, _ = run_attn(w)
    O = oracle.bf16_bits_to_f64(ob)
    assert np.all(np.abs(O - 1.5) <= 2.0 ** -7)


@pytest.mark.parametrize("name", SMALL_NAMES[:4])
def test_pages_outside_tables_are_never_read(name):
    w = small(name)
    # Poison every working page that is not in its head's table with NaN: the
    # output must be bit-identical to the clean run.
    print(f"case {w.name}: NaN-poisoned pages outside the tables", flush=True)
    ob, lse, _, _ = run_attn(w)
    used = set()
    for r in range(w.num_requests):
        for h in range(w.num_kv_heads):
            used.update(int(x) for x in oracle.page_table(w, r, h)[0])
    unused = np.array(sorted(set(range(w.k_work.shape[0])) - used), dtype=np.int64)
    assert len(unused) > 0
    wk, wv = w.k_work.copy(), w.v_work.copy()
    wk[unused] = 0x7FC0
    wv[unused] = 0x7FC0
    dev = Dev(w)
    dev.k_work, dev.v_work = bf16(wk), bf16(v_pages(wv))
    ob2, lse2, _, _ = run_attn(w, dev)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(ob2)))
    assert np.array_equal(ob2, ob) and np.array_equal(lse2, lse)


def test_sentinel_keys_at_window_edges():
    # Keys aligned with a row's query (score ~ +30) planted just outside and
    # just inside the visible boundaries of LOCAL and RETRIEVAL heads.
    w = small("retr_mixed")  # retrieval, local, global, dense heads over two requests
    print("case retr_mixed: sentinel keys", flush=True)
    P, Hkv, D = 16, w.num_kv_heads, w.head_dim
    kf = oracle.bf16_bits_to_f64(w.k_work)

    def plant(r, h, j, qvec):
        for s in w.segments_of(r):
            b = int(w.seg_start[s])
            if b <= j < b + int(w.seg_len[s]):
                pid = w.seg_pages[w.seg_page_indptr[s * Hkv + h] + (j - b) // P]
                alpha = 30.0 * np.sqrt(D) / float(qvec @ qvec)
                w.k_work[pid, (j - b) % P] = oracle.f64_to_bf16_bits(alpha * qvec)
                w.v_work[pid, (j - b) % P] = oracle.f64_to_bf16_bits(np.full(D, 0.5))

    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        Lq = int(w.cu_q[r + 1] - w.cu_q[r])
        t = Lq // 2
        i = bq + t
        row = int(w.cu_q[r]) + t
        for h in range(Hkv):
            qv = oracle.bf16_bits_to_f64(w.q[row, h])
            ivs = oracle.visible_intervals(w, r, h, i)
            for lo, hi in ivs:
                for j in (lo - 1, lo, hi - 1, hi):
                    if 0 <= j < w.context_len(r) and j != i:
                        plant(r, h, j, qv)
    ob, lse, _, _ = run_attn(w)
    O, L = oracle.attention(w)
    assert_attn_close(ob, lse, O, L, name="sentinels")


def _plant_aligned_key(w, r, h, j, qvec, score):
    """Key j of (request r, kv head h) := a multiple of qvec whose scaled score
    against qvec is `score`; its V row := 0.5."""
    P, Hkv, D = w.page_size, w.num_kv_heads, w.head_dim
    for s in w.segments_of(r):
        b = int(w.seg_start[s])
        if b <= j < b + int(w.seg_len[s]):
            pid = w.seg_pages[w.seg_page_indptr[s * Hkv + h] + (j - b) // P]
            alpha = score * np.sqrt(D) / float(qvec @ qvec)
            w.k_work[pid, (j - b) % P] = oracle.f64_to_bf16_bits(alpha * qvec)
            w.v_work[pid, (j - b) % P] = oracle.f64_to_bf16_bits(np.full(D, 0.5))
            return
    raise AssertionError((r, h, j))


@pytest.mark.parametrize("score", [35.0, 100.0])
@pytest.mark.parametrize("name", ["g4_d128_q512", "ragged_g8"])
def test_late_score_jump(name, score):
    # A key near the end of a row's visible range whose score stands `score`
    # above the row's typical scores (which are O(1)): 35 stays within the
    # growth a single pass allows over the row's first running max, 100 (about
    # 2^140 in probability) exceeds it and takes the exact-max pass. Both must
    # match the oracle, and nothing may overflow.
    w = small(name)
    print(f"case {w.name}: late score jump {score}", flush=True)
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        Lq = int(w.cu_q[r + 1] - w.cu_q[r])
        for t in sorted({Lq - 1, Lq // 2}):
            i, row = bq + t, int(w.cu_q[r]) + t
            for h in range(w.num_kv_heads):
                ivs = oracle.visible_intervals(w, r, h, i)
                cached = [hi - 1 for lo, hi in ivs if hi - 1 < bq] + [bq - 1 for lo, hi in ivs if lo < bq <= hi - 1]
                j = max(cached) if cached else i - 1
                if j < 0:
                    continue
                _plant_aligned_key(w, r, h, j, oracle.bf16_bits_to_f64(w.q[row, h * G]), score)
    ob, lse, _, _ = run_attn(w)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(ob))) and np.all(np.isfinite(lse))
    O, L = oracle.attention(w)
    assert_attn_close(ob, lse, O, L, name=f"{w.name}+jump{score:g}")


@pytest.mark.parametrize("name", ["mistral7b_32k", "qwen3_32b_varlen", "long_64k"])
def test_full_size_all_rows(name):
    """Every query row and head of the full-size layouts against the oracle
    (every m-tile and every split-KV chunk is compared element-wise)."""
    w = workloads.make(name)
    print(f"case {name}: attention at full size, all rows", flush=True)
    ob, lse, layer, dev = run_attn(w)
    O, L = oracle.attention(w)
    assert_attn_close(ob, lse, O, L, name=name)
    out2, lse2 = layer.attention(dev.q, dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out2), ob)


@pytest.mark.parametrize("name", ["mistral7b_32k", "long_64k"])
def test_full_size_zero_q_counts_visible_keys(name):
    """Q = 0 at full size: every visible score is 0, so exp(LSE) equals each
    row's visible-key count exactly (the fp32 row sum of ones is exact below
    2^24), and O is the mean of the visible V rows."""
    w = workloads.make(name)
    w.q[:] = 0
    print(f"case {name}: Q=0 count probe at full size", flush=True)
    _, lse, _, _ = run_attn(w)
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            row = int(w.cu_q[r]) + t
            n = np.array([oracle.visible_count(w, r, h, bq + t) for h in range(w.num_kv_heads)], np.float64)
            got = lse[row].astype(np.float64)
            assert np.all(np.abs(got - np.log(np.repeat(n, G))) <= 1e-5 * np.log(np.repeat(n, G)) + 1e-6), row


def test_items_longer_than_the_table_ring():
    """4096 query rows, 64 q heads over 8 global kv heads, 36,864 keys: 1024
    m-tiles, so the plan splits none and each item walks its whole m-tile,
    up to 576 key tiles, refilling its 256-tile LDS table ring twice. Q = 0
    probes every row (exp(LSE) = position + 1); the real Q is compared with
    the oracle on rows spread over the m-tiles."""
    w = workloads.make_custom("ring_576", Hq=64, Hkv=8, D=128, theta=1e6,
                              seg_lens_per_req=[[16384, 16384, 4096]], orig_starts_per_req=[[0, 0, None]],
                              classes=[G_] * 8, windows=[0] * 8)
    print(f"case {w.name}: items of up to 576 tiles", flush=True)
    layer, dev = build(w)
    assert layer.sizes["attn_workspace_bytes"] == 0  # no item is split
    rows = list(range(0, 4096, 61)) + [4095]
    out, lse = layer.attention(dev.q, dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    O, L = oracle.attention(w, rows=rows)
    assert_attn_close(bits(out), lse.cpu().numpy(), O, L, rows=rows, name=w.name)
    _, lse0 = layer.attention(torch.zeros_like(dev.q), dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    pos = 32768 + np.arange(4096, dtype=np.float64)
    assert np.all(np.abs(lse0.cpu().numpy().astype(np.float64) - np.log(pos + 1)[:, None]) <= 1e-5 * np.log(pos + 1)[:, None])


@pytest.mark.parametrize("make", [workloads.tiny, workloads.mistral_32k], ids=["tiny_224", "mistral7b_32k"])
def test_relocate_then_attend(make):
    """BUILDSTATE relocation (head-aware moves) followed by EXECUTE attention;
    the oracle relocates in fp64 and stores bf16 (the working pool's format)."""
    w = make(fill_reused_work=False)
    print(f"case {w.name}: relocate -> attention", flush=True)
    layer, dev = build(w)
    layer.relocate(dev.k_cache, dev.k_work, dev.v_cache, dev.v_work, w.rope_theta)
    out, lse = layer.attention(dev.q, dev.k_work, dev.v_work)
    torch.cuda.synchronize()
    # oracle working pool: every reused page relocated in fp64, rounded once to bf16
    k_ref, v_ref = w.k_work.copy(), w.v_work.copy()
    Hkv = w.num_kv_heads
    for r in range(w.num_requests):
        for s in w.segments_of(r)[:-1]:
            delta = int(w.seg_start[s] - w.seg_orig_start[s])
            for h in range(Hkv):
                cp = w.cache_pages[w.cache_page_indptr[s * Hkv + h]:w.cache_page_indptr[s * Hkv + h + 1]]
                wp = w.seg_pages[w.seg_page_indptr[s * Hkv + h]:w.seg_page_indptr[s * Hkv + h + 1]]
                k_ref[wp] = oracle.f64_to_bf16_bits(
                    oracle.relocate(oracle.bf16_bits_to_f64(w.k_cache[cp]), delta, w.rope_theta))
                v_ref[wp] = w.v_cache[cp]
    O, L = oracle.attention(w, k_pool=k_ref, v_pool=v_ref)
    assert_attn_close(bits(out), lse.cpu().numpy(), O, L, name=w.name + "+relocate")
