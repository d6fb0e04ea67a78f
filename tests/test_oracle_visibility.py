"""Pins for visible sets, page tables, spans and move lists (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from conftest import GOLDEN

GOLD = json.load(open(os.path.join(GOLDEN, "visible_pairs.json")))


def _total_pairs(w):
    G = w.num_q_heads // w.num_kv_heads
    tot = 0
    for r in range(w.num_requests):
        bq = int(w.seg_start[w.query_segment(r)])
        for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
            for h in range(w.num_kv_heads):
                tot += G * oracle.visible_count(w, r, h, bq + t)
    return tot


def _variants():
    yield workloads.tiny()
    yield workloads.tiny(window=8)
    yield workloads.make_custom("tiny_retr", Hq=4, Hkv=4, D=64, theta=1e4,
                                seg_lens_per_req=[[64, 32, 48, 64, 27], [16, 16, 16]],
                                orig_starts_per_req=[[5, 0, 100, 3, None], [0, 40, None]],
                                classes=[2, 1, 0, 2, 3, 1, 2, 0], windows=[0, 40, 0, 0, 0, 5, 0, 0],
                                retr=[(2, 0), None, None, (1, 3), None, None, (0, 1), None])


def test_brute_and_interval_visibility_agree():
    for w in _variants():
        for r in range(w.num_requests):
            bq = int(w.seg_start[w.query_segment(r)])
            for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
                for h in range(w.num_kv_heads):
                    i = bq + t
                    ivs = oracle.visible_intervals(w, r, h, i)
                    flat = [j for lo, hi in ivs for j in range(lo, hi)]
                    assert flat == oracle.visible_brute(w, r, h, i)
                    # intervals are maximal: sorted, disjoint and non-adjacent
                    for (a0, a1), (b0, b1) in zip(ivs, ivs[1:]):
                        assert a1 < b0


def test_closed_form_row_counts():
    w = workloads.tiny(window=8)
    bq = 192
    for t in range(32):
        i = bq + t
        assert oracle.visible_count(w, 0, 0, i) == i + 1
        assert oracle.visible_count(w, 0, 3, i) == i + 1
        assert oracle.visible_count(w, 0, 1, i) == i - max(0, min(bq, i - 8 + 1)) + 1


@pytest.mark.parametrize("name,key", [("tiny_224", "tiny_224"), ("mistral7b_32k", "mistral7b_32k"),
                                      ("long_64k", "long_64k")])
def test_visible_pair_totals_golden(name, key):
    w = workloads.make(name, with_data=False)
    assert _total_pairs(w) == GOLD[key]["visible_pairs"]
    indptr, _, _ = oracle.page_tables(w)
    assert list(np.diff(indptr)) == GOLD[key]["table_sizes"]


def test_tiny_w8_golden():
    w = workloads.tiny(window=8)
    assert _total_pairs(w) == GOLD["tiny_224_w8"]["visible_pairs"]
    indptr, _, _ = oracle.page_tables(w)
    assert list(np.diff(indptr)) == GOLD["tiny_224_w8"]["table_sizes"]


def test_varlen_per_class_counts_golden():
    w = workloads.qwen_varlen(with_data=False)
    g = GOLD["qwen3_32b_varlen_per_q_head"]
    seen = set()
    for r in range(4):
        bq = int(w.seg_start[w.query_segment(r)])
        for h in range(8):
            cls = int(w.head_class[r * 8 + h])
            tot = sum(oracle.visible_count(w, r, h, bq + t) for t in range(512))
            exp = {0: g["global_dense"][r], 3: g["global_dense"][r], 1: g["local"], 2: g["retrieval"]}[cls]
            assert tot == exp
            seen.add(cls)
    assert seen == {0, 1, 2, 3}
    assert sorted(np.bincount(w.head_class, minlength=4)) == sorted([5, 22, 3, 2])


def test_page_table_brute_force():
    # The table is exactly the pages holding a key some row sees (brute force),
    # ascending, mapped through the per-(segment, head) page runs.
    for w in _variants():
        for r in range(w.num_requests):
            bq = int(w.seg_start[w.query_segment(r)])
            for h in range(w.num_kv_heads):
                keys = set()
                for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
                    keys.update(oracle.visible_brute(w, r, h, bq + t))
                pages = sorted({j // 16 for j in keys})
                ids, pos = oracle.page_table(w, r, h)
                assert list(pos) == [16 * p for p in pages]
                for p, pid in zip(pages, ids):
                    # the physical page must be the one the store lists for that token
                    hits = []
                    for s in w.segments_of(r):
                        b = int(w.seg_start[s])
                        if b <= 16 * p < b + int(w.seg_len[s]):
                            hits.append(int(w.seg_pages[w.seg_page_indptr[s * w.num_kv_heads + h] + (16 * p - b) // 16]))
                    assert hits == [pid]


def test_spans_and_moves():
    w = workloads.tiny()
    sp = oracle.visible_spans(w)
    assert sp.shape == (32, 4, 3, 2)
    assert tuple(sp[0, 0, 0]) == (0, 193) and tuple(sp[0, 0, 1]) == (-1, -1)
    assert tuple(sp[0, 1, 0]) == (161, 193)
    src, dst, delta = oracle.move_list(w)
    # global/dense heads move all 12 reused pages, local heads the 2 pages of [160, 192)
    assert len(src) == 12 + 2 + 2 + 12
    assert sorted(set(delta.tolist())) == [0, 64, 128]
    w3 = next(v for v in _variants() if v.name == "tiny_retr")
    sp3 = oracle.visible_spans(w3)
    # request 0, head 0 is RETRIEVAL over segments 2 ([96,144)) and 0 ([0,64)); query at 208
    assert [tuple(x) for x in sp3[0, 0]] == [(0, 64), (96, 144), (208, 209)]
    # request 1 head 2: retrieval of both reused segments [0,16) and [16,32), query at 32 -> one span
    assert [tuple(x) for x in sp3[27, 2]] == [(0, 33), (-1, -1), (-1, -1)]


def _moves_by_token_walk(w):
    """Head-aware moves rebuilt from scratch by walking every visible token:
    for each (r, h) in order, every key some query row sees (per-index
    predicate) that lies in a reused segment names its page; that page's cache
    copy moves to its working copy, shifted by the segment's delta. Pages are
    listed once, in ascending position."""
    P, Hkv = w.page_size, w.num_kv_heads
    src, dst, delta = [], [], []
    for r in range(w.num_requests):
        sq = w.query_segment(r)
        bq = int(w.seg_start[sq])
        for h in range(Hkv):
            keys = set()
            for t in range(int(w.cu_q[r + 1] - w.cu_q[r])):
                keys.update(oracle.visible_brute(w, r, h, bq + t))
            seen = set()
            for j in sorted(keys):
                s = next(s for s in w.segments_of(r)
                         if int(w.seg_start[s]) <= j < int(w.seg_start[s]) + int(w.seg_len[s]))
                if s == sq or j // P in seen:
                    continue
                seen.add(j // P)
                qp = (j - int(w.seg_start[s])) // P
                src.append(int(w.cache_pages[w.cache_page_indptr[s * Hkv + h] + qp]))
                dst.append(int(w.seg_pages[w.seg_page_indptr[s * Hkv + h] + qp]))
                delta.append(int(w.seg_start[s]) - int(w.seg_orig_start[s]))
    return src, dst, delta


def test_move_list_token_walk():
    # RedKnot README "About" (per-head page tables) and paooo.com "如何使用RedKnot"
    # (SELECTVISIBLESTATE: only the KV a head can see is reused and relocated):
    # every (cache page, working page, delta) triple is the one the token walk
    # names, in the same order; the variants cover negative deltas (original
    # starts past the new ones), retrieval heads, windows that cut a segment and
    # two requests.
    for w in _variants():
        src, dst, delta = oracle.move_list(w)
        s2, d2, dl2 = _moves_by_token_walk(w)
        assert list(src) == s2 and list(dst) == d2 and list(delta) == dl2, w.name
    w3 = next(v for v in _variants() if v.name == "tiny_retr")
    assert min(oracle.move_list(w3)[2]) < 0
