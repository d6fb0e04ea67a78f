"""Per-head visible key sets, page tables, spans and relocation move lists.

Pages: RedKnot README (topairepos.com), "About" (each (layer, kv_head) is one
of global / local / retrieval / dense; the SegPagedAttention runtime gives
each head class its own visible window through a per-head page table);
aitrends.kr "주요 기능" (per-class visible windows, only needed pages loaded);
paooo.com "如何使用RedKnot" (SELECTVISIBLESTATE picks the reused local-head KV
and the global-head ranges).

Readings (the pages fix no formula):
  * query row t of request r sits at absolute position i = b_q + t, where
    [b_q, b_q + Lq) is the request's last (recomputed) segment;
  * GLOBAL and DENSE see every key j <= i (causal);
  * LOCAL(W) sees its own segment causally plus a W-token causal sliding
    window that includes the row itself: {b_q <= j <= i} U {i-W+1 <= j <= i};
  * RETRIEVAL(S) sees its own segment causally plus the two chosen reused
    segments in full: {b_q <= j <= i} U [b_s, b_s + n_s) for s in S.
Two independent routines evaluate this: a per-index predicate
(``visible_brute``) and interval arithmetic (``visible_intervals``); tests
check that they agree.
"""
import numpy as np

GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3


def _head(w, r, h):
    k = r * w.num_kv_heads + h
    return int(w.head_class[k]), int(w.window[k]), [int(x) for x in w.retr_seg[2 * k:2 * k + 2]]


def visible_brute(w, r, h, i):
    """Sorted list of visible key positions for the row at position i, by predicate."""
    cls, W, retr = _head(w, r, h)
    sq = w.query_segment(r)
    bq = int(w.seg_start[sq])
    out = []
    for j in range(w.context_len(r)):
        own = bq <= j <= i
        if cls in (GLOBAL, DENSE):
            ok = j <= i
        elif cls == LOCAL:
            ok = own or (i - W + 1 <= j <= i)
        elif cls == RETRIEVAL:
            ok = own or any(int(w.seg_start[s]) <= j < int(w.seg_start[s] + w.seg_len[s]) for s in retr)
        else:
            raise ValueError(cls)
        if ok:
            out.append(j)
    return out


def visible_intervals(w, r, h, i):
    """Visible set of the row at position i as sorted, merged half-open intervals."""
    cls, W, retr = _head(w, r, h)
    bq = int(w.seg_start[w.query_segment(r)])
    if cls in (GLOBAL, DENSE):
        ivs = [(0, i + 1)]
    elif cls == LOCAL:
        ivs = [(max(0, min(bq, i - W + 1)), i + 1)]
    elif cls == RETRIEVAL:
        ivs = [(bq, i + 1)] + [(int(w.seg_start[s]), int(w.seg_start[s] + w.seg_len[s])) for s in retr]
    else:
        raise ValueError(cls)
    ivs.sort()
    merged = []
    for lo, hi in ivs:
        if merged and lo <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], hi))
        else:
            merged.append((lo, hi))
    return merged


def visible_count(w, r, h, i):
    return sum(hi - lo for lo, hi in visible_intervals(w, r, h, i))


def _logical_pages(w, r, h):
    """Logical pages that hold at least one key visible to some query row."""
    P = w.page_size
    sq = w.query_segment(r)
    bq, lq = int(w.seg_start[sq]), int(w.seg_len[sq])
    ivs = sorted(iv for t in range(lq) for iv in visible_intervals(w, r, h, bq + t))
    union = []
    for lo, hi in ivs:
        if union and lo <= union[-1][1]:
            union[-1] = (union[-1][0], max(union[-1][1], hi))
        else:
            union.append((lo, hi))
    pages = set()
    for lo, hi in union:
        pages.update(range(lo // P, (hi - 1) // P + 1))
    return sorted(pages)


def _physical(w, r, h, p):
    """Physical working page of logical page p of request r, kv head h."""
    P, Hkv = w.page_size, w.num_kv_heads
    for s in w.segments_of(r):
        b, n = int(w.seg_start[s]), int(w.seg_len[s])
        if b <= p * P < b + n:
            return s, int(w.seg_pages[w.seg_page_indptr[s * Hkv + h] + (p * P - b) // P])
    raise ValueError("page outside the context")


def page_table(w, r, h):
    """(physical page ids, logical start positions) of every page holding a key
    visible to at least one query row of (r, h), in ascending position order."""
    lp = _logical_pages(w, r, h)
    return (np.array([_physical(w, r, h, p)[1] for p in lp], np.int32),
            np.array([p * w.page_size for p in lp], np.int32))


def page_tables(w):
    """CSR over (request, kv head): (indptr, page_ids, page_pos)."""
    indptr, ids, pos = [0], [], []
    for r in range(w.num_requests):
        for h in range(w.num_kv_heads):
            a, b = page_table(w, r, h)
            ids.append(a)
            pos.append(b)
            indptr.append(indptr[-1] + len(a))
    return (np.array(indptr, np.int32), np.concatenate(ids).astype(np.int32),
            np.concatenate(pos).astype(np.int32))


def visible_spans(w, max_spans=3):
    """[T_q, Hkv, 3, 2] int32: each row's visible intervals, padded with (-1, -1)."""
    out = np.full((w.total_q_rows, w.num_kv_heads, max_spans, 2), -1, np.int32)
    for r in range(w.num_requests):
        sq = w.query_segment(r)
        bq, lq = int(w.seg_start[sq]), int(w.seg_len[sq])
        for t in range(lq):
            row = int(w.cu_q[r]) + t
            for h in range(w.num_kv_heads):
                for k, iv in enumerate(visible_intervals(w, r, h, bq + t)):
                    out[row, h, k] = iv
    return out


def move_list(w):
    """Head-aware relocation moves: for each (r, h) in order and each table page
    that lies in a reused segment, (cache page, working page, delta = b_s - o_s).
    Only pages some row of that head can see are moved."""
    P, Hkv = w.page_size, w.num_kv_heads
    src, dst, delta = [], [], []
    for r in range(w.num_requests):
        sq = w.query_segment(r)
        for h in range(Hkv):
            for p in _logical_pages(w, r, h):
                s, phys = _physical(w, r, h, p)
                if s == sq:
                    continue
                q = (p * P - int(w.seg_start[s])) // P
                src.append(int(w.cache_pages[w.cache_page_indptr[s * Hkv + h] + q]))
                dst.append(phys)
                delta.append(int(w.seg_start[s]) - int(w.seg_orig_start[s]))
    return np.array(src, np.int32), np.array(dst, np.int32), np.array(delta, np.int32)
