"""Seeded synthetic workloads for the SegPagedAttention prefill path.

This module only draws random numbers and lays them out in memory. It holds
none of the method's arithmetic: no RoPE, no visibility rule, no page table,
no softmax. Both the fp64 oracle (``oracle/``) and the GPU harness
(``tests/``, ``bench.py``) consume what it returns, so the two sides always see
bit-identical inputs.

Structure follows the RedKnot pages (topairepos.com README, "About" and "Key
Ideas"; paooo.com, "如何使用RedKnot"): a request's context is a run of reused
segments whose KV was cached offline at some original position, followed by the
recomputed query segment whose Q/K/V are produced online. Every (segment,
kv head) owns its own run of 16-token pages in a paged store ("SegPagedAttention
storage: per-head paged segmented KV"); the order of physical pages is a seeded
permutation, so page gathers are genuinely scattered.

Values: bf16 drawn from N(0, 1) (FFN weights from N(0, 0.02)) in fp64 with
numpy's PCG64, rounded fp64 -> fp32 -> bf16 (round-to-nearest-even at each
step; this double rounding is part of the input recipe, not of the method).
Cached K stands for K already rotated at its original positions and query K/Q
for K/Q already rotated at their new positions: a rotation of i.i.d. N(0, 1)
pairs is again i.i.d. N(0, 1), so drawing them directly has the same law as
rotating raw draws.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

PAGE = 16
GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3
CLASS_NAMES = {GLOBAL: "global", LOCAL: "local", RETRIEVAL: "retrieval", DENSE: "dense"}


def _bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 bit pattern (uint16), both steps RNE. Input recipe only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0, draw: bool = True) -> np.ndarray:
    if not draw:  # structure-only workloads: same layout, zero contents, no draws consumed
        return np.zeros(shape, dtype=np.uint16)
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 22
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        out[lo:hi] = _bf16_bits_from_f64(rng.standard_normal(hi - lo) * std)
    return out.reshape(shape)


def decode_inputs(w, seed: int = 0):
    """Inputs of one decode step: the new token of every request, at position
    L_k(r). Returns (q_new [R, Hq, D], k_new [R, Hkv, D], v_new [R, Hkv, D]),
    bf16 bit patterns drawn like the workload's own Q and K/V (standard
    normal). Input recipe only."""
    rng = np.random.Generator(np.random.PCG64(10_000 + seed))
    R, Hq, Hkv, D = w.num_requests, w.num_q_heads, w.num_kv_heads, w.head_dim
    return (_normal_bf16(rng, (R, Hq, D)), _normal_bf16(rng, (R, Hkv, D)), _normal_bf16(rng, (R, Hkv, D)))



def layer_inputs(w, hidden_size: int, seed: int = 0):
    """Inputs of one layer's projections around the attention: the query rows'
    residual stream and random-init weights. Returns bf16 bit patterns
    (hidden [T_q, hidden_size] ~ N(0, 1); w_qkv [(Hq + 2 Hkv) D, hidden_size]
    ~ N(0, 1/hidden_size); w_o [hidden_size, Hq D] ~ N(0, 1/(Hq D))), so every
    projected value has unit variance. Input recipe only."""
    rng = np.random.Generator(np.random.PCG64(20_000 + seed))
    Hq, Hkv, D, T = w.num_q_heads, w.num_kv_heads, w.head_dim, w.total_q_rows
    hidden = _normal_bf16(rng, (T, hidden_size))
    w_qkv = _normal_bf16(rng, ((Hq + 2 * Hkv) * D, hidden_size), std=hidden_size ** -0.5)
    w_o = _normal_bf16(rng, (hidden_size, Hq * D), std=(Hq * D) ** -0.5)
    return hidden, w_qkv, w_o


def stack_inputs(w, n_layers: int, hidden_size: int, inter: int, seed: int = 0):
    """Per-layer weights of a synthetic stack over w's layout: list of dicts of
    bf16 bit patterns (w_qkv, w_o as in ``layer_inputs``; w_gate, w_up
    ~ N(0, 1/hidden_size), w_down ~ N(0, 0.04/inter)), plus the query rows'
    residual stream [T_q, hidden_size] ~ N(0, 1). Input recipe only. The
    small down projection keeps the residual stream of order one through the
    layers: with no normalisation layer, SwiGLU grows with the square of
    its input, and unit-scale weights let the stream grow layer after layer."""
    rng = np.random.Generator(np.random.PCG64(30_000 + seed))
    Hq, Hkv, D, T = w.num_q_heads, w.num_kv_heads, w.head_dim, w.total_q_rows
    hidden = _normal_bf16(rng, (T, hidden_size))
    layers = []
    for _ in range(n_layers):
        layers.append(dict(
            w_qkv=_normal_bf16(rng, ((Hq + 2 * Hkv) * D, hidden_size), std=hidden_size ** -0.5),
            w_o=_normal_bf16(rng, (hidden_size, Hq * D), std=(Hq * D) ** -0.5),
            w_gate=_normal_bf16(rng, (inter, hidden_size), std=hidden_size ** -0.5),
            w_up=_normal_bf16(rng, (inter, hidden_size), std=hidden_size ** -0.5),
            w_down=_normal_bf16(rng, (hidden_size, inter), std=0.2 * inter ** -0.5)))
    return hidden, layers

@dataclasses.dataclass
class Workload:
    """One synthetic batch. Arrays holding bf16 data are uint16 bit patterns.

    Token positions are absolute within a request. Segment ``s`` of request
    ``r`` occupies ``[seg_start[s], seg_start[s] + seg_len[s])``; segments of a
    request are listed in ``[seg_indptr[r], seg_indptr[r+1])`` and the last one
    is the recomputed query segment.
    """
    name: str
    num_requests: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    rope_theta: float
    seg_indptr: np.ndarray        # int32 [R+1]
    seg_start: np.ndarray         # int32 [S]   new (insertion) start
    seg_len: np.ndarray           # int32 [S]
    seg_orig_start: np.ndarray    # int32 [S]   position the segment was cached at (query: = new start)
    head_class: np.ndarray        # int8  [R*Hkv]
    window: np.ndarray            # int32 [R*Hkv] (LOCAL only, else 0)
    retr_seg: np.ndarray          # int32 [R*Hkv*2] absolute segment ids (RETRIEVAL only, else -1)
    # working (attention) store: one page run per (segment, kv head)
    seg_page_indptr: np.ndarray   # int32 [S*Hkv+1]
    seg_pages: np.ndarray         # int32 physical page ids in the working pool
    k_work: np.ndarray            # uint16 [num_work_pages, P, D]
    v_work: np.ndarray            # uint16 [num_work_pages, P, D]
    # offline segment cache (reused segments only; query segments own no cache pages)
    cache_page_indptr: np.ndarray  # int32 [S*Hkv+1]
    cache_pages: np.ndarray       # int32 physical page ids in the cache pool
    k_cache: np.ndarray           # uint16 [num_cache_pages, P, D]
    v_cache: np.ndarray           # uint16 [num_cache_pages, P, D]
    # queries of the recomputed segment, rows of request r at cu_q[r]..cu_q[r+1]
    cu_q: np.ndarray              # int32 [R+1]
    q: np.ndarray                 # uint16 [T_q, Hq, D]
    # sparse-FFN inputs (only the FFN workload has them)
    hidden: Optional[np.ndarray] = None   # uint16 [n_tokens, hidden]
    w_gate: Optional[np.ndarray] = None   # uint16 [inter, hidden]
    w_up: Optional[np.ndarray] = None     # uint16 [inter, hidden]
    w_down: Optional[np.ndarray] = None   # uint16 [hidden, inter]
    n_last: int = 64
    topk: int = 0

    # ---- plain structural accessors (no method arithmetic) ----
    @property
    def num_segments(self) -> int:
        return int(self.seg_start.shape[0])

    def segments_of(self, r: int) -> List[int]:
        return list(range(int(self.seg_indptr[r]), int(self.seg_indptr[r + 1])))

    def query_segment(self, r: int) -> int:
        return int(self.seg_indptr[r + 1]) - 1

    def context_len(self, r: int) -> int:
        s = self.query_segment(r)
        return int(self.seg_start[s] + self.seg_len[s])

    @property
    def total_q_rows(self) -> int:
        return int(self.cu_q[-1])


def _layout(seg_lens_per_req, orig_starts_per_req, Hkv, D, rng, fill_reused_work=True, with_data=True):
    """Allocate per-(segment, kv head) page runs and draw the store contents."""
    seg_indptr = [0]
    seg_start, seg_len, seg_orig = [], [], []
    for lens, origs in zip(seg_lens_per_req, orig_starts_per_req):
        b = 0
        for n, o in zip(lens, origs):
            seg_start.append(b)
            seg_len.append(n)
            seg_orig.append(b if o is None else o)
            b += n
        seg_indptr.append(len(seg_start))
    S = len(seg_start)
    is_query = np.zeros(S, dtype=bool)
    for r in range(len(seg_indptr) - 1):
        is_query[seg_indptr[r + 1] - 1] = True

    npages = [-(-n // PAGE) for n in seg_len]
    work_counts = [npages[s] for s in range(S) for _ in range(Hkv)]
    cache_counts = [0 if is_query[s] else npages[s] for s in range(S) for _ in range(Hkv)]
    seg_page_indptr = np.concatenate([[0], np.cumsum(work_counts)]).astype(np.int32)
    cache_page_indptr = np.concatenate([[0], np.cumsum(cache_counts)]).astype(np.int32)
    n_work = int(seg_page_indptr[-1])
    n_cache = int(cache_page_indptr[-1])
    seg_pages = rng.permutation(n_work).astype(np.int32)
    cache_pages = rng.permutation(n_cache).astype(np.int32)

    # contents: cache pool for reused segments, working pool for query segments,
    # and (optionally) a stand-in for already-relocated reused K/V in the working pool
    k_cache = _normal_bf16(rng, (n_cache, PAGE, D), draw=with_data)
    v_cache = _normal_bf16(rng, (n_cache, PAGE, D), draw=with_data)
    k_work = _normal_bf16(rng, (n_work, PAGE, D), draw=with_data)
    v_work = _normal_bf16(rng, (n_work, PAGE, D), draw=with_data)
    if not fill_reused_work:
        for s in range(S):
            if is_query[s]:
                continue
            for h in range(Hkv):
                ids = seg_pages[seg_page_indptr[s * Hkv + h]:seg_page_indptr[s * Hkv + h + 1]]
                k_work[ids] = 0
                v_work[ids] = 0
    # zero the slot tails beyond a segment's last token (documented precondition)
    for s in range(S):
        tail = npages[s] * PAGE - seg_len[s]
        if tail == 0:
            continue
        for h in range(Hkv):
            for pool, ip, ids in ((k_work, seg_page_indptr, seg_pages), (v_work, seg_page_indptr, seg_pages),
                                  (k_cache, cache_page_indptr, cache_pages), (v_cache, cache_page_indptr, cache_pages)):
                run = ids[ip[s * Hkv + h]:ip[s * Hkv + h + 1]]
                if len(run):
                    pool[run[-1], PAGE - tail:, :] = 0
    return dict(
        seg_indptr=np.asarray(seg_indptr, np.int32), seg_start=np.asarray(seg_start, np.int32),
        seg_len=np.asarray(seg_len, np.int32), seg_orig_start=np.asarray(seg_orig, np.int32),
        seg_page_indptr=seg_page_indptr, seg_pages=seg_pages, k_work=k_work, v_work=v_work,
        cache_page_indptr=cache_page_indptr, cache_pages=cache_pages, k_cache=k_cache, v_cache=v_cache,
    )


def make_custom(name, *, Hq, Hkv, D, theta, seg_lens_per_req, orig_starts_per_req, classes, windows,
                retr=None, seed=0, fill_reused_work=True, rng=None, with_data=True) -> Workload:
    """Build a workload from an explicit structure.

    ``classes``/``windows`` are per (request, kv head), flattened request-major.
    ``retr`` gives, per (request, kv head), the two chosen reused-segment
    indices *local to the request* (ignored unless the class is RETRIEVAL).
    """
    rng = np.random.Generator(np.random.PCG64(seed)) if rng is None else rng
    R = len(seg_lens_per_req)
    lay = _layout(seg_lens_per_req, orig_starts_per_req, Hkv, D, rng, fill_reused_work, with_data)
    seg_indptr = lay["seg_indptr"]
    retr_abs = np.full(R * Hkv * 2, -1, np.int32)
    if retr is not None:
        for r in range(R):
            for h in range(Hkv):
                if classes[r * Hkv + h] == RETRIEVAL:
                    a, b = retr[r * Hkv + h]
                    retr_abs[(r * Hkv + h) * 2] = seg_indptr[r] + a
                    retr_abs[(r * Hkv + h) * 2 + 1] = seg_indptr[r] + b
    q_lens = [lens[-1] for lens in seg_lens_per_req]
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = _normal_bf16(rng, (int(cu_q[-1]), Hq, D), draw=with_data)
    return Workload(name=name, num_requests=R, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    page_size=PAGE, rope_theta=float(theta), head_class=np.asarray(classes, np.int8),
                    window=np.asarray(windows, np.int32), retr_seg=retr_abs, cu_q=cu_q, q=q, **lay)


# ---------------------------------------------------------------------------
# The five workloads. Readings of what the pages leave open are listed in the
# design notes; the numbers below are the concrete choices.
# ---------------------------------------------------------------------------

def tiny(seed: int = 0, window: int = 32, fill_reused_work: bool = True, with_data: bool = True) -> Workload:
    """224-token, 8 q-head / 4 kv-head, D=64 layer: 3 x 64 reused + 32 query.

    Cached segment K sits at original positions 0..63 (so the three segments
    move by 0, 64 and 128); classes per kv head are global, local(32),
    local(32), dense; RoPE theta 1e4.
    """
    return make_custom("tiny_224" if window == 32 else f"tiny_224_w{window}", Hq=8, Hkv=4, D=64, theta=1e4,
                       seg_lens_per_req=[[64, 64, 64, 32]], orig_starts_per_req=[[0, 0, 0, None]],
                       classes=[GLOBAL, LOCAL, LOCAL, DENSE], windows=[0, window, window, 0],
                       seed=seed, fill_reused_work=fill_reused_work, with_data=with_data)


def mistral_32k(seed: int = 0, fill_reused_work: bool = True, with_data: bool = True) -> Workload:
    """32K context, 32 q / 8 kv heads, D=128, theta 1e6: 16 x 2048 reused + 512 query.

    Reused segments come from random cached offsets U{0..30720}; kv head 0 is
    global, kv heads 1..7 are local with a 1024-token window.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    nseg, seglen, qlen = 16, 2048, 512
    orig = [int(x) for x in rng.integers(0, nseg * seglen - seglen + 1, size=nseg)]
    Hkv = 8
    classes = [GLOBAL] + [LOCAL] * (Hkv - 1)
    windows = [0] + [1024] * (Hkv - 1)
    return make_custom("mistral7b_32k", Hq=32, Hkv=Hkv, D=128, theta=1e6,
                       seg_lens_per_req=[[seglen] * nseg + [qlen]], orig_starts_per_req=[orig + [None]],
                       classes=classes, windows=windows, rng=rng, fill_reused_work=fill_reused_work,
                       with_data=with_data)


def qwen_varlen(seed: int = 0, fill_reused_work: bool = True, with_data: bool = True) -> Workload:
    """Varlen batch of 4 requests (8K/16K/24K/32K reused + 512 query), 64 q / 8 kv heads.

    Class quota over the 32 (request, kv head) slots by largest remainder of
    15/70/10/5 %: 5 global, 22 local(1024), 3 retrieval, 2 dense, placed by a
    seeded shuffle. Each retrieval head sees its own segment plus two distinct
    reused segments of its request drawn without replacement.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    Hkv, seglen, qlen = 8, 2048, 512
    nsegs = [4, 8, 12, 16]
    R = len(nsegs)
    slots = R * Hkv
    shares = [(GLOBAL, 0.15), (LOCAL, 0.70), (RETRIEVAL, 0.10), (DENSE, 0.05)]
    raw = [(c, f * slots) for c, f in shares]
    quota = {c: int(np.floor(x)) for c, x in raw}
    left = slots - sum(quota.values())
    for c, x in sorted(raw, key=lambda cx: -(cx[1] - np.floor(cx[1])))[:left]:
        quota[c] += 1
    pool = [c for c, _ in shares for _ in range(quota[c])]
    classes = [int(c) for c in rng.permutation(pool)]
    windows = [1024 if c == LOCAL else 0 for c in classes]
    orig_all, retr = [], []
    for r, ns in enumerate(nsegs):
        lreused = ns * seglen
        orig_all.append([int(x) for x in rng.integers(0, lreused - seglen + 1, size=ns)] + [None])
    for r, ns in enumerate(nsegs):
        for h in range(Hkv):
            pick = rng.choice(ns, size=2, replace=False)
            retr.append((int(pick[0]), int(pick[1])))
    return make_custom("qwen3_32b_varlen", Hq=64, Hkv=Hkv, D=128, theta=1e6,
                       seg_lens_per_req=[[seglen] * ns + [qlen] for ns in nsegs],
                       orig_starts_per_req=orig_all, classes=classes, windows=windows, retr=retr,
                       rng=rng, fill_reused_work=fill_reused_work, with_data=with_data)


def long_64k(seed: int = 0, fill_reused_work: bool = True, with_data: bool = True) -> Workload:
    """64K context, 32 q / 4 kv heads, D=128: 32 x 2048 reused + 1024 query.

    kv head 0 global, kv heads 1..3 local with a 2048-token window; reused
    segments come from random cached offsets.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    nseg, seglen, qlen = 32, 2048, 1024
    orig = [int(x) for x in rng.integers(0, nseg * seglen - seglen + 1, size=nseg)]
    Hkv = 4
    return make_custom("long_64k", Hq=32, Hkv=Hkv, D=128, theta=1e6,
                       seg_lens_per_req=[[seglen] * nseg + [qlen]], orig_starts_per_req=[orig + [None]],
                       classes=[GLOBAL] + [LOCAL] * 3, windows=[0] + [2048] * 3, rng=rng,
                       fill_reused_work=fill_reused_work, with_data=with_data)


def sparse_ffn_8k(seed: int = 0, hidden: int = 4096, inter: int = 14336, n_tokens: int = 8192,
                  n_last: int = 64, with_ffn: bool = True, with_data: bool = True) -> Workload:
    """8K dense-causal context, 32 q / 8 kv heads, D=128, Q only for the last 64 rows.

    Hidden states [8192, 4096] ~ N(0, 1); SwiGLU weights (gate/up [14336, 4096],
    down [4096, 14336]) ~ N(0, 0.02); k = 25% of the context.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    Hkv = 8
    w = make_custom("sparse_ffn_8k", Hq=32, Hkv=Hkv, D=128, theta=1e6,
                    seg_lens_per_req=[[n_tokens - n_last, n_last]], orig_starts_per_req=[[None, None]],
                    classes=[DENSE] * Hkv, windows=[0] * Hkv, rng=rng, with_data=with_data)
    w.n_last = n_last
    w.topk = n_tokens // 4
    if with_ffn:
        w.hidden = _normal_bf16(rng, (n_tokens, hidden), draw=with_data)
        w.w_gate = _normal_bf16(rng, (inter, hidden), 0.02, draw=with_data)
        w.w_up = _normal_bf16(rng, (inter, hidden), 0.02, draw=with_data)
        w.w_down = _normal_bf16(rng, (hidden, inter), 0.02, draw=with_data)
    return w


def ffn_only(seed: int = 0, n_tokens: int = 64, hidden: int = 256, inter: int = 512):
    """Small hidden/weight draw for FFN-only cases (same recipe as the 8K workload)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return dict(hidden=_normal_bf16(rng, (n_tokens, hidden)),
                w_gate=_normal_bf16(rng, (inter, hidden), 0.02),
                w_up=_normal_bf16(rng, (inter, hidden), 0.02),
                w_down=_normal_bf16(rng, (hidden, inter), 0.02))


def uniform_f32(seed: int, n: int, lo: float = 0.0, hi: float = 1.0, levels: int = 0) -> np.ndarray:
    """Random non-negative fp32 scores; ``levels > 0`` quantises them to force exact ties."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if levels > 0:
        return (rng.integers(0, levels, size=n).astype(np.float32) / np.float32(levels)).astype(np.float32)
    return rng.uniform(lo, hi, size=n).astype(np.float32)


CONFIGS = {
    "tiny_224": tiny,
    "mistral7b_32k": mistral_32k,
    "qwen3_32b_varlen": qwen_varlen,
    "long_64k": long_64k,
    "sparse_ffn_8k": sparse_ffn_8k,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)
