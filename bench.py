#!/usr/bin/env python3
"""SegPagedAttention prefill benchmark on one MI355X.

One step is one pass of the whole SegPaged prefill path over the 32K-context,
Mistral-7B-shaped layer (32 q heads, 8 kv heads, D=128, 16 reused 2K segments
+ a 512-token query segment; kv head 0 global, 1..7 local with a 1024 window):
  1. segkv_build_pages     per-head page tables, head-aware move list, plan
  2. rope_relocate         head-aware moves: cached K rotated + V gathered
  3. segpaged_attn_prefill attention over the visible pages (+ split merge)
  4. token_importance_topk importance over the last 64 rows, top 25% of keys
`value` is the visible-pair attention FLOPs (4 * D * sum of visible keys over
every (query head, row)) per second of whole-step time. The line also carries
the attention call's own rate against the bf16 MFMA peak (roofline), the full
relocation's HBM bandwidth, the sparse FFN of the 8K selection workload, and
the fp64 oracle timed on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs_per_row(w):
    """Per query row: visible keys summed over query heads (closed form per class)."""
    import numpy as np
    G = w.num_q_heads // w.num_kv_heads
    out = np.zeros(w.total_q_rows, dtype=np.int64)
    for r in range(w.num_requests):
        sq = w.query_segment(r)
        bq, lq = int(w.seg_start[sq]), int(w.seg_len[sq])
        i = np.arange(bq, bq + lq, dtype=np.int64)
        for h in range(w.num_kv_heads):
            k = r * w.num_kv_heads + h
            c = int(w.head_class[k])
            if c in (0, 3):
                n = i + 1
            elif c == 1:
                n = i - np.maximum(0, np.minimum(bq, i - int(w.window[k]) + 1)) + 1
            else:
                segs = [int(s) for s in w.retr_seg[2 * k:2 * k + 2]]
                n = (i - bq + 1) + sum(int(w.seg_len[s]) for s in segs)
            out[int(w.cu_q[r]):int(w.cu_q[r + 1])] += G * n
    return out


def decode_visible_pages(w):
    """Pages holding a key visible to the decode row (position L_k) of each (r, h): the
    same closed forms per class, at i = L_k, over the stored keys [0, L_k)."""
    total = 0
    for r in range(w.num_requests):
        sq = w.query_segment(r)
        bq, Lk = int(w.seg_start[sq]), w.context_len(r)
        for h in range(w.num_kv_heads):
            k = r * w.num_kv_heads + h
            c = int(w.head_class[k])
            if c in (0, 3):
                ivs = [(0, Lk)]
            elif c == 1:
                ivs = [(max(0, min(bq, Lk - int(w.window[k]) + 1)), Lk)]
            else:
                segs = [int(s) for s in w.retr_seg[2 * k:2 * k + 2]]
                ivs = [(bq, Lk)] + [(int(w.seg_start[s]), int(w.seg_start[s] + w.seg_len[s])) for s in segs]
            pages = set()
            for lo, hi in ivs:
                pages.update(range(lo // 16, (hi + 15) // 16))
            total += len(pages)
    return total


def profile_traffic(kernel_tag, src_hash):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("|") and ":" not in line.split("|")[1]:
            continue
        if line.startswith("- ") and "=" in line:
            k, v = line[2:].split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != src_hash or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def source_hash(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "head_aware_paged_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(w, pairs_per_row, min_seconds):
    """The fp64 oracle on the same workload: whole passes over every query row
    (all heads) until at least min_seconds of host time have been spent, with
    the BLAS pool set to the cores this process may run on (capped by
    OMP_NUM_THREADS, the job's share of the host, when that is set)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(affinity, share) if share > 0 else affinity
    blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    vendor = ",".join(sorted({f"{d.get('internal_api')} {d.get('version')}" for d in blas})) or "unknown"
    passes, dt = 0, 0.0
    with threadpool_limits(limits=threads, user_api="blas"):
        used = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
        while passes == 0 or dt < min_seconds:
            t0 = time.perf_counter()
            oracle.attention(w)
            dt += time.perf_counter() - t0
            passes += 1
    flops = 4.0 * w.head_dim * float(pairs_per_row.sum()) * passes
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(used), "affinity_cores": affinity,
            "blas": vendor, "kind": "oracle",
            "sample": f"fp64 oracle attention (explicit per-head masks) over all {w.total_q_rows} query rows x "
                      f"{w.num_q_heads} q heads of {w.name}, {passes} pass(es): {flops / 1e9:.1f} GFLOP of "
                      f"visible pairs in {dt:.1f} s"}


def relocation_bandwidth(w, dev, i32, k_only=False, reps=20):
    """rope_relocate on a workload's structure: every reused page (full) and the
    head-aware move list, K+V (and K alone if k_only), each timed per call with
    HIP events on the launching stream over rotating sets of pools that
    together exceed 3x the 256 MB Infinity Cache, so every call reads and
    writes HBM. Pools hold N(0, 1) bf16 drawn on the device."""
    import numpy as np
    import torch
    from head_aware_paged_amd import rope_relocate
    from head_aware_paged_amd.session import SegPagedLayer
    Hkv, D = w.num_kv_heads, w.head_dim
    src, dst, dl = [], [], []
    for r in range(w.num_requests):
        for s in w.segments_of(r)[:-1]:
            for h in range(Hkv):
                a, b = w.cache_page_indptr[s * Hkv + h], w.cache_page_indptr[s * Hkv + h + 1]
                c, d = w.seg_page_indptr[s * Hkv + h], w.seg_page_indptr[s * Hkv + h + 1]
                src.extend(w.cache_pages[a:b])
                dst.extend(w.seg_pages[c:d])
                dl.extend([int(w.seg_start[s] - w.seg_orig_start[s])] * (b - a))
    layer = SegPagedLayer(w.num_q_heads, Hkv, D, w.seg_indptr, w.seg_start, w.seg_len, w.head_class, w.window,
                          w.retr_seg, page_size=16, device=dev)
    layer.build_pages(i32(w.seg_page_indptr), i32(w.seg_pages), i32(w.cache_page_indptr), i32(w.cache_pages),
                      i32(w.seg_orig_start))
    lists = {"full": (i32(src), i32(dst), i32(dl), len(src)),
             "head_aware": (layer.move_src, layer.move_dst, layer.move_delta, layer.num_moves)}
    n_cache, n_work = int(w.cache_page_indptr[-1]), int(w.seg_page_indptr[-1])
    set_bytes = 2 * (n_cache + n_work) * 16 * D * 2
    nsets = max(3, math.ceil(3 * 256e6 / set_bytes))
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)

    def pool(n, shape):
        return torch.randn(n, *shape, generator=gen, device=dev).to(torch.bfloat16)
    sets = [(pool(n_cache, (16, D)), pool(n_cache, (D, 16)), pool(n_work, (16, D)), pool(n_work, (D, 16)))
            for _ in range(nsets)]
    out = {}
    for lname, (s_, d_, dl_, n) in lists.items():
        for kv in ((True, False) if (k_only and lname == "full") else (True,)):
            def call(rep):
                kc, vc, kw, vw = sets[rep % nsets]
                rope_relocate(kc, kw, vc if kv else None, vw if kv else None, s_, d_, dl_, n, 16, D, w.rope_theta)
            tot = 0.0
            for rep in range(reps + nsets):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call(rep)
                e1.record()
                torch.cuda.synchronize()
                if rep >= nsets:
                    tot += e0.elapsed_time(e1)
            t = tot / reps
            # the same calls back to back (still rotating over the sets), so the
            # per-call time excludes the launch gap an isolated call pays
            nb = 4 * nsets
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for rep in range(nb):
                call(rep)
            e1.record()
            torch.cuda.synchronize()
            tb = e0.elapsed_time(e1) / nb
            nbytes = 2.0 * n * 16 * D * 2 * (2 if kv else 1)
            out[f"{lname}_{'kv' if kv else 'k'}"] = {
                "moves": n, "bytes": nbytes, "us": t * 1e3, "GB/s": nbytes / (t * 1e-3) / 1e9,
                "pct_hbm_peak": 100.0 * nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "us_back_to_back": tb * 1e3, "GB/s_back_to_back": nbytes / (tb * 1e-3) / 1e9,
                "pct_hbm_peak_back_to_back": 100.0 * nbytes / (tb * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    out["rotating_sets"] = f"{nsets} x {set_bytes / 1e6:.0f} MB"
    del sets, layer
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum host time of the oracle baseline")
    ap.add_argument("--skip-extras", action="store_true", help="only the timed steps (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(a kv-head-sharded design is described in the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from head_aware_paged_amd.session import SegPagedLayer, SparseFFN

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"

    def bf16(u):
        return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    log("generating mistral7b_32k workload")
    w = workloads.mistral_32k(fill_reused_work=False)
    per_row = visible_pairs_per_row(w)
    pairs = int(per_row.sum())
    flops = 4.0 * w.head_dim * pairs
    log(f"visible pairs {pairs} ({flops / 1e9:.2f} GFLOP per attention call)")
    layer = SegPagedLayer(w.num_q_heads, w.num_kv_heads, w.head_dim, w.seg_indptr, w.seg_start, w.seg_len,
                          w.head_class, w.window, w.retr_seg, device=dev)
    # V pools are d-major per page ([pages][D][page_size]); the workload holds them token-major
    q, k_work, v_work = bf16(w.q), bf16(w.k_work), bf16(np.swapaxes(w.v_work, 1, 2))
    k_cache, v_cache = bf16(w.k_cache), bf16(np.swapaxes(w.v_cache, 1, 2))
    spi, sp = i32(w.seg_page_indptr), i32(w.seg_pages)
    cpi, cp, sos = i32(w.cache_page_indptr), i32(w.cache_pages), i32(w.seg_orig_start)
    T, Hq, D = w.total_q_rows, w.num_q_heads, w.head_dim
    out = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
    Lk = w.context_len(0)
    n_last, ksel = 64, [Lk // 4]
    imp = torch.empty(Lk, dtype=torch.float32, device=dev)
    idx = torch.empty(ksel[0], dtype=torch.int32, device=dev)

    phases = {
        "pages": lambda: layer.build_pages(spi, sp, cpi, cp, sos),
        "reloc": lambda: layer.relocate(k_cache, k_work, v_cache, v_work, w.rope_theta),
        "attn": lambda: layer.attention(q, k_work, v_work, out=out, lse=lse),
        "imp": lambda: layer.importance_topk(q, k_work, lse, n_last, ksel, importance=imp, topk_idx=idx),
    }

    def step():
        for fn in phases.values():
            fn()

    log(f"warmup {args.warmup} eager steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    ref = [t.clone() for t in (out, lse, imp, idx)]

    # HIP graphs: the whole step, and each phase on its own. A replay runs the
    # captured kernel launches with no host work and no launch gaps, as a
    # serving loop runs a layer; every graph's outputs are checked against the
    # eager step before anything is timed.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            fn()
        return g

    def check_outputs(what):
        torch.cuda.synchronize()
        for a, b in zip((out, lse, imp, idx), ref):
            if not torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b):
                raise RuntimeError(f"{what}: graph replay differs from the eager step")

    graph = capture(step)
    per_graph = 10  # calls of one phase per phase graph, so graph launch cost is amortised

    def repeat(fn):
        def run():
            for _ in range(per_graph):
                fn()
        return run

    pgraphs = {n: capture(repeat(fn)) for n, fn in phases.items()}
    for t in (out, lse, imp, idx):
        t.zero_()
    graph.replay()
    check_outputs("step graph")
    for t in (out, lse, imp, idx):
        t.zero_()
    for n in phases:
        pgraphs[n].replay()
    check_outputs("phase graphs")

    def time_graph(g, reps):
        """Average GPU time of one replay, HIP events on the replaying stream."""
        for _ in range(args.warmup):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_phase = {n: time_graph(g, max(args.steps // 2, 10)) / per_graph for n, g in pgraphs.items()}
    t_pages, t_reloc, t_attn, t_imp = (t_phase[n] for n in ("pages", "reloc", "attn", "imp"))

    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} graph-replayed steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    # a plain 64 MiB device copy, the known-size reference for HBM byte counters
    xa = torch.empty(32 << 20, dtype=torch.bfloat16, device=dev)
    torch.empty_like(xa).copy_(xa)
    torch.cuda.synchronize()
    del xa
    attn_tflops = flops / (t_attn * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms (graph), {ms_eager:.3f} ms eager: pages {t_pages * 1e3:.1f} us, relocate "
        f"{t_reloc * 1e3:.1f} us, attention {t_attn * 1e3:.1f} us ({attn_tflops:.1f} TFLOP/s), importance+topk "
        f"{t_imp * 1e3:.1f} us")
    ha_bytes = 2.0 * layer.num_moves * 16 * D * 2 * 2  # K+V pages, read + write

    result = {
        "metric": "visible-pair attention TFLOP/s + % bf16 MFMA peak at 32K; relocate GB/s",
        "value": flops * args.steps / elapsed / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "ms_per_step_eager": ms_eager, "step_mode": "hip_graph_replay",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mistral7b_32k", "context": Lk, "query_rows": T, "q_heads": Hq,
                   "kv_heads": w.num_kv_heads, "head_dim": D, "page_size": 16,
                   "head_classes": "kv0 global, kv1-7 local(1024)", "visible_pairs": pairs,
                   "step": "build_pages + rope_relocate(head-aware moves, K+V) + segpaged_attn_prefill + "
                           "token_importance_topk(last 64 rows, k=25%)"},
        "breakdown_us": {"build_pages": t_pages * 1e3, "rope_relocate_head_aware": t_reloc * 1e3,
                         "segpaged_attn_prefill": t_attn * 1e3, "token_importance_topk": t_imp * 1e3},
        "attention": {"tflops": attn_tflops, "pct_bf16_peak": 100.0 * attn_tflops / PEAK_BF16_TFLOPS},
        "relocate_head_aware": {"moves": layer.num_moves, "us_in_step": t_reloc * 1e3,
                                "GB/s_in_step": ha_bytes / (t_reloc * 1e-3) / 1e9,
                                "note": "in_step: 10 calls per graph on the same 41 MB, cache-resident; "
                                        "hbm: per call on rotating buffer sets"},
    }
    traffic = profile_traffic("attn_main_mistral7b_32k", source_hash(["attention.hip", "plan.h", "common.h"]))
    result["roofline"] = {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                          "kernel": "segpaged_attn_prefill (attn_main_kernel + attn_combine_kernel)",
                          "algorithmic": f"{flops / 1e9:.3f} GFLOP per launch = 4*D*visible pairs"}

    if not args.skip_extras:
        # relocation bandwidth on HBM (rotating buffer sets) for the three attention layouts
        result["relocate"] = {"mistral7b_32k": relocation_bandwidth(w, dev, i32, k_only=True)}
        for wname, make in (("qwen3_32b_varlen", workloads.qwen_varlen), ("long_64k", workloads.long_64k)):
            result["relocate"][wname] = relocation_bandwidth(make(with_data=False), dev, i32)
        # plain device copy of 256 MiB (torch), for calibration
        xa = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev)
        xb = torch.empty_like(xa)
        for _ in range(3):
            xb.copy_(xa)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(10):
            xb.copy_(xa)
        a1.record()
        torch.cuda.synchronize()
        result["copy_256MiB_GB/s"] = 2.0 * xa.numel() * 2 * 10 / (a0.elapsed_time(a1) * 1e-3) / 1e9
        del xa, xb
        rl = result["relocate"]
        result["relocate_head_aware"]["GB/s_hbm"] = rl["mistral7b_32k"]["head_aware_kv"]["GB/s"]
        result["relocate_head_aware"]["us_hbm"] = rl["mistral7b_32k"]["head_aware_kv"]["us"]
        result["relocate_head_aware"]["GB/s_hbm_back_to_back"] = rl["mistral7b_32k"]["head_aware_kv"]["GB/s_back_to_back"]
        for wname, r_ in rl.items():
            log(f"relocate {wname}: full K+V {r_['full_kv']['GB/s']:.0f} GB/s "
                f"({r_['full_kv']['GB/s_back_to_back']:.0f} back to back), head-aware K+V "
                f"{r_['head_aware_kv']['GB/s']:.0f} GB/s ({r_['head_aware_kv']['us']:.1f} us; "
                f"{r_['head_aware_kv']['GB/s_back_to_back']:.0f} GB/s back to back)")
        log(f"copy {result['copy_256MiB_GB/s']:.0f} GB/s")

        # decode step of the same layer: one new row per request over the same page tables
        dq, dk, dv = (bf16(x) for x in workloads.decode_inputs(w, seed=0))
        dout = torch.empty(w.num_requests, Hq, D, dtype=torch.bfloat16, device=dev)
        dlse = torch.empty(w.num_requests, Hq, dtype=torch.float32, device=dev)
        dgraph = capture(repeat(lambda: layer.decode(dq, dk, dv, k_work, v_work, out=dout, lse=dlse)))
        t = time_graph(dgraph, 20) / per_graph
        n_vis = decode_visible_pages(w)
        n_tab = int(layer.sizes["table_entries"])
        nbytes = n_vis * 16 * D * 2 * 2.0  # K + V of every page holding a visible key
        result["decode_32k"] = {
            "us": t * 1e3, "visible_pages": n_vis, "table_pages_read": n_tab, "bytes": nbytes,
            "GB/s": nbytes / (t * 1e-3) / 1e9, "pct_hbm_peak": 100.0 * nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "kernels": "decode_main_kernel + decode_combine_kernel",
            "algorithmic": "K+V of every page holding a key visible to the new row, per kv head"}
        log(f"decode {t * 1e3:.1f} us, {result['decode_32k']['GB/s']:.0f} GB/s of visible K+V pages")

        # the layer glue around the attention: fused QKV projection + RoPE + append, output projection
        log("generating layer weights (hidden 4096)")
        hs = 4096
        lh, lwqkv, lwo = (bf16(x) for x in workloads.layer_inputs(w, hs, seed=0))
        lq = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=dev)
        seg_pi, seg_pg = i32(w.seg_page_indptr), i32(w.seg_pages)
        qgraph = capture(repeat(lambda: layer.qkv_rope_append(lh, lwqkv, w.rope_theta, seg_pi, seg_pg, k_work,
                                                              v_work, q_out=lq)))
        t_qkv = time_graph(qgraph, 20) / per_graph
        attn_rows = torch.empty(T, Hq * D, dtype=torch.bfloat16, device=dev).normal_()
        ograph = capture(repeat(lambda: layer.out_proj_residual(attn_rows, lwo, lh)))
        t_out = time_graph(ograph, 20) / per_graph
        qkv_flops = 2.0 * T * hs * (Hq + 2 * w.num_kv_heads) * D
        out_flops = 2.0 * T * hs * Hq * D
        result["layer_glue_32k"] = {
            "hidden": hs, "rows": T,
            "qkv_rope_append_us": t_qkv * 1e3, "qkv_tflops": qkv_flops / (t_qkv * 1e-3) / 1e12,
            "out_proj_us": t_out * 1e3, "out_proj_tflops": out_flops / (t_out * 1e-3) / 1e12,
            "layer_us": (t_qkv + t_pages + t_reloc + t_attn + t_out) * 1e3,
            "layer": "qkv_rope_append + build_pages + rope_relocate + segpaged_attn_prefill + out_proj_residual"}
        log(f"layer glue: qkv {t_qkv * 1e3:.1f} us ({result['layer_glue_32k']['qkv_tflops']:.0f} TFLOP/s), "
            f"out_proj {t_out * 1e3:.1f} us ({result['layer_glue_32k']['out_proj_tflops']:.0f} TFLOP/s)")
        del lh, lwqkv, lwo, qgraph, ograph

        # masked-dense comparator: the same attention over a dense per-head layout with an explicit mask
        from head_aware_paged_amd import masked_dense_attn, segkv_masked_dense_workspace_size
        Hkv = w.num_kv_heads
        L = -(-w.context_len(0) // 64) * 64
        kd = np.zeros((Hkv, L, D), np.uint16)
        vd = np.zeros((Hkv, L, D), np.uint16)
        for h in range(Hkv):
            for s in w.segments_of(0):
                b, n = int(w.seg_start[s]), int(w.seg_len[s])
                run = w.seg_pages[w.seg_page_indptr[s * Hkv + h]:w.seg_page_indptr[s * Hkv + h + 1]]
                kd[h, b:b + n] = w.k_work[run].reshape(-1, D)[:n]
                vd[h, b:b + n] = w.v_work[run].reshape(-1, D)[:n]
        kd_t = bf16(kd)
        vdt_t = bf16(np.ascontiguousarray(np.swapaxes(vd, 1, 2)))
        del kd, vd
        spans = layer.visible_spans().permute(1, 0, 2, 3)  # [Hkv][T][3][(lo, hi)], (-1, -1) padded
        jj = torch.arange(L, device=dev, dtype=torch.int32)
        dmask = torch.zeros(Hkv, T, L, dtype=torch.bool, device=dev)
        for x in range(3):
            lo, hi = spans[..., x, 0:1], spans[..., x, 1:2]
            dmask |= (jj >= lo) & (jj < hi)
        dmask = dmask.to(torch.uint8)
        dws = torch.empty(segkv_masked_dense_workspace_size(T, Hq, Hkv, D, L), dtype=torch.uint8, device=dev)
        dout = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=dev)
        dlse = torch.empty(T, Hq, dtype=torch.float32, device=dev)
        mgraph = capture(repeat(lambda: masked_dense_attn(q, kd_t, vdt_t, dmask, layer.scale, dout, dlse, dws)))
        t_dense = time_graph(mgraph, 3) / per_graph
        dense_flops = 4.0 * D * T * Hq * L
        result["masked_dense_32k"] = {
            "us": t_dense * 1e3, "keys": L, "dense_tflops": dense_flops / (t_dense * 1e-3) / 1e12,
            "mask_bytes": Hkv * T * L, "segpaged_attn_us": t_attn * 1e3, "penalty": t_dense / t_attn,
            "kernels": "dense_main_kernel + dense_combine_kernel"}
        log(f"masked dense {t_dense * 1e3:.1f} us ({result['masked_dense_32k']['dense_tflops']:.0f} TFLOP/s dense), "
            f"{t_dense / t_attn:.2f}x the SegPaged attention")
        del kd_t, vdt_t, dws, mgraph
        # the tuned attention kernel in mask mode over all-global (dense) page tables
        from head_aware_paged_amd.session import SegPagedLayer
        glayer = SegPagedLayer(Hq, Hkv, D, w.seg_indptr, w.seg_start, w.seg_len, np.zeros_like(w.head_class),
                               np.zeros_like(w.window), np.full_like(w.retr_seg, -1), page_size=16, device=dev)
        glayer.build_pages(seg_pi, seg_pg)
        ggraph = capture(repeat(lambda: glayer.attention_masked(q, k_work, v_work, dmask, out=dout, lse=dlse)))
        t_gm = time_graph(ggraph, 5) / per_graph
        dense_pairs = 0
        for h in range(Hkv):  # every key of every computed tile: rows x keys up to the row's m-tile end
            dense_pairs += w.num_q_heads // Hkv * T * w.context_len(0)
        result["masked_dense_tuned_32k"] = {
            "us": t_gm * 1e3, "dense_tflops": 4.0 * D * dense_pairs / (t_gm * 1e-3) / 1e12,
            "segpaged_attn_us": t_attn * 1e3, "penalty": t_gm / t_attn,
            "kernels": "attn_main_kernel<D, true> + attn_combine_kernel over all-global page tables"}
        log(f"masked dense (tuned kernel, mask mode) {t_gm * 1e3:.1f} us, {t_gm / t_attn:.2f}x the SegPaged attention")
        del dmask, ggraph, glayer

        # layer-wise elastic policy: 4 layers of the 32K layout (2 shallow: all-local heads + dense FFN;
        # 2 deep: the class map + FFN on the top 25 % query rows), against 4 uniform layers (class map + dense FFN)
        from head_aware_paged_amd.session import ElasticStack
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        inter = 14336

        def rnd(*shape, std):
            return (torch.randn(*shape, generator=gen, device=dev) * std).to(torch.bfloat16)
        slayers = []
        for _ in range(4):
            slayers.append(dict(w_qkv=rnd((Hq + 2 * Hkv) * D, hs, std=hs ** -0.5), w_o=rnd(hs, Hq * D, std=(Hq * D) ** -0.5),
                                w_gate=rnd(inter, hs, std=hs ** -0.5), w_up=rnd(inter, hs, std=hs ** -0.5),
                                w_down=rnd(hs, inter, std=0.2 * inter ** -0.5), k_pool=k_work, v_pool=v_work))
        shid0 = rnd(T, hs, std=1.0)
        shid = shid0.clone()
        stack_args = (Hq, Hkv, D, w.seg_indptr, w.seg_start, w.seg_len, w.head_class, w.window, w.retr_seg,
                      seg_pi, seg_pg, slayers)
        res = {}
        for name, n_sh, kk in (("elastic", 2, T // 4), ("uniform", 0, T)):
            st = ElasticStack(*stack_args, n_shallow=n_sh, shallow_window=1024, k=kk, n_last=64,
                              rope_theta=w.rope_theta)

            def fwd(st=st):
                shid.copy_(shid0)
                st.forward(shid)
            fwd()
            torch.cuda.synchronize()
            sg = capture(fwd)
            res[name] = time_graph(sg, 5)
            del sg, st
        result["elastic_stack_32k"] = {
            "layers": 4, "hidden": hs, "inter": inter, "elastic_us": res["elastic"] * 1e3,
            "uniform_us": res["uniform"] * 1e3, "speedup": res["uniform"] / res["elastic"],
            "elastic": "layers 0-1 all-local(1024) + dense FFN; layers 2-3 class map + FFN on the top 128 of 512 rows",
            "uniform": "every layer the class map + dense FFN",
            "note": "random-init weights; the layers share one set of pools (timing only)"}
        log(f"elastic stack {res['elastic'] * 1e3:.0f} us vs uniform {res['uniform'] * 1e3:.0f} us "
            f"({res['uniform'] / res['elastic']:.2f}x)")
        del slayers, shid, shid0

        # the attention on the two other full-size layouts: the 4-request varlen batch and the 64K layer
        # (structure from the workload generators; pools and Q drawn on the device, N(0, 1) bf16)
        from head_aware_paged_amd.session import SegPagedLayer
        for wname, make in (("qwen3_32b_varlen", workloads.qwen_varlen), ("long_64k", workloads.long_64k)):
            wx = make(with_data=False)
            xl = SegPagedLayer(wx.num_q_heads, wx.num_kv_heads, wx.head_dim, wx.seg_indptr, wx.seg_start, wx.seg_len,
                               wx.head_class, wx.window, wx.retr_seg, page_size=16, device=dev)
            xl.build_pages(i32(wx.seg_page_indptr), i32(wx.seg_pages))
            gen = torch.Generator(device=dev)
            gen.manual_seed(11)
            Dx, np_ = wx.head_dim, wx.k_work.shape[0]
            qx = torch.randn(wx.total_q_rows, wx.num_q_heads, Dx, generator=gen, device=dev).to(torch.bfloat16)
            kx = torch.randn(np_, 16, Dx, generator=gen, device=dev).to(torch.bfloat16)
            vx = torch.randn(np_, Dx, 16, generator=gen, device=dev).to(torch.bfloat16)
            ox = torch.empty_like(qx)
            lx = torch.empty(wx.total_q_rows, wx.num_q_heads, dtype=torch.float32, device=dev)
            xg = capture(repeat(lambda: xl.attention(qx, kx, vx, out=ox, lse=lx)))
            tx = time_graph(xg, 5) / per_graph
            px = int(visible_pairs_per_row(wx).sum())
            fx = 4.0 * Dx * px
            result[f"attention_{wname}"] = {
                "us": tx * 1e3, "visible_pairs": px, "gflop": fx / 1e9, "tflops": fx / (tx * 1e-3) / 1e12,
                "pct_bf16_peak": 100.0 * fx / (tx * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
            log(f"attention {wname}: {tx * 1e3:.1f} us, {fx / (tx * 1e-3) / 1e12:.0f} TFLOP/s")
            del xl, qx, kx, vx, ox, lx, xg

        # sparse SwiGLU FFN of the 8K selection workload (k = 2048 rows, 4096 -> 14336)
        log("generating sparse_ffn_8k FFN inputs")
        w5 = workloads.sparse_ffn_8k()
        hid0 = bf16(w5.hidden)
        hid = hid0.clone()
        ffn = SparseFFN(bf16(w5.w_gate), bf16(w5.w_up), bf16(w5.w_down), k_max=w5.topk)
        sel = i32(np.arange(0, 8192, 4))
        # every call starts from the same hidden rows (the FFN updates them in
        # place); the restoring copy sits outside each call's events. 20 calls
        # (about 20 ms) bring the clocks to their steady state first.
        ts = []
        for rep in range(30):
            hid.copy_(hid0)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            ffn(hid, sel, w5.topk)
            a1.record()
            torch.cuda.synchronize()
            if rep >= 20:
                ts.append(a0.elapsed_time(a1))
        t = sum(ts) / len(ts)
        ffn_flops = 6.0 * w5.topk * 4096 * 14336
        result["sparse_ffn_8k"] = {"rows": w5.topk, "us": t * 1e3, "tflops": ffn_flops / (t * 1e-3) / 1e12,
                                   "pct_bf16_peak": 100.0 * ffn_flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        log(f"sparse FFN {result['sparse_ffn_8k']['tflops']:.1f} TFLOP/s")
        del hid, hid0, ffn

        log("cpu baseline: fp64 oracle on the same workload")
        result["cpu_baseline"] = cpu_baseline(w, per_row, args.cpu_seconds)
        log(f"cpu baseline {result['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
