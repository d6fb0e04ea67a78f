// SELECTVISIBLESTATE: per-(request, kv head) page tables, the head-aware
// relocation move list, the attention work plan, and the visible-span export.
//
// RedKnot README ("About": per-head page table + segmented KV store, per-class
// visible windows); paooo.com "如何使用RedKnot" (SELECTVISIBLESTATE chooses
// the local-head KV to reuse and the global-head ranges to recompute). All of
// it is integer work on small metadata; it runs on the device so that nothing
// has to be copied from the host between the calls of one layer.
#include "common.h"

namespace segkv {
namespace {

constexpr int kScanThreads = 1024;

// DPP moves inside rows of 16 lanes; a lane whose source lies outside its row reads 0
template <int CTRL>
__device__ __forceinline__ int dpp_row(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;

// Inclusive prefix sum over the 64 lanes of a wave: row_shr steps inside each
// 16-lane row, then the totals of the rows below (read from lanes 15, 31, 47).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += dpp_row<kDppRowShr1>(x);
  x += dpp_row<kDppRowShr2>(x);
  x += dpp_row<kDppRowShr4>(x);
  x += dpp_row<kDppRowShr8>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// N exclusive prefix sums at once over n items: value(i, v) fills v[0..N),
// write(i, p) receives the prefixes; totals[] receives the sums (uniform
// across the block). Block-wide, all threads call it; s holds at least
// N * kScanThreads / 64 ints. Two barriers per 1024 items; up to 64 items take one wave.
template <int N, class F, class W>
__device__ void block_scan(int n, F value, W write, int (&totals)[N], int* s) {
  constexpr int NW = kScanThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= 64) {
    // one wave scans, the others only wait for the totals: one barrier
    if (wave == 0) {
      int v[N], p[N];
#pragma unroll
      for (int c = 0; c < N; ++c) v[c] = 0;
      if (lane < n) value(lane, v);
#pragma unroll
      for (int c = 0; c < N; ++c) {
        const int x = wave_inclusive_scan(v[c]);
        p[c] = x - v[c];
        if (lane == 63) s[c] = x;
      }
      if (lane < n) write(lane, p);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < N; ++c) totals[c] = s[c];
    __syncthreads();  // s is free again for the next scan
    return;
  }
  int carry[N];
#pragma unroll
  for (int c = 0; c < N; ++c) carry[c] = 0;
  for (int base = 0; base < n; base += kScanThreads) {
    const int i = base + tid;
    int v[N], x[N];
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = 0;
    if (i < n) value(i, v);
#pragma unroll
    for (int c = 0; c < N; ++c) {
      x[c] = wave_inclusive_scan(v[c]);
      if (lane == 63) s[c * NW + wave] = x[c];
    }
    __syncthreads();
    int p[N];
#pragma unroll
    for (int c = 0; c < N; ++c) {
      int before = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int sw = s[c * NW + w];
        before += w < wave ? sw : 0;
        tot += sw;
      }
      p[c] = carry[c] + before + x[c] - v[c];
      carry[c] += tot;
    }
    if (i < n) write(i, p);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < N; ++c) totals[c] = carry[c];
}

struct PagesArgs {
  segkv_meta m;
  const int32_t* cu_q;
  const int32_t* seg_page_indptr;
  const int32_t* seg_pages;
  int32_t* page_indptr;
  int32_t* page_ids;
  int32_t* page_pos;
  const int32_t* cache_page_indptr;
  const int32_t* cache_pages;
  const int32_t* seg_orig_start;
  int32_t* move_src;
  int32_t* move_dst;
  int32_t* move_delta;
  char* plan;
  int R, Hkv, G;
  int chunk_tiles;
  int n_mtiles, n_split;  // host counts (bounds of the plan arrays)
  int key_blocks;         // 64-key blocks of the longest request
  int n_items;      // launch slots of the attention kernel (a multiple of 8)
  int n_imp_items;  // importance work items (64-key blocks of every table)
  PlanLayout L;
};

constexpr int kMaxPairs = 1024;     // (request, kv head) pairs of one layout
constexpr int kMaxMTiles = 8192;    // attention m-tiles of one layout

// Per-pair facts, staged in LDS once.
struct PairInfo {
  int cls, W, bq, Lq, cu_q, tbase;
  PageRuns pr;
};

__device__ PairInfo pair_info(const PagesArgs& a, int k) {
  const int r = k / a.Hkv, h = k % a.Hkv;
  const HeadView v = head_view_dev(a.m, a.Hkv, r, h);
  PairInfo p;
  p.cls = v.cls;
  p.W = v.W;
  p.bq = v.bq;
  p.Lq = v.Lq;
  p.cu_q = a.cu_q[r];
  p.tbase = 0;
  p.pr = head_page_runs(v);
  return p;
}

// One launch: block 0 plans; fill blocks each fill up to 1024 table entries of
// one (request, kv head) pair; mask blocks write the importance head masks;
// item blocks write up to 1024 importance items each. Fill and item blocks
// derive the offsets they need themselves, so no block waits for another.
__global__ __launch_bounds__(kScanThreads) void build_kernel(PagesArgs a, int fill_blocks_per_pair) {
  __shared__ int s[kScanThreads];
  __shared__ int sseg[kScanThreads];  // fill blocks: segment starts of the pair's request
  __shared__ int pair_maxc[kMaxPairs];  // most chunks of any m-tile of the pair
  __shared__ int pair_ib[kMaxPairs];    // first group-major item position of the pair
  __shared__ int pair_imp[kMaxPairs];   // first importance item of the pair
  __shared__ PairInfo info[kMaxPairs];
  __shared__ int req_off[kMaxPairs + 1];
  __shared__ int mt_chunks[kMaxMTiles];
  __shared__ int red[2][kScanThreads / 64];
  const int tid = threadIdx.x;
  const int n_pairs = a.R * a.Hkv;

  const int n_fill = n_pairs * fill_blocks_per_pair;
  const int n_mask = a.R * cdiv(a.key_blocks, kScanThreads);
  if ((int)blockIdx.x > n_fill + n_mask) {
    // ---------------- importance items [c * 1024, (c + 1) * 1024) ----------------
    // every 64-key block of every table, pair by pair; this block derives the
    // pairs' table offsets, item offsets and the requests' key offsets itself
    const int c = blockIdx.x - 1 - n_fill - n_mask;
    for (int k = tid; k < n_pairs; k += kScanThreads) info[k] = pair_info(a, k);
    __syncthreads();
    int it_tot[3];
    block_scan<3>(
        n_pairs,
        [&](int k, int (&v)[3]) {
          v[0] = runs_count(info[k].pr);
          v[1] = runs_count(block_runs(info[k].pr));
          v[2] = k % a.Hkv == 0 ? info[k].bq + info[k].Lq : 0;
        },
        [&](int k, const int (&p)[3]) {
          info[k].tbase = p[0];
          pair_imp[k] = p[1];
          if (k % a.Hkv == 0) req_off[k / a.Hkv] = p[2];
        },
        it_tot, s);
    ImpItem* imp_items = reinterpret_cast<ImpItem*>(a.plan + a.L.imp_items_off);
    const int x = c * kScanThreads + tid;
    if (x >= imin(it_tot[1], a.n_imp_items)) return;
    int lo = 0, hi = n_pairs - 1;  // pair: last k with pair_imp[k] <= x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pair_imp[mid] <= x) lo = mid; else hi = mid - 1;
    }
    const PairInfo& pi = info[lo];
    ImpItem it;
    it.pair = lo;
    it.block = runs_page(block_runs(pi.pr), x - pair_imp[lo]);
    it.cls = pi.cls;
    it.W = pi.W;
    it.bq = pi.bq;
    it.Lq = pi.Lq;
    it.cu_q = pi.cu_q;
    it.key_off = req_off[lo / a.Hkv];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int page = it.block * (kTileKeys / kPage) + i, rk = runs_rank(pi.pr, page);
      it.entry[i] = runs_rank(pi.pr, page + 1) - rk == 1 ? pi.tbase + rk : -1;
    }
    imp_items[x] = it;
    return;
  }
  if ((int)blockIdx.x > n_fill) {
    // ---------------- importance head masks of request r, blocks [c * 1024, ...) ----------------
    // (kv heads <= 64; otherwise no masks are written)
    const int mb = blockIdx.x - 1 - n_fill, per_req = cdiv(a.key_blocks, kScanThreads);
    const int r = mb / per_req, blk = (mb % per_req) * kScanThreads + tid;
    if (a.Hkv > 64) return;
    for (int h = tid; h < a.Hkv; h += kScanThreads) info[h].pr = block_runs(pair_info(a, r * a.Hkv + h).pr);
    __syncthreads();
    if (blk >= a.key_blocks) return;
    uint64_t mk = 0;
    for (int h = 0; h < a.Hkv; ++h) {
      const PageRuns& b = info[h].pr;
      if (runs_rank(b, blk + 1) - runs_rank(b, blk) == 1) mk |= 1ull << h;
    }
    reinterpret_cast<uint64_t*>(a.plan + a.L.imp_mask_off)[(size_t)r * a.key_blocks + blk] = mk;
    return;
  }
  if (blockIdx.x > 0) {
    // ---------------- table fill for pair k, entries [blk * 1024, ...) ----------------
    const int k = (blockIdx.x - 1) / fill_blocks_per_pair;
    const int blk = (blockIdx.x - 1) % fill_blocks_per_pair;
    int tsum = 0, msum = 0;  // table sizes and move counts of the pairs before k
    for (int q = tid; q < k; q += kScanThreads) {
      const PairInfo p = pair_info(a, q);
      tsum += runs_count(p.pr);
      msum += runs_rank(p.pr, p.bq / kPage);
    }
    for (int o = 32; o > 0; o >>= 1) {
      tsum += __shfl_xor(tsum, o);
      msum += __shfl_xor(msum, o);
    }
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = tsum;
      red[1][tid >> 6] = msum;
    }
    const PairInfo p = pair_info(a, k);
    {
      const int rr = k / a.Hkv, t0 = a.m.seg_indptr[rr], t1 = a.m.seg_indptr[rr + 1];
      if (t1 - t0 <= kScanThreads && tid < t1 - t0) sseg[tid] = a.m.seg_start[t0 + tid];
    }
    __syncthreads();
    int base = 0, mbase = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      base += red[0][w];
      mbase += red[1][w];
    }
    const int e = blk * kScanThreads + tid;
    if (e >= runs_count(p.pr)) return;
    const int r = k / a.Hkv, h = k % a.Hkv;
    const int s0 = a.m.seg_indptr[r], s1 = a.m.seg_indptr[r + 1];
    const int tok = runs_page(p.pr, e) * kPage;
    int lo = s0, hi = s1 - 1;  // segment holding this page: last segment with start <= tok
    if (s1 - s0 <= kScanThreads) {  // starts staged in LDS (the request's segments, one load each)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sseg[mid - s0] <= tok) lo = mid; else hi = mid - 1;
      }
    } else {
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.m.seg_start[mid] <= tok) lo = mid; else hi = mid - 1;
      }
    }
    const int sg = lo;
    const int sstart = s1 - s0 <= kScanThreads ? sseg[sg - s0] : a.m.seg_start[sg];
    const int qpage = (tok - sstart) / kPage;
    const int phys = a.seg_pages[a.seg_page_indptr[sg * a.Hkv + h] + qpage];
    a.page_ids[base + e] = phys;
    a.page_pos[base + e] = tok;
    if (a.move_src != nullptr && sg != s1 - 1) {
      // reused pages precede the query segment's pages in the ascending table
      const int mi = mbase + e;
      a.move_src[mi] = a.cache_pages[a.cache_page_indptr[sg * a.Hkv + h] + qpage];
      a.move_dst[mi] = phys;
      a.move_delta[mi] = sstart - a.seg_orig_start[sg];
    }
    return;
  }

  // ---------------- block 0: table offsets and the attention plan ----------------
  PlanHeader* hdr = reinterpret_cast<PlanHeader*>(a.plan);
  int32_t* move_off = reinterpret_cast<int32_t*>(a.plan + a.L.move_off_off);
  int32_t* req_off_g = reinterpret_cast<int32_t*>(a.plan + a.L.req_mt_off);
  MTile* mt = reinterpret_cast<MTile*>(a.plan + a.L.mtiles_off);
  Item* items = reinterpret_cast<Item*>(a.plan + a.L.items_off);
  SplitTile* split = reinterpret_cast<SplitTile*>(a.plan + a.L.split_off);
  const int MP = mtile_positions(a.G);
  const int S = a.chunk_tiles;

  for (int k = tid; k < n_pairs; k += kScanThreads) info[k] = pair_info(a, k);
  __syncthreads();
  // per pair: table entries, head-aware moves, importance blocks
  int pt[3];
  block_scan<3>(
      n_pairs,
      [&](int k, int (&v)[3]) {
        v[0] = runs_count(info[k].pr);
        v[1] = runs_rank(info[k].pr, info[k].bq / kPage);
        v[2] = runs_count(block_runs(info[k].pr));
      },
      [&](int k, const int (&p)[3]) {
        a.page_indptr[k] = p[0];
        info[k].tbase = p[0];
        move_off[k] = p[1];
        pair_imp[k] = p[2];
      },
      pt, s);
  // per request: m-tiles
  int rt[1];
  block_scan<1>(
      a.R, [&](int r, int (&v)[1]) { v[0] = a.Hkv * cdiv(info[r * a.Hkv].Lq, MP); },
      [&](int r, const int (&p)[1]) {
        req_off[r] = p[0];
        req_off_g[r] = p[0];
      },
      rt, s);
  const int n_mt = imin(rt[0], a.n_mtiles);  // equal unless the layout changed since sizing
  if (tid == 0) {
    a.page_indptr[n_pairs] = pt[0];
    move_off[n_pairs] = pt[1];
    req_off[a.R] = n_mt;
    req_off_g[a.R] = n_mt;
  }
  __syncthreads();

  // descriptors, one m-tile per thread
  for (int i = tid; i < n_mt; i += kScanThreads) {
    int lo = 0, hi = a.R - 1;  // request: last r with req_off[r] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (req_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int nj = (req_off[r + 1] - req_off[r]) / a.Hkv;
    const int h = (i - req_off[r]) / nj, j = (i - req_off[r]) % nj;
    const PairInfo& p = info[r * a.Hkv + h];
    HeadView v;
    v.cls = p.cls;
    v.W = p.W;
    v.bq = p.bq;
    v.Lq = p.Lq;
    v.Lk = p.bq + p.Lq;
    const int t0 = j * MP;
    const int i_lo = p.bq + t0, i_hi = p.bq + imin(p.Lq, t0 + MP) - 1;
    int e0, e1;
    mtile_entries(v, p.pr, i_lo, i_hi, &e0, &e1);
    MTile d;
    d.r = r;
    d.h = h;
    d.q_row0 = p.cu_q + t0;
    d.n_pos = imin(p.Lq, t0 + MP) - t0;
    d.pos0 = i_lo;
    d.cls = p.cls;
    d.W = p.W;
    d.bq = p.bq;
    d.e_begin = p.tbase + e0;
    d.e_end = p.tbase + e1;
    d.n_tiles = cdiv(e1 - e0, kTilePages);
    d.n_chunks = num_chunks(d.n_tiles, S);
    d.partial_base = -1;
    d.pad[0] = d.pad[1] = d.pad[2] = 0;
    mt_chunks[i] = d.n_chunks;
    mt[i] = d;
  }
  __syncthreads();

  // per m-tile: partial slots and split list
  int mt_tot[2];
  block_scan<2>(
      n_mt,
      [&](int i, int (&v)[2]) {
        v[0] = mt_chunks[i] > 1 ? mt_chunks[i] : 0;
        v[1] = mt_chunks[i] > 1 ? 1 : 0;
      },
      [&](int i, const int (&p)[2]) {
        if (mt_chunks[i] > 1) {
          mt[i].partial_base = p[0];
          if (p[1] < a.n_split) {
            const MTile& d = mt[i];  // written by this work-group before the scan's barriers
            split[p[1]] = SplitTile{p[0], mt_chunks[i], d.q_row0, d.h, d.n_pos, {0, 0, 0}};
          }
        }
      },
      mt_tot, s);
  const int n_partials = mt_tot[0], n_split = mt_tot[1];

  // items in XCD-aware order (see xcd_slot): group-major position of item
  // (m-tile j of pair k, chunk c) = pair_ib[k] + c * nj_k + j
  for (int k = tid; k < n_pairs; k += kScanThreads) {
    const int r = k / a.Hkv, h = k % a.Hkv;
    const int nj = (req_off[r + 1] - req_off[r]) / a.Hkv, i0 = req_off[r] + h * nj;
    int mc = 0;
    for (int j = 0; j < nj; ++j) mc = imax(mc, mt_chunks[i0 + j]);
    pair_maxc[k] = mc;
  }
  __syncthreads();
  int pos_tot[1];
  block_scan<1>(
      n_pairs,
      [&](int k, int (&v)[1]) {
        const int r = k / a.Hkv;
        v[0] = pair_maxc[k] * ((req_off[r + 1] - req_off[r]) / a.Hkv);
      },
      [&](int k, const int (&p)[1]) { pair_ib[k] = p[0]; }, pos_tot, s);
  const int n_pos = pos_tot[0];
  // one launch slot per thread: slot b runs on XCD b % 8 and takes position
  // (b % 8) q8 + b / 8 of the group-major list
  const int q8 = a.n_items / kXcds;
  for (int b = tid; b < a.n_items; b += kScanThreads) {
    const int p = (b & (kXcds - 1)) * q8 + (b >> 3);
    Item it{};
    it.mtile = -1;
    if (p < n_pos) {
      int lo = 0, hi = n_pairs - 1;  // pair: last k with pair_ib[k] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pair_ib[mid] <= p) lo = mid; else hi = mid - 1;
      }
      const int k = lo, r = k / a.Hkv, h = k % a.Hkv;
      const int nj = (req_off[r + 1] - req_off[r]) / a.Hkv;
      const int rel = p - pair_ib[k], c = rel / nj, i = req_off[r] + h * nj + rel % nj;
      if (c < mt_chunks[i]) {
        const MTile d = mt[i];  // complete since the scans' barriers
        it.mtile = i;
        it.chunk = c;
        it.t_lo = chunk_tile_lo(d.n_tiles, d.n_chunks, c);
        it.T = chunk_tile_lo(d.n_tiles, d.n_chunks, c + 1) - it.t_lo;
        it.h = d.h;
        it.q_row0 = d.q_row0;
        it.n_pos = d.n_pos;
        it.pos0 = d.pos0;
        it.cls = d.cls;
        it.W = d.W;
        it.bq = d.bq;
        it.e_lo = d.e_begin + kTilePages * it.t_lo;
        it.e_end = d.e_end;
        it.partial_slot = d.partial_base >= 0 ? d.partial_base + c : -1;
      }
    }
    items[b] = it;
  }

  // importance: first key of each request, and per (request, 64-key block)
  // the kv heads whose tables touch the block (kv heads <= 64)
  int32_t* req_key = reinterpret_cast<int32_t*>(a.plan + a.L.req_key_off);
  int kt[1];
  block_scan<1>(
      a.R, [&](int r, int (&v)[1]) { v[0] = info[r * a.Hkv].bq + info[r * a.Hkv].Lq; },
      [&](int r, const int (&p)[1]) { req_key[r] = p[0]; }, kt, s);
  if (tid == 0) req_key[a.R] = kt[0];

  const int n_imp = pt[2];  // importance items (written by the item blocks)
  if (tid == 0) {
    PlanHeader h;
    h.n_mtiles = n_mt;
    h.n_items = a.n_items;
    h.n_split = n_split;
    h.chunk_tiles = S;
    h.n_partials = n_partials;
    h.total_q_rows = a.cu_q[a.R];
    h.max_tiles = 0;
    h.n_imp_items = n_imp;
    for (int q = 0; q < 8; ++q) h.pad[q] = 0;
    *hdr = h;
  }
}

// One thread per (query row, kv head).
__global__ __launch_bounds__(256) void spans_kernel(segkv_meta m, const int32_t* cu_q, int R, int Hkv,
                                                    int total_rows, int32_t* spans) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_rows * Hkv) return;
  const int row = gid / Hkv, h = gid % Hkv;
  int lo = 0, hi = R - 1;  // request: last r with cu_q[r] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const HeadView v = head_view_dev(m, Hkv, r, h);
  const int i = v.bq + (row - cu_q[r]);
  int a[3], b[3], n = 0;
  if (v.cls == kClassLocal) {
    a[0] = local_lo(i, v.bq, v.W);
    b[0] = i + 1;
    n = 1;
  } else if (v.cls == kClassRetrieval) {
    int x[3] = {v.rlo[0], v.rlo[1], v.bq}, y[3] = {v.rhi[0], v.rhi[1], i + 1};
    for (int p = 1; p < 3; ++p)
      for (int q = p; q > 0 && x[q] < x[q - 1]; --q) {
        int t = x[q]; x[q] = x[q - 1]; x[q - 1] = t;
        t = y[q]; y[q] = y[q - 1]; y[q - 1] = t;
      }
    for (int p = 0; p < 3; ++p) {
      if (n > 0 && x[p] <= b[n - 1]) {
        b[n - 1] = imax(b[n - 1], y[p]);
      } else {
        a[n] = x[p];
        b[n] = y[p];
        ++n;
      }
    }
  } else {
    a[0] = 0;
    b[0] = i + 1;
    n = 1;
  }
  int32_t* o = spans + (size_t)gid * 6;
  for (int p = 0; p < 3; ++p) {
    o[2 * p] = p < n ? a[p] : -1;
    o[2 * p + 1] = p < n ? b[p] : -1;
  }
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" int32_t segkv_build_pages(const segkv_dims* dims, const segkv_meta* meta_host,
                                     const segkv_meta* meta_dev, const int32_t* cu_q_dev,
                                     const int32_t* seg_page_indptr_dev, const int32_t* seg_pages_dev,
                                     int32_t* page_indptr_dev, int32_t* page_ids_dev, int32_t* page_pos_dev,
                                     int64_t table_capacity, const int32_t* cache_page_indptr_dev,
                                     const int32_t* cache_pages_dev, const int32_t* seg_orig_start_dev,
                                     int32_t* move_src_dev, int32_t* move_dst_dev, int32_t* move_delta_dev,
                                     int64_t move_capacity, void* plan_dev, size_t plan_bytes, void* stream) {
  clear_error();
  HostPlan hp;
  int32_t st = compute_host_plan(dims, meta_host, &hp);
  if (st != SEGKV_OK) return st;
  if (meta_dev == nullptr || !meta_dev->seg_indptr || !meta_dev->seg_start || !meta_dev->seg_len ||
      !meta_dev->head_class || !meta_dev->window || !meta_dev->retr_seg)
    return fail(SEGKV_ERR_INVALID_ARG, "device metadata pointer is NULL");
  if (!cu_q_dev || !seg_page_indptr_dev || !seg_pages_dev || !page_indptr_dev || !page_ids_dev ||
      !page_pos_dev || !plan_dev)
    return fail(SEGKV_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (table_capacity < hp.table_entries)
    return fail(SEGKV_ERR_CAPACITY, "table capacity " + std::to_string(table_capacity) + " < " +
                                         std::to_string(hp.table_entries));
  const bool moves = move_src_dev != nullptr;
  if (moves) {
    if (!move_dst_dev || !move_delta_dev || !cache_page_indptr_dev || !cache_pages_dev || !seg_orig_start_dev)
      return fail(SEGKV_ERR_INVALID_ARG, "move list requested but a move/cache pointer is NULL");
    if (move_capacity < hp.move_entries)
      return fail(SEGKV_ERR_CAPACITY, "move capacity " + std::to_string(move_capacity) + " < " +
                                           std::to_string(hp.move_entries));
  }
  if (plan_bytes < hp.plan_bytes)
    return fail(SEGKV_ERR_WORKSPACE, "plan buffer " + std::to_string(plan_bytes) + " < " +
                                         std::to_string(hp.plan_bytes));
  if (dims->num_requests * dims->num_kv_heads > kMaxPairs)
    return fail(SEGKV_ERR_UNSUPPORTED, "more than 1024 (request, kv head) pairs in one call");
  if (hp.n_mtiles > kMaxMTiles) return fail(SEGKV_ERR_UNSUPPORTED, "more than 8192 attention m-tiles in one call");
  if (!aligned16(plan_dev)) return fail(SEGKV_ERR_ALIGNMENT, "plan buffer must be 16-byte aligned");

  PagesArgs a;
  a.m = *meta_dev;
  a.cu_q = cu_q_dev;
  a.seg_page_indptr = seg_page_indptr_dev;
  a.seg_pages = seg_pages_dev;
  a.page_indptr = page_indptr_dev;
  a.page_ids = page_ids_dev;
  a.page_pos = page_pos_dev;
  a.cache_page_indptr = cache_page_indptr_dev;
  a.cache_pages = cache_pages_dev;
  a.seg_orig_start = seg_orig_start_dev;
  a.move_src = moves ? move_src_dev : nullptr;
  a.move_dst = move_dst_dev;
  a.move_delta = move_delta_dev;
  a.plan = static_cast<char*>(plan_dev);
  a.R = dims->num_requests;
  a.Hkv = dims->num_kv_heads;
  a.G = dims->num_q_heads / dims->num_kv_heads;
  a.chunk_tiles = hp.chunk_tiles;
  a.n_items = hp.n_items;
  a.n_imp_items = hp.n_imp_items;
  a.n_mtiles = hp.n_mtiles;
  a.n_split = hp.n_split;
  a.key_blocks = hp.key_blocks;
  a.L = host_plan_layout(*dims, hp);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int max_pages = 1;
  for (int r = 0; r < a.R; ++r) {
    const int sq = meta_host->seg_indptr[r + 1] - 1;
    max_pages = imax(max_pages, cdiv(meta_host->seg_start[sq] + meta_host->seg_len[sq], kPage));
  }
  const int per_pair = cdiv(max_pages, kScanThreads);
  const int mask_blocks = a.R * cdiv(hp.key_blocks, kScanThreads);
  const int item_blocks = cdiv(hp.n_imp_items, kScanThreads);
  build_kernel<<<1 + a.R * a.Hkv * per_pair + mask_blocks + item_blocks, kScanThreads, 0, s>>>(a, per_pair);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}

extern "C" int32_t segkv_visible_spans(const segkv_dims* dims, const segkv_meta* meta_host,
                                       const segkv_meta* meta_dev, const int32_t* cu_q_dev, int32_t* spans_dev,
                                       void* stream) {
  clear_error();
  HostPlan hp;
  int32_t st = compute_host_plan(dims, meta_host, &hp);
  if (st != SEGKV_OK) return st;
  if (meta_dev == nullptr || !meta_dev->seg_indptr || !cu_q_dev || !spans_dev)
    return fail(SEGKV_ERR_INVALID_ARG, "a required device pointer is NULL");
  const int n = (int)hp.total_q_rows * dims->num_kv_heads;
  if (n == 0) return SEGKV_OK;
  spans_kernel<<<cdiv(n, 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      *meta_dev, cu_q_dev, dims->num_requests, dims->num_kv_heads, (int)hp.total_q_rows, spans_dev);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}
