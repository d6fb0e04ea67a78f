// Shared host/device planning arithmetic for the SegPaged prefill path.
//
// Everything here is integer bookkeeping that both the host (sizing, grid
// shapes) and the device (table fill, attention plan) evaluate; compiling the
// same functions for both sides keeps them in exact agreement.
//
// Visible sets (RedKnot README, "About": each (layer, kv_head) is global /
// local / retrieval / dense, and each head class has its own visible window
// over a per-head page table): a query row at position i of request r sees
//   GLOBAL, DENSE : j <= i
//   LOCAL(W)      : j in [max(0, min(b_q, i - W + 1)), i]
//   RETRIEVAL(S)  : j in [b_q, i]  U  [b_s, b_s + n_s) for the two chosen s
// The table of (r, h) is the ascending list of pages holding any key some
// query row of (r, h) sees; it is a union of at most three page intervals.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SEGKV_HD __host__ __device__ inline
#else
#define SEGKV_HD inline
#endif

namespace segkv {

constexpr int kPage = 16;          // tokens per page
constexpr int kTilePages = 4;      // pages per attention key tile
constexpr int kTileKeys = kPage * kTilePages;
constexpr int kMRows = 256;        // query rows per attention work-group (G heads x 256/G positions)
constexpr int kMaxItemRounds = 4;  // attention work items are at most this many rounds of resident slots
constexpr int kClassGlobal = 0, kClassLocal = 1, kClassRetrieval = 2, kClassDense = 3;

SEGKV_HD int cdiv(int a, int b) { return (a + b - 1) / b; }
SEGKV_HD int imin(int a, int b) { return a < b ? a : b; }
SEGKV_HD int imax(int a, int b) { return a > b ? a : b; }

// Layout facts of one (request, kv head) pair, read from the metadata.
struct HeadView {
  int cls, W;
  int bq, Lq, Lk;      // query segment start/length, context length
  int rlo[2], rhi[2];  // retrieval segments [lo, hi) in tokens
};

// First visible key of a LOCAL row at position i.
SEGKV_HD int local_lo(int i, int bq, int W) { return imax(0, imin(bq, i - W + 1)); }

// Ascending, disjoint, non-adjacent page intervals [lo, hi).
struct PageRuns {
  int n;
  int lo[3], hi[3];
};

SEGKV_HD PageRuns head_page_runs(const HeadView& v) {
  PageRuns pr;
  pr.n = 0;
  pr.lo[0] = pr.hi[0] = pr.lo[1] = pr.hi[1] = pr.lo[2] = pr.hi[2] = 0;
  const int last = cdiv(v.Lk, kPage);
  if (v.cls == kClassLocal) {
    pr.lo[0] = local_lo(v.bq, v.bq, v.W) / kPage;  // lo() is nondecreasing in i
    pr.hi[0] = last;
    pr.n = 1;
  } else if (v.cls == kClassRetrieval) {
    int lo[3] = {v.rlo[0] / kPage, v.rlo[1] / kPage, v.bq / kPage};
    int hi[3] = {cdiv(v.rhi[0], kPage), cdiv(v.rhi[1], kPage), last};
    // sort three intervals by lo (insertion sort), then merge touching ones
    for (int a = 1; a < 3; ++a)
      for (int b = a; b > 0 && lo[b] < lo[b - 1]; --b) {
        int t = lo[b]; lo[b] = lo[b - 1]; lo[b - 1] = t;
        t = hi[b]; hi[b] = hi[b - 1]; hi[b - 1] = t;
      }
    // merge (the three slots are written through constant indices only)
    pr.lo[0] = lo[0];
    pr.hi[0] = hi[0];
    pr.n = 1;
    pr.lo[1] = pr.hi[1] = pr.lo[2] = pr.hi[2] = 0;
    if (lo[1] <= pr.hi[0]) {
      pr.hi[0] = imax(pr.hi[0], hi[1]);
    } else {
      pr.lo[1] = lo[1];
      pr.hi[1] = hi[1];
      pr.n = 2;
    }
    if (pr.n == 1 && lo[2] <= pr.hi[0]) {
      pr.hi[0] = imax(pr.hi[0], hi[2]);
    } else if (pr.n == 2 && lo[2] <= pr.hi[1]) {
      pr.hi[1] = imax(pr.hi[1], hi[2]);
    } else if (pr.n == 1) {
      pr.lo[1] = lo[2];
      pr.hi[1] = hi[2];
      pr.n = 2;
    } else {
      pr.lo[2] = lo[2];
      pr.hi[2] = hi[2];
      pr.n = 3;
    }
  } else {
    pr.lo[0] = 0;
    pr.hi[0] = last;
    pr.n = 1;
  }
  return pr;
}

// (fixed trip counts with guards, so the run arrays stay in registers)
SEGKV_HD int runs_count(const PageRuns& pr) {
  int n = 0;
#pragma unroll
  for (int a = 0; a < 3; ++a)
    if (a < pr.n) n += pr.hi[a] - pr.lo[a];
  return n;
}

// Number of table pages with page index < p.
SEGKV_HD int runs_rank(const PageRuns& pr, int p) {
  int n = 0;
#pragma unroll
  for (int a = 0; a < 3; ++a)
    if (a < pr.n) n += imax(0, imin(p, pr.hi[a]) - pr.lo[a]);
  return n;
}

// Logical page of table entry e (0 <= e < runs_count).
SEGKV_HD int runs_page(const PageRuns& pr, int e) {
  int page = -1;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int len = a < pr.n ? pr.hi[a] - pr.lo[a] : 0;
    if (page < 0 && e < len) page = pr.lo[a] + e;
    e -= len;
  }
  return page;
}

// The 64-key blocks (kTilePages pages) holding any page of a head's table, as
// at most three ascending, disjoint block runs (slots written through constant
// indices only).
SEGKV_HD PageRuns block_runs(const PageRuns& pr) {
  PageRuns b;
  b.lo[1] = b.hi[1] = b.lo[2] = b.hi[2] = 0;
  b.lo[0] = pr.lo[0] / kTilePages;
  b.hi[0] = cdiv(pr.hi[0], kTilePages);
  b.n = 1;
  if (pr.n >= 2) {
    const int lo = pr.lo[1] / kTilePages, hi = cdiv(pr.hi[1], kTilePages);
    if (lo <= b.hi[0]) {
      b.hi[0] = imax(b.hi[0], hi);
    } else {
      b.lo[1] = lo;
      b.hi[1] = hi;
      b.n = 2;
    }
  }
  if (pr.n >= 3) {
    const int lo = pr.lo[2] / kTilePages, hi = cdiv(pr.hi[2], kTilePages);
    if (b.n == 1 && lo <= b.hi[0]) {
      b.hi[0] = imax(b.hi[0], hi);
    } else if (b.n == 1) {
      b.lo[1] = lo;
      b.hi[1] = hi;
      b.n = 2;
    } else if (lo <= b.hi[1]) {
      b.hi[1] = imax(b.hi[1], hi);
    } else {
      b.lo[2] = lo;
      b.hi[2] = hi;
      b.n = 3;
    }
  }
  return b;
}

// Table entry range [e0, e1) (relative to the (r, h) table) that query rows at
// positions [i_lo, i_hi] can see. Rows are never empty: e1 > e0.
SEGKV_HD void mtile_entries(const HeadView& v, const PageRuns& pr, int i_lo, int i_hi, int* e0, int* e1) {
  *e1 = runs_rank(pr, i_hi / kPage + 1);
  *e0 = (v.cls == kClassLocal) ? runs_rank(pr, local_lo(i_lo, v.bq, v.W) / kPage) : 0;
}

// Query positions per m-tile for group size G (G divides kMRows).
SEGKV_HD int mtile_positions(int G) { return kMRows / G; }

// Split of an m-tile's n_tiles key tiles into chunks of at most S tiles, as
// evenly as possible: the first n % k chunks take one tile more than the rest.
SEGKV_HD int num_chunks(int n_tiles, int S) { return imax(1, cdiv(n_tiles, S)); }
SEGKV_HD int chunk_tile_lo(int n_tiles, int n_chunks, int c) {
  const int q = n_tiles / n_chunks, r = n_tiles - q * n_chunks;
  return c * q + imin(c, r);
}

// ---- device plan layout (opaque to callers) ----
struct PlanHeader {
  int32_t n_mtiles, n_items, n_split, chunk_tiles;
  int32_t n_partials, total_q_rows, max_tiles, n_imp_items;
  int32_t pad[8];
};

struct MTile {
  int32_t r, h;
  int32_t q_row0;        // global Q row of the m-tile's first position
  int32_t n_pos;         // valid positions in this m-tile (<= kMRows / G)
  int32_t pos0;          // absolute position of the first row (b_q + t0)
  int32_t cls, W, bq;
  int32_t e_begin, e_end;  // absolute table entries [e_begin, e_end)
  int32_t n_tiles, n_chunks;
  int32_t partial_base;  // first partial slot, -1 when the m-tile is not split
  int32_t pad[3];
};

// An attention work item: one chunk of one m-tile, with the m-tile facts its
// work-group needs, so that the item is the only plan record it reads.
struct Item {
  int32_t mtile, chunk;    // mtile < 0: empty slot, the work-group exits
  int32_t t_lo, T;         // the chunk's key tiles [t_lo, t_lo + T) of the m-tile
  int32_t h, q_row0, n_pos, pos0;
  int32_t cls, W, bq;
  int32_t e_lo;            // absolute table entry of the chunk's first tile
  int32_t e_end;           // absolute table entry past the m-tile's last one
  int32_t partial_slot;    // the chunk's split-KV partial slot, -1 when the m-tile is not split
  int32_t pad[2];
};

// A split m-tile as its combine work-group reads it.
struct SplitTile {
  int32_t partial_base, n_chunks, q_row0, h, n_pos;
  int32_t pad[3];
};

// XCD-aware item order. Work-groups are dispatched round-robin over the 8 XCDs
// of the chip, each with its own L2, so launch slot b runs on XCD b % 8. Items
// are first listed group-major: per (request, kv head) pair, chunk c of every
// m-tile of the pair, then chunk c + 1, ... (holes where an m-tile has fewer
// chunks). The m-tiles of a group read the same key pages. That list is cut
// into 8 equal runs of q8 positions, and run x goes to the slots of XCD x in
// order, so a group's items run side by side on one XCD and share its L2.
constexpr int kXcds = 8;
SEGKV_HD int xcd_slot(int p, int q8) { return kXcds * (p % q8) + p / q8; }

// Importance work item: one 64-key block of one (request, kv head) table,
// with what its work-group needs before it reads the block's page ids.
struct ImpItem {
  int32_t pair, block;
  int32_t cls, W;          // the kv head's class and window
  int32_t bq, Lq;          // the request's query segment: start position and length
  int32_t cu_q, key_off;   // the request's first Q row and first key of the importance vector
  int32_t entry[4];        // table entry of each of the block's 4 pages, -1 when the table has none
};

struct PlanLayout {
  size_t move_off_off;   // int32 [R*Hkv + 1]: first move of each (r, h)
  size_t req_mt_off;     // int32 [R + 1]: first m-tile of each request
  size_t mtiles_off, items_off, split_off, imp_items_off;
  size_t req_key_off;    // int32 [R + 1]: first key of each request in the importance vector
  size_t imp_mask_off;   // uint64 [R][key_blocks]: kv heads whose tables touch each 64-key block
  size_t total;
};

SEGKV_HD size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// key_blocks: 64-key blocks of the longest request.
SEGKV_HD PlanLayout plan_layout(int n_pairs, int n_requests, int n_mtiles, int n_items, int n_split,
                                int n_imp_items, int key_blocks) {
  PlanLayout L;
  L.move_off_off = align256(sizeof(PlanHeader));
  L.req_mt_off = L.move_off_off + align256(sizeof(int32_t) * (size_t)(n_pairs + 1));
  L.mtiles_off = L.req_mt_off + align256(sizeof(int32_t) * (size_t)(n_requests + 1));
  L.items_off = L.mtiles_off + align256(sizeof(MTile) * (size_t)imax(n_mtiles, 1));
  L.split_off = L.items_off + align256(sizeof(Item) * (size_t)imax(n_items, 1));
  L.imp_items_off = L.split_off + align256(sizeof(SplitTile) * (size_t)imax(n_split, 1));
  L.req_key_off = L.imp_items_off + align256(sizeof(ImpItem) * (size_t)imax(n_imp_items, 1));
  L.imp_mask_off = L.req_key_off + align256(sizeof(int32_t) * (size_t)(n_requests + 1));
  L.total = L.imp_mask_off + align256(sizeof(uint64_t) * (size_t)n_requests * (size_t)imax(key_blocks, 1));
  return L;
}

// One partial result slot (one chunk of one split m-tile): kMRows rows of the
// chunk's normalised output O_c / l_c in bf16, then kMRows (m_c, l_c) fp32
// pairs (m in log2 units).
SEGKV_HD size_t partial_o_bytes(int D) { return (size_t)kMRows * (size_t)D * 2; }
SEGKV_HD size_t partial_slot_bytes(int D) { return partial_o_bytes(D) + (size_t)kMRows * 2 * sizeof(float); }

}  // namespace segkv
