// Host side of libsegkv: status strings, argument validation and the host
// mirror of the attention plan (sizes and chunking decisions).
#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "common.h"

namespace segkv {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
int32_t fail(int32_t code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

#define REQUIRE(cond, code, msg)          \
  do {                                    \
    if (!(cond)) return fail((code), (msg)); \
  } while (0)

int32_t validate_layout(const segkv_dims* d, const segkv_meta* m) {
  REQUIRE(d != nullptr, SEGKV_ERR_INVALID_ARG, "dims is NULL");
  REQUIRE(m != nullptr, SEGKV_ERR_INVALID_ARG, "host metadata is NULL");
  REQUIRE(d->num_requests > 0 && d->num_q_heads > 0 && d->num_kv_heads > 0 && d->head_dim > 0 &&
              d->page_size > 0 && d->num_segments > 0,
          SEGKV_ERR_INVALID_ARG, "every dimension must be positive");
  REQUIRE(d->num_q_heads % d->num_kv_heads == 0, SEGKV_ERR_INVALID_ARG,
          "num_q_heads must be a multiple of num_kv_heads");
  REQUIRE(d->head_dim == 64 || d->head_dim == 128, SEGKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  REQUIRE(d->page_size == kPage, SEGKV_ERR_UNSUPPORTED, "page_size must be 16");
  const int G = d->num_q_heads / d->num_kv_heads;
  REQUIRE(G <= kMRows && kMRows % G == 0, SEGKV_ERR_UNSUPPORTED, "group size Hq/Hkv must divide 256");
  REQUIRE(m->seg_indptr && m->seg_start && m->seg_len && m->head_class && m->window && m->retr_seg,
          SEGKV_ERR_INVALID_ARG, "a metadata array is NULL");
  const int R = d->num_requests, S = d->num_segments, Hkv = d->num_kv_heads;
  REQUIRE(m->seg_indptr[0] == 0 && m->seg_indptr[R] == S, SEGKV_ERR_INVALID_ARG,
          "seg_indptr must start at 0 and end at num_segments");
  for (int r = 0; r < R; ++r) {
    const int s0 = m->seg_indptr[r], s1 = m->seg_indptr[r + 1];
    REQUIRE(s1 > s0, SEGKV_ERR_INVALID_ARG, "request " + std::to_string(r) + " has no segment");
    int64_t pos = 0;
    for (int s = s0; s < s1; ++s) {
      REQUIRE(m->seg_len[s] > 0, SEGKV_ERR_INVALID_ARG, "segment " + std::to_string(s) + " is empty");
      REQUIRE(m->seg_start[s] == pos, SEGKV_ERR_INVALID_ARG,
              "segment " + std::to_string(s) + " does not start where the previous one ends");
      REQUIRE(m->seg_start[s] % kPage == 0, SEGKV_ERR_INVALID_ARG,
              "segment " + std::to_string(s) + " start is not page-aligned");
      pos += m->seg_len[s];
    }
    REQUIRE(pos <= (1 << 24), SEGKV_ERR_UNSUPPORTED, "context longer than 2^24 tokens");
    for (int h = 0; h < Hkv; ++h) {
      const int k = r * Hkv + h;
      const int c = m->head_class[k];
      REQUIRE(c >= 0 && c <= 3, SEGKV_ERR_INVALID_ARG, "unknown head class at (" + std::to_string(r) + ", " +
                                                          std::to_string(h) + ")");
      if (c == kClassLocal)
        REQUIRE(m->window[k] > 0, SEGKV_ERR_INVALID_ARG, "LOCAL head needs window > 0");
      if (c == kClassRetrieval) {
        const int a = m->retr_seg[2 * k], b = m->retr_seg[2 * k + 1];
        REQUIRE(a >= s0 && a < s1 - 1 && b >= s0 && b < s1 - 1, SEGKV_ERR_INVALID_ARG,
                "RETRIEVAL segments must be reused segments of the same request");
        REQUIRE(a != b, SEGKV_ERR_INVALID_ARG, "RETRIEVAL segments must be distinct");
      }
    }
  }
  return SEGKV_OK;
}

HeadView head_view_host(const segkv_dims& d, const segkv_meta& m, int r, int h) {
  HeadView v;
  const int sq = m.seg_indptr[r + 1] - 1;
  v.bq = m.seg_start[sq];
  v.Lq = m.seg_len[sq];
  v.Lk = v.bq + v.Lq;
  const int k = r * d.num_kv_heads + h;
  v.cls = m.head_class[k];
  v.W = m.window[k];
  v.rlo[0] = v.rhi[0] = v.rlo[1] = v.rhi[1] = 0;
  if (v.cls == kClassRetrieval)
    for (int a = 0; a < 2; ++a) {
      const int s = m.retr_seg[2 * k + a];
      v.rlo[a] = m.seg_start[s];
      v.rhi[a] = m.seg_start[s] + m.seg_len[s];
    }
  return v;
}

int attention_slots() {
  // Resident attention work-groups: 1 per CU (512 threads, two waves per SIMD).
  static std::once_flag once;
  static int cus = 256;
  std::call_once(once, [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    (void)hipGetLastError();
  });
  return cus;
}

// Greedy longest-processing-time schedule of `sizes` on `bins` identical slots.
static int64_t lpt_makespan(std::vector<int>& sizes, int bins) {
  std::sort(sizes.begin(), sizes.end(), std::greater<int>());
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> q;
  for (int b = 0; b < bins; ++b) q.push(0);
  int64_t mk = 0;
  for (int s : sizes) {
    int64_t t = q.top() + s;
    q.pop();
    q.push(t);
    mk = std::max(mk, t);
  }
  return mk;
}

// Chunk cap S (tiles per work item): balance items over the resident slots
// while keeping the number of split-KV partials small. Splits serve the
// balance only (at most 4 rounds of slots), so the partials are bounded by
// the slot count, not by query rows x keys.
static int choose_chunk_tiles(const std::vector<int>& tiles, int slots) {
  int64_t total = 0;
  int tmax = 1;
  for (int t : tiles) {
    total += t;
    tmax = std::max(tmax, t);
  }
  auto items_for = [&](int S) {
    int64_t n = 0;
    for (int t : tiles) n += num_chunks(t, S);
    return n;
  };
  int best_S = tmax;
  double best_cost = 1e300;
  for (int rounds = 1; rounds <= kMaxItemRounds; ++rounds) {
    const int64_t target = (int64_t)rounds * slots;
    int lo = (int)std::max<int64_t>(1, (total + target - 1) / target), hi = tmax;
    if (lo > hi) lo = hi;
    while (lo < hi) {  // smallest S with items_for(S) <= target (items_for is nonincreasing)
      int mid = lo + (hi - lo) / 2;
      if (items_for(mid) <= target) hi = mid; else lo = mid + 1;
    }
    const int S = lo;
    std::vector<int> sizes;
    int64_t partials = 0;
    for (int t : tiles) {
      const int k = num_chunks(t, S);
      if (k > 1) partials += k;
      for (int c = 0; c < k; ++c) sizes.push_back(chunk_tile_lo(t, k, c + 1) - chunk_tile_lo(t, k, c));
    }
    // one partial costs about one key tile of extra traffic, spread over all slots
    const double cost = (double)lpt_makespan(sizes, slots) + 2.0 * (double)partials / slots;
    if (cost < best_cost) {
      best_cost = cost;
      best_S = S;
    }
  }
  return best_S;
}

static int32_t plan_layout_uncached(const segkv_dims* d, const segkv_meta* m, HostPlan* out) {
  HostPlan p;
  const int R = d->num_requests, Hkv = d->num_kv_heads;
  const int G = d->num_q_heads / Hkv;
  const int MP = mtile_positions(G);
  std::vector<int> tiles, pair_of_mtile;
  for (int r = 0; r < R; ++r) {
    for (int h = 0; h < Hkv; ++h) {
      const HeadView v = head_view_host(*d, *m, r, h);
      const PageRuns pr = head_page_runs(v);
      const int cnt = runs_count(pr);
      p.table_entries += cnt;
      p.n_imp_items += runs_count(block_runs(pr));
      p.move_entries += runs_rank(pr, v.bq / kPage);
      if (h == 0) {
        p.total_q_rows += v.Lq;
        p.total_keys += v.Lk;
        p.key_blocks = std::max(p.key_blocks, cdiv(v.Lk, kTileKeys));
      }
      for (int t0 = 0; t0 < v.Lq; t0 += MP) {
        const int i_lo = v.bq + t0, i_hi = v.bq + imin(v.Lq, t0 + MP) - 1;
        int e0, e1;
        mtile_entries(v, pr, i_lo, i_hi, &e0, &e1);
        tiles.push_back(cdiv(e1 - e0, kTilePages));
        pair_of_mtile.push_back(r * Hkv + h);
      }
    }
  }
  REQUIRE(p.table_entries < (int64_t)1 << 31, SEGKV_ERR_UNSUPPORTED, "more than 2^31 table entries");
  p.n_mtiles = (int)tiles.size();
  p.chunk_tiles = choose_chunk_tiles(tiles, attention_slots());
  int64_t positions = 0;  // group-major item positions (holes included)
  for (size_t i0 = 0; i0 < tiles.size();) {
    // the m-tiles of one (request, kv head) pair are consecutive
    size_t i1 = i0;
    int maxc = 0;
    while (i1 < tiles.size() && pair_of_mtile[i1] == pair_of_mtile[i0]) {
      maxc = std::max(maxc, num_chunks(tiles[i1], p.chunk_tiles));
      ++i1;
    }
    positions += (int64_t)maxc * (int64_t)(i1 - i0);
    i0 = i1;
  }
  for (int t : tiles) {
    const int k = num_chunks(t, p.chunk_tiles);
    p.max_tiles = std::max(p.max_tiles, t);
    if (k > 1) {
      ++p.n_split;
      p.n_partials += k;
    }
  }
  REQUIRE(positions < (int64_t)1 << 30, SEGKV_ERR_UNSUPPORTED, "too many attention work items");
  p.n_items = kXcds * (int)((positions + kXcds - 1) / kXcds);
  const PlanLayout L = host_plan_layout(*d, p);
  p.plan_bytes = L.total;
  p.workspace_bytes = (size_t)p.n_partials * partial_slot_bytes(d->head_dim);
  *out = p;
  return SEGKV_OK;
}

// The host plan of a layout, cached: every entry point of a layer (page build,
// attention, importance) plans the same layout, once per call, so the last few
// layouts' plans are kept, keyed by the complete layout (dims, every metadata
// array and the slot count).
int32_t compute_host_plan(const segkv_dims* d, const segkv_meta* m, HostPlan* out) {
  int32_t st = validate_layout(d, m);
  if (st != SEGKV_OK) return st;
  const int R = d->num_requests, S = d->num_segments, RH = R * d->num_kv_heads;
  std::vector<int32_t> key = {d->num_requests, d->num_q_heads, d->num_kv_heads, d->head_dim, d->page_size,
                              d->num_segments, attention_slots()};
  key.reserve(key.size() + (R + 1) + 2 * S + 4 * RH);
  key.insert(key.end(), m->seg_indptr, m->seg_indptr + R + 1);
  key.insert(key.end(), m->seg_start, m->seg_start + S);
  key.insert(key.end(), m->seg_len, m->seg_len + S);
  for (int k = 0; k < RH; ++k) key.push_back(m->head_class[k]);
  key.insert(key.end(), m->window, m->window + RH);
  key.insert(key.end(), m->retr_seg, m->retr_seg + 2 * RH);
  static std::mutex mu;
  static std::vector<std::pair<std::vector<int32_t>, HostPlan>> cache;  // most recent last
  constexpr size_t kCacheLayouts = 16;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (size_t i = 0; i < cache.size(); ++i)
      if (cache[i].first == key) {
        *out = cache[i].second;
        if (i + 1 != cache.size()) std::rotate(cache.begin() + i, cache.begin() + i + 1, cache.end());
        return SEGKV_OK;
      }
  }
  HostPlan p;
  st = plan_layout_uncached(d, m, &p);
  if (st != SEGKV_OK) return st;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() == kCacheLayouts) cache.erase(cache.begin());
    cache.emplace_back(std::move(key), p);
  }
  *out = p;
  return SEGKV_OK;
}

}  // namespace segkv

using namespace segkv;

extern "C" const char* segkv_status_string(int32_t s) {
  switch (s) {
    case SEGKV_OK: return "SEGKV_OK";
    case SEGKV_ERR_INVALID_ARG: return "SEGKV_ERR_INVALID_ARG";
    case SEGKV_ERR_UNSUPPORTED: return "SEGKV_ERR_UNSUPPORTED";
    case SEGKV_ERR_CAPACITY: return "SEGKV_ERR_CAPACITY";
    case SEGKV_ERR_ALIGNMENT: return "SEGKV_ERR_ALIGNMENT";
    case SEGKV_ERR_WORKSPACE: return "SEGKV_ERR_WORKSPACE";
    case SEGKV_ERR_HIP: return "SEGKV_ERR_HIP";
    case SEGKV_ERR_DEVICE_CHECK: return "SEGKV_ERR_DEVICE_CHECK";
    default: return "SEGKV_ERR_UNKNOWN";
  }
}

extern "C" const char* segkv_last_error(void) { return g_last_error.c_str(); }

extern "C" int32_t segkv_plan_sizes(const segkv_dims* dims, const segkv_meta* meta_host, segkv_sizes* sizes) {
  clear_error();
  if (sizes == nullptr) return fail(SEGKV_ERR_INVALID_ARG, "sizes is NULL");
  HostPlan p;
  int32_t st = compute_host_plan(dims, meta_host, &p);
  if (st != SEGKV_OK) return st;
  sizes->table_entries = p.table_entries;
  sizes->move_entries = p.move_entries;
  sizes->total_q_rows = p.total_q_rows;
  sizes->total_keys = p.total_keys;
  sizes->plan_bytes = p.plan_bytes;
  sizes->attn_workspace_bytes = p.workspace_bytes;
  sizes->importance_workspace_bytes = importance_workspace_bytes(*dims, p.total_keys);
  return SEGKV_OK;
}
