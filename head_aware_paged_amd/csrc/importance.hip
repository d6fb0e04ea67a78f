// EXECUTE selection: attention-importance token scores and top-k selection.
//
// RedKnot README "About" (Elastic Sparsity: a token-selective FFN driven by
// attention importance); paooo.com "RedKnot的主要功能" and "RedKnot的核心优势"
// (the top-k tokens by attention score go through the dense FFN, the rest take
// the identity residual).
//
// importance_j = sum over query heads g and the last n_last query rows i of
//   exp(scale * q_{g,i} . k_j - lse_{g,i})  for visible j (else 0).
// One work-group owns 64 consecutive key positions of one request and loops
// over every kv head whose table holds them, so each score is summed in a
// fixed order and no float atomics are needed. Scores come from the gfx950
// 32x32x16 bf16 MFMA; the probabilities stay fp32.
//
// Top-k: radix select (4 passes of 8 bits) on the fp32 bit patterns, which
// order like the values for non-negative scores, then one ordered compaction:
// every key above the threshold plus the lowest-indexed keys equal to it.
#include "common.h"

namespace segkv {
namespace {

constexpr int kImpThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct ImpArgs {
  segkv_meta m;
  const int32_t* cu_q;
  const uint16_t* q;
  const uint16_t* k_pool;
  int64_t pool_pages;
  const int32_t* page_indptr;
  const int32_t* page_ids;
  const float* lse;
  float* importance;
  float scale_log2;
  int R, Hq, Hkv, G, n_last;
};

constexpr int kImpMaxHeads = 64;  // kv heads per request handled by one work-group

template <int D>
__global__ __launch_bounds__(kImpThreads) void importance_kernel(ImpArgs a) {
  constexpr int KS = D / 16;
  constexpr int KCH = D / 8;
  constexpr int kStride = D + 8;
  constexpr int KLOADS = kTileKeys * KCH / kImpThreads;
  __shared__ uint16_t ks_[kTileKeys * kStride];
  __shared__ float colsum[4][kTileKeys];
  __shared__ float s_lse[kImpMaxHeads * 8 * 64 / 8];  // Hq * n_last <= 4096 values
  __shared__ int s_pid[kImpMaxHeads][kTilePages];      // page of each head's table at this key block, -1 if none
  __shared__ int s_cls[kImpMaxHeads], s_W[kImpMaxHeads];

  const int r = blockIdx.y;
  const int sq = a.m.seg_indptr[r + 1] - 1;
  const int bq = a.m.seg_start[sq], Lq = a.m.seg_len[sq], Lk = bq + Lq;
  const int kb0 = blockIdx.x * kTileKeys;
  if (kb0 >= Lk) return;
  int off = 0;  // output offset of request r: sum of earlier context lengths
  for (int rr = 0; rr < r; ++rr) {
    const int s2 = a.m.seg_indptr[rr + 1] - 1;
    off += a.m.seg_start[s2] + a.m.seg_len[s2];
  }
  const int n = imin(a.n_last, Lq);
  const int nb_head = cdiv(n, 32);  // 32-row blocks per query head (rows padded per head)
  const int nrb = a.G * nb_head;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int q_base = a.cu_q[r] + Lq - n;  // first of the last n query rows

  // ---- everything per head that does not depend on the rows, loaded once ----
  for (int x = tid; x < a.Hkv * kTilePages; x += kImpThreads) {
    const int h = x / kTilePages, pp = x % kTilePages;
    const HeadView v = head_view_dev(a.m, a.Hkv, r, h);
    const PageRuns pr = head_page_runs(v);
    const int page = kb0 / kPage + pp;
    const int rk = runs_rank(pr, page);
    int pid = -1;
    if (runs_rank(pr, page + 1) - rk == 1) {
      pid = a.page_ids[a.page_indptr[r * a.Hkv + h] + rk];
      if (pid < 0 || pid >= a.pool_pages) pid = -1;
    }
    s_pid[h][pp] = pid;
    if (pp == 0) {
      s_cls[h] = v.cls;
      s_W[h] = v.W;
    }
  }
  // log2-scaled LSE of the last n rows, [g][t]: all loads of a thread are
  // issued before its stores (a plain loop would wait once per iteration)
  for (int x0 = 0; x0 < a.Hq * n; x0 += 8 * kImpThreads) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = x0 + u * kImpThreads + tid;
      v[u] = x < a.Hq * n ? a.lse[(size_t)(q_base + x % n) * a.Hq + x / n] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = x0 + u * kImpThreads + tid;
      if (x < a.Hq * n) s_lse[x] = v[u] * kLog2e;
    }
  }
  __syncthreads();

  float acc0 = 0.f, acc1 = 0.f;  // keys lrow and 32 + lrow, this lane's rows
  auto active = [&](int h) {
    return s_pid[h][0] >= 0 || s_pid[h][1] >= 0 || s_pid[h][2] >= 0 || s_pid[h][3] >= 0;
  };
  u32x4 kreg[KLOADS];
  auto load_k = [&](int h) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int qd = tid + u * kImpThreads;
      const int key = qd / KCH, c = qd % KCH;
      const int pid = s_pid[h][key >> 4];
      kreg[u] = pid >= 0 ? *reinterpret_cast<const u32x4*>(a.k_pool + ((size_t)pid * kPage + (key & 15)) * D + 8 * c)
                         : u32x4{0, 0, 0, 0};
    }
  };
  int h = 0;
  while (h < a.Hkv && !active(h)) ++h;
  if (h < a.Hkv) load_k(h);
  while (h < a.Hkv) {
    int h_next = h + 1;
    while (h_next < a.Hkv && !active(h_next)) ++h_next;
    __syncthreads();  // previous head's LDS reads are done
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int qd = tid + u * kImpThreads;
      *reinterpret_cast<u32x4*>(&ks_[(qd / KCH) * kStride + 8 * (qd % KCH)]) = kreg[u];
    }
    __syncthreads();
    if (h_next < a.Hkv) load_k(h_next);  // lands while this head computes

    const int cls = s_cls[h], W = s_W[h];
    const int pa = (lrow >> 4) ? s_pid[h][1] : s_pid[h][0], pb = (lrow >> 4) ? s_pid[h][3] : s_pid[h][2];
    const int j0 = pa < 0 ? INT_MAX : kb0 + (lrow >> 4) * kPage + (lrow & 15);
    const int j1 = pb < 0 ? INT_MAX : kb0 + 2 * kPage + (lrow >> 4) * kPage + (lrow & 15);
    for (int rb = wave; rb < nrb; rb += 4) {
      const int hg = rb / nb_head, tb = (rb % nb_head) * 32;
      // A operand: Q of row tb + lrow of head hg (rows past n are clamped, masked below)
      const uint16_t* qp = a.q + ((size_t)(q_base + imin(tb + lrow, n - 1)) * a.Hq + h * a.G + hg) * D + 8 * lg;
      bf16x8 qf[KS];
#pragma unroll
      for (int kstep = 0; kstep < KS; ++kstep) qf[kstep] = *reinterpret_cast<const bf16x8*>(qp + 16 * kstep);
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kstep = 0; kstep < KS; ++kstep)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks_[(32 * kb + lrow) * kStride + 16 * kstep + 8 * lg]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[kstep], kf, s[kb], 0, 0, 0);
        }
      // lane holds keys (j0, j1) for rows t = tb + 8(i/4) + 4 lg + i%4 of head hg
      const float* lse_h = &s_lse[(h * a.G + hg) * n];
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tb + 8 * (i >> 2) + 4 * lg + (i & 3);
        const bool row_ok = t < n;
        const int pos = bq + Lq - n + t;
        const int lo = cls == kClassLocal ? local_lo(pos, bq, W) : 0;
        const float l2 = lse_h[imin(t, n - 1)];
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[0][i], a.scale_log2, -l2));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[1][i], a.scale_log2, -l2));
        p0 += (row_ok && j0 <= pos && j0 >= lo) ? e0 : 0.f;
        p1 += (row_ok && j1 <= pos && j1 >= lo) ? e1 : 0.f;
      }
      acc0 += p0;
      acc1 += p1;
    }
    h = h_next;
  }
  // lanes lg = 0 / 1 hold different rows of the same keys; then waves in order
  acc0 += __shfl_xor(acc0, 32);
  acc1 += __shfl_xor(acc1, 32);
  __syncthreads();
  if (lg == 0) {
    colsum[wave][lrow] = acc0;
    colsum[wave][32 + lrow] = acc1;
  }
  __syncthreads();
  if (tid < kTileKeys) {
    const int j = kb0 + tid;
    if (j < Lk) a.importance[off + j] = ((colsum[0][tid] + colsum[1][tid]) + colsum[2][tid]) + colsum[3][tid];
  }
}

constexpr int kTopkThreads = 1024;

// One work-group selects the top k of one score vector. Vectors of up to
// kTopkCache keys are first copied into LDS, so the four radix passes and the
// compaction read LDS; longer ones are streamed from memory on every pass.
constexpr int kTopkCache = 36864;  // 144 KiB of fp32 keys

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int32_t* idx_out, int n,
                                                            int k) {
  __shared__ uint32_t cache[kTopkCache];
  __shared__ int hist[256];
  __shared__ int s_scan[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  __shared__ int wcnt[2][kTopkThreads / 64][2];
  if (k <= 0) return;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores);
  const int tid = threadIdx.x;
  const bool cached = n <= kTopkCache;
  if (cached) {
    // all loads of a thread in flight together (kTopkCache / 4 / kTopkThreads = 9 vectors at most)
    const int n4 = (reinterpret_cast<uintptr_t>(bits) & 15) == 0 ? n / 4 : 0;
    constexpr int V = (kTopkCache / 4 + kTopkThreads - 1) / kTopkThreads;
    u32x4 v[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int x = u * kTopkThreads + tid;
      if (x < n4) v[u] = reinterpret_cast<const u32x4*>(bits)[x];
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int x = u * kTopkThreads + tid;
      if (x < n4) reinterpret_cast<u32x4*>(cache)[x] = v[u];
    }
    for (int j = 4 * n4 + tid; j < n; j += kTopkThreads) cache[j] = bits[j];
    __syncthreads();
  }
  auto key_at = [&](int j) { return cached ? cache[j] : bits[j]; };
  const int rounds = cdiv(n, kTopkThreads);
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll 4
    for (int w = 0; w < rounds; ++w) {  // uniform trip count: wave votes stay converged
      const int j = tid + w * kTopkThreads;
      const uint32_t key = j < n ? key_at(j) : 0u;
      const bool in = j < n && (key & mask) == prefix;
      const uint32_t bin = (key >> shift) & 255u;
      // skewed digits (the exponent byte) would serialise 64 lanes on one LDS
      // counter: a wave whose candidates all share one bin adds them at once
      const uint32_t b0 = __builtin_amdgcn_readfirstlane(in ? bin : 256u);
      const uint64_t cand = __ballot(in);
      const uint64_t same = __ballot(in && bin == b0);
      if (cand != 0 && same == cand) {
        if (__lane_id() == (uint32_t)__builtin_ctzll(cand)) atomicAdd(&hist[b0], (int)__popcll(cand));
      } else if (in) {
        atomicAdd(&hist[bin], 1);
      }
    }
    __syncthreads();
    // digit holding the krem-th largest candidate: suffix sums over the 256 bins
    const int c = tid < 256 ? hist[tid] : 0;
    if (tid < 256) s_scan[tid] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive suffix sum (bins above and including tid)
      const int t = (tid < 256 && tid + o < 256) ? s_scan[tid + o] : 0;
      __syncthreads();
      if (tid < 256) s_scan[tid] += t;
      __syncthreads();
    }
    if (tid < 256) {
      const int above = s_scan[tid] - c;
      if (above < krem && krem <= s_scan[tid]) {
        s_prefix = prefix | ((uint32_t)tid << shift);
        s_krem = krem - above;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix = the k-th largest key: take all keys > prefix and the first krem keys
  // == prefix, in index order. Round w covers keys [1024 w, 1024 w + 1024); a
  // wave's 64 consecutive keys are ranked with ballots, waves with LDS counts.
  const int wave = tid >> 6, lane = tid & 63;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int gt_carry = 0, eq_carry = 0;  // selected-above and tied keys in earlier rounds
  for (int w = 0; w < rounds; ++w) {
    const int j = tid + w * kTopkThreads;
    const uint32_t key = j < n ? key_at(j) : 0u;
    const bool gt = j < n && key > prefix;
    const bool eq = j < n && key == prefix;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    const int buf = w & 1;
    if (lane == 0) {
      wcnt[buf][wave][0] = __popcll(bgt);
      wcnt[buf][wave][1] = __popcll(beq);
    }
    __syncthreads();
    int gt_before = gt_carry + __popcll(bgt & lt_mask), eq_before = eq_carry + __popcll(beq & lt_mask);
    int gt_round = 0, eq_round = 0;
    for (int v = 0; v < kTopkThreads / 64; ++v) {
      const int g = wcnt[buf][v][0], e = wcnt[buf][v][1];
      if (v < wave) {
        gt_before += g;
        eq_before += e;
      }
      gt_round += g;
      eq_round += e;
    }
    if (gt || (eq && eq_before < krem)) idx_out[gt_before + imin(eq_before, krem)] = j;
    gt_carry += gt_round;
    eq_carry += eq_round;
  }
}

int32_t launch_topk(const float* scores, int32_t* idx, int n, int k, hipStream_t s) {
  if (k <= 0) return SEGKV_OK;
  topk_kernel<<<1, kTopkThreads, 0, s>>>(scores, idx, n, k);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" int32_t token_importance_topk(const segkv_dims* dims, const segkv_meta* meta_host,
                                         const segkv_meta* meta_dev, const int32_t* cu_q_dev, const void* q,
                                         const void* k_pool, int64_t pool_pages, const int32_t* page_indptr_dev,
                                         const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                         const float* lse_dev, float softmax_scale, int32_t n_last,
                                         const int32_t* k_host, float* importance_dev, int32_t* topk_idx_dev,
                                         void* stream) {
  clear_error();
  HostPlan hp;
  int32_t st = compute_host_plan(dims, meta_host, &hp);
  if (st != SEGKV_OK) return st;
  if (!meta_dev || !meta_dev->seg_indptr || !cu_q_dev || !q || !k_pool || !page_indptr_dev || !page_ids_dev ||
      !page_pos_dev || !lse_dev || !importance_dev)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (n_last <= 0) return fail(SEGKV_ERR_INVALID_ARG, "n_last must be > 0");
  const int G = dims->num_q_heads / dims->num_kv_heads;
  if (dims->num_kv_heads > kImpMaxHeads) return fail(SEGKV_ERR_UNSUPPORTED, "num_kv_heads must be <= 64");
  if ((int64_t)dims->num_q_heads * n_last > 4096)
    return fail(SEGKV_ERR_UNSUPPORTED, "num_q_heads * n_last must be <= 4096");
  if (!(softmax_scale > 0.f)) return fail(SEGKV_ERR_INVALID_ARG, "softmax_scale must be > 0");
  if (pool_pages <= 0) return fail(SEGKV_ERR_INVALID_ARG, "pool_pages must be > 0");
  if (!aligned16(q) || !aligned16(k_pool)) return fail(SEGKV_ERR_ALIGNMENT, "q and k_pool must be 16-byte aligned");
  const int R = dims->num_requests;
  int max_lk = 0;
  for (int r = 0; r < R; ++r) {
    const int sq = meta_host->seg_indptr[r + 1] - 1;
    max_lk = imax(max_lk, meta_host->seg_start[sq] + meta_host->seg_len[sq]);
  }
  if (topk_idx_dev != nullptr) {
    if (k_host == nullptr) return fail(SEGKV_ERR_INVALID_ARG, "k is NULL");
    for (int r = 0; r < R; ++r) {
      const int sq = meta_host->seg_indptr[r + 1] - 1;
      const int lk = meta_host->seg_start[sq] + meta_host->seg_len[sq];
      if (k_host[r] < 0 || k_host[r] > lk) return fail(SEGKV_ERR_INVALID_ARG, "k must be in [0, L_k]");
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  ImpArgs a;
  a.m = *meta_dev;
  a.cu_q = cu_q_dev;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.pool_pages = pool_pages;
  a.page_indptr = page_indptr_dev;
  a.page_ids = page_ids_dev;
  a.lse = lse_dev;
  a.importance = importance_dev;
  a.scale_log2 = softmax_scale * kLog2e;
  a.R = R;
  a.Hq = dims->num_q_heads;
  a.Hkv = dims->num_kv_heads;
  a.G = G;
  a.n_last = n_last;
  dim3 grid(cdiv(max_lk, kTileKeys), R);
  if (dims->head_dim == 128)
    importance_kernel<128><<<grid, kImpThreads, 0, s>>>(a);
  else
    importance_kernel<64><<<grid, kImpThreads, 0, s>>>(a);
  SEGKV_LAUNCH_CHECK();
  if (topk_idx_dev == nullptr) return SEGKV_OK;
  // one selection per request on the same stream (host knows every offset)
  int64_t off = 0, koff = 0;
  for (int r = 0; r < R; ++r) {
    const int sq = meta_host->seg_indptr[r + 1] - 1;
    const int lk = meta_host->seg_start[sq] + meta_host->seg_len[sq];
    st = launch_topk(importance_dev + off, topk_idx_dev + koff, lk, k_host[r], s);
    if (st != SEGKV_OK) return st;
    off += lk;
    koff += k_host[r];
  }
  return SEGKV_OK;
}

extern "C" int32_t segkv_topk_select(const float* scores_dev, int32_t n, int32_t k, int32_t* idx_dev,
                                     void* stream) {
  clear_error();
  if (n < 0 || k < 0 || k > n) return fail(SEGKV_ERR_INVALID_ARG, "need 0 <= k <= n");
  if (k == 0) return SEGKV_OK;
  if (!scores_dev || !idx_dev) return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  return launch_topk(scores_dev, idx_dev, n, k, static_cast<hipStream_t>(stream));
}
