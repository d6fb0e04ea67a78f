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

template <int D>
__global__ __launch_bounds__(kImpThreads) void importance_kernel(ImpArgs a) {
  constexpr int KS = D / 16;
  constexpr int KCH = D / 8;
  constexpr int kStride = D + 8;
  constexpr int KLOADS = kTileKeys * KCH / kImpThreads;
  __shared__ uint16_t ks_[kTileKeys * kStride];
  __shared__ float colsum[4][kTileKeys];
  __shared__ int s_pos[kTilePages];
  __shared__ float s_lse[kMRows * 4];  // G * n_last <= 512 rows

  const int r = blockIdx.y;
  const int sq = a.m.seg_indptr[r + 1] - 1;
  const int bq = a.m.seg_start[sq], Lq = a.m.seg_len[sq], Lk = bq + Lq;
  const int kb0 = blockIdx.x * kTileKeys;
  if (kb0 >= Lk) return;
  // output offset of request r: sum of earlier context lengths
  int off = 0;
  for (int rr = 0; rr < r; ++rr) {
    const int s2 = a.m.seg_indptr[rr + 1] - 1;
    off += a.m.seg_start[s2] + a.m.seg_len[s2];
  }
  const int n = imin(a.n_last, Lq);
  const int nb_head = cdiv(n, 32);  // 32-row blocks per query head (rows padded per head)
  const int nrb = a.G * nb_head;
  const int rows = a.G * n;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  float acc0 = 0.f, acc1 = 0.f;  // keys lrow and 32 + lrow, this lane's rows

  for (int h = 0; h < a.Hkv; ++h) {
    const HeadView v = head_view_dev(a.m, a.Hkv, r, h);
    const PageRuns pr = head_page_runs(v);
    const int base = a.page_indptr[r * a.Hkv + h];
    int pids[kTilePages], ppos[kTilePages];
    bool any = false;
#pragma unroll
    for (int pp = 0; pp < kTilePages; ++pp) {
      const int page = kb0 / kPage + pp;
      const int rk = runs_rank(pr, page);
      const bool in = (runs_rank(pr, page + 1) - rk) == 1;
      int pid = in ? a.page_ids[base + rk] : -1;
      if (pid >= a.pool_pages) pid = -1;
      pids[pp] = pid;
      ppos[pp] = pid >= 0 ? page * kPage : INT_MAX;
      any = any || pid >= 0;
    }
    if (!any) continue;  // uniform across the block
    __syncthreads();     // previous head's LDS reads are done
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int qd = tid + u * kImpThreads;
      const int key = qd / KCH, c = qd % KCH;
      const int pg = key >> 4;
      const int pid = pg == 0 ? pids[0] : pg == 1 ? pids[1] : pg == 2 ? pids[2] : pids[3];
      u32x4 val = {0, 0, 0, 0};
      if (pid >= 0) val = *reinterpret_cast<const u32x4*>(a.k_pool + ((size_t)pid * kPage + (key & 15)) * D + 8 * c);
      *reinterpret_cast<u32x4*>(&ks_[key * kStride + 8 * c]) = val;
    }
    for (int x = tid; x < rows; x += kImpThreads) {
      const int hg = x / n, t = x % n;
      const int qrow = a.cu_q[r] + Lq - n + t;
      s_lse[x] = a.lse[(size_t)qrow * a.Hq + h * a.G + hg] * kLog2e;
    }
    __syncthreads();
    // key positions of this lane (INT_MAX: page not in the table)
    const int pa = (lrow >> 4) ? ppos[1] : ppos[0], pb = (lrow >> 4) ? ppos[3] : ppos[2];
    const int j0 = pa == INT_MAX ? INT_MAX : pa + (lrow & 15);
    const int j1 = pb == INT_MAX ? INT_MAX : pb + (lrow & 15);

    for (int rb = wave; rb < nrb; rb += 4) {
      const int hg = rb / nb_head, tb = (rb % nb_head) * 32;
      // A operand: Q of row tb + lrow of head hg (rows past n are clamped, masked below)
      const int qrow = a.cu_q[r] + Lq - n + imin(tb + lrow, n - 1);
      const uint16_t* qp = a.q + ((size_t)qrow * a.Hq + h * a.G + hg) * D + 8 * lg;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kstep = 0; kstep < KS; ++kstep) {
        const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qp + 16 * kstep);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks_[(32 * kb + lrow) * kStride + 16 * kstep + 8 * lg]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf, s[kb], 0, 0, 0);
        }
      }
      // lane holds keys (j0, j1) for rows t = tb + 8(i/4) + 4 lg + i%4 of head hg
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tb + 8 * (i >> 2) + 4 * lg + (i & 3);
        const bool row_ok = t < n;
        const int pos = bq + Lq - n + t;
        const int lo = v.cls == kClassLocal ? local_lo(pos, v.bq, v.W) : 0;
        const float l2 = s_lse[hg * n + imin(t, n - 1)];
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[0][i], a.scale_log2, -l2));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[1][i], a.scale_log2, -l2));
        p0 += (row_ok && j0 <= pos && j0 >= lo) ? e0 : 0.f;
        p1 += (row_ok && j1 <= pos && j1 >= lo) ? e1 : 0.f;
      }
      acc0 += p0;
      acc1 += p1;
    }
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

// One work-group selects the top k of one score vector. ITEMS > 0: every
// thread keeps its ITEMS strided keys in registers across the radix passes;
// ITEMS == 0: the passes stream the keys from memory.
template <int ITEMS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int32_t* idx_out,
                                                            int n, int k) {
  __shared__ int hist[256];
  __shared__ int s_scan[kTopkThreads];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  if (k <= 0) return;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores);
  const int tid = threadIdx.x;
  constexpr int kCache = ITEMS > 0 ? ITEMS : 1;
  uint32_t kv[kCache];
  if (ITEMS > 0) {
#pragma unroll
    for (int u = 0; u < kCache; ++u) {
      const int j = tid + u * kTopkThreads;
      kv[u] = j < n ? bits[j] : 0u;
    }
  }
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  const int rounds = ITEMS > 0 ? ITEMS : cdiv(n, kTopkThreads);
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (ITEMS > 0 ? kCache : 1); ++u) {
      for (int v = 0; v < (ITEMS > 0 ? 1 : rounds); ++v) {  // uniform trip counts: wave votes stay converged
        const int w = ITEMS > 0 ? u : v;
        const int j = tid + w * kTopkThreads;
        const uint32_t key = ITEMS > 0 ? kv[u] : (j < n ? bits[j] : 0u);
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
    }
    __syncthreads();
    // digit d holding the krem-th largest candidate: suffix sums over the 256 bins
    const int c = tid < 256 ? hist[tid] : 0;
    s_scan[tid] = c;
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
  __shared__ int wcnt[2][kTopkThreads / 64][2];
  const int wave = tid >> 6, lane = tid & 63;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int gt_carry = 0, eq_carry = 0;  // selected-above and tied keys in earlier rounds
  for (int w = 0; w < rounds; ++w) {
    const int j = tid + w * kTopkThreads;
    uint32_t key = 0;
    if (ITEMS > 0) {
#pragma unroll
      for (int u = 0; u < kCache; ++u)
        if (u == w) key = kv[u];
    } else {
      key = j < n ? bits[j] : 0u;
    }
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
  if (n <= 4 * kTopkThreads)
    topk_kernel<4><<<1, kTopkThreads, 0, s>>>(scores, idx, n, k);
  else if (n <= 16 * kTopkThreads)
    topk_kernel<16><<<1, kTopkThreads, 0, s>>>(scores, idx, n, k);
  else if (n <= 64 * kTopkThreads)
    topk_kernel<64><<<1, kTopkThreads, 0, s>>>(scores, idx, n, k);
  else
    topk_kernel<0><<<1, kTopkThreads, 0, s>>>(scores, idx, n, k);
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
  if ((int64_t)G * n_last > 512) return fail(SEGKV_ERR_UNSUPPORTED, "(Hq/Hkv) * n_last must be <= 512");
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
