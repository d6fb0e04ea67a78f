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
constexpr int kImpWaves = kImpThreads / 64;
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
  const char* plan;     // attention plan of the layout (its importance item list)
  PlanLayout L;
  float* partial;       // workspace [Hkv][total_keys]: per-kv-head importance
  float* importance;
  int64_t total_keys;
  float scale_log2;
  int R, Hq, Hkv, G, n_last;
};

constexpr int kImpMaxLse = 4096;  // Hq * (n_last rounded up to 32) values (bounds one head's G * NP)

// One work-group per importance item of the plan: a 64-key block that one
// (request, kv head) table touches. It computes that head's share of the
// block's importance as (32-row block of one of its G query heads) units,
// wave w taking units [U w / 4, U (w + 1) / 4), and writes the block's 64
// partial sums; a second kernel adds, key by key, the partials of the heads
// whose tables touch the key's block, in head order. Each score is thus summed
// in a fixed order with no float atomics. K and Q fragments go from memory
// straight into MFMA operand registers; the next unit's Q is in flight while
// the current one computes; units whose 32 rows see all 64 keys skip every
// mask.
template <int D>
__global__ __launch_bounds__(kImpThreads, 3) void importance_kernel(ImpArgs a) {
  constexpr int KS = D / 16;
  constexpr int KCH = D / 8;            // 16-byte chunks per key row
  constexpr int kStride = D + 8;        // padded LDS row (elements)
  constexpr int KLOADS = kTileKeys * KCH / kImpThreads;
  __shared__ __attribute__((aligned(16))) uint16_t ks[kTileKeys * kStride];
  __shared__ __attribute__((aligned(16))) float s_lse[kImpMaxLse];
  __shared__ int s_pid[kTilePages];  // this head's page at each page of the key block, -1 if none
  __shared__ float colsum[kImpWaves][kTileKeys];

  const ImpItem item = reinterpret_cast<const ImpItem*>(a.plan + a.L.imp_items_off)[blockIdx.x];
  if (item.pair < 0 || item.pair >= a.R * a.Hkv || item.block < 0) return;  // not a plan of this layout
  const int r = item.pair / a.Hkv, hh = item.pair % a.Hkv;
  const int sq = a.m.seg_indptr[r + 1] - 1;
  const int bq = a.m.seg_start[sq], Lq = a.m.seg_len[sq], Lk = bq + Lq;
  const int kb0 = item.block * kTileKeys;
  if (kb0 >= Lk) return;
  const int n = imin(a.n_last, Lq);
  const int nb_head = cdiv(n, 32);  // 32-row blocks per query head
  const int NP = 32 * nb_head;      // staged rows per query head (the last row repeated)
  const int U = a.G * nb_head;      // units of this kv head
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int q_base = a.cu_q[r] + Lq - n;  // first of the last n query rows
  const int pos_base = Lk - n;            // its position
  const int u_lo = U * wave / kImpWaves, u_hi = U * (wave + 1) / kImpWaves;

  // the wave's first Q fragment (A operand: Q row tb + lrow of query head hg)
  // is requested before the page lookups, so its latency overlaps them
  bf16x8 qa[KS];
  auto q_load = [&](bf16x8* dst, int uu) {
    const int hg = uu / nb_head, tb = (uu % nb_head) * 32;
    const uint16_t* qp = a.q + ((size_t)(q_base + imin(tb + lrow, n - 1)) * a.Hq + hh * a.G + hg) * D + 8 * lg;
#pragma unroll
    for (int k8 = 0; k8 < KS; ++k8) dst[k8] = *reinterpret_cast<const bf16x8*>(qp + 16 * k8);
  };
  if (u_lo < u_hi) q_load(qa, u_lo);

  const HeadView v = head_view_dev(a.m, a.Hkv, r, hh);
  if (tid < kTilePages) {
    const PageRuns pr = head_page_runs(v);
    const int page = kb0 / kPage + tid;
    const int rk = runs_rank(pr, page);
    int pid = -1;
    if (runs_rank(pr, page + 1) - rk == 1) {
      pid = a.page_ids[a.page_indptr[r * a.Hkv + hh] + rk];
      if (pid < 0 || pid >= a.pool_pages) pid = -1;
    }
    s_pid[tid] = pid;
  }
  // log2-scaled LSE of the last n rows of this head's G query heads, [g][t]
  // with t < NP (rows past n repeat row n - 1); loads first, then stores
  for (int x0 = 0; x0 < a.G * NP; x0 += 4 * kImpThreads) {
    float lv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = x0 + u * kImpThreads + tid;
      lv[u] = x < a.G * NP ? a.lse[(size_t)(q_base + imin(x % NP, n - 1)) * a.Hq + hh * a.G + x / NP] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = x0 + u * kImpThreads + tid;
      if (x < a.G * NP) s_lse[x] = lv[u] * kLog2e;
    }
  }
  __syncthreads();
  // K tile -> LDS (rows of missing pages are zero)
  {
    u32x4 kr[KLOADS];
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int qd = tid + u * kImpThreads, key = qd / KCH, c = qd % KCH;
      const int pid = s_pid[key >> 4];
      kr[u] = pid >= 0 ? *reinterpret_cast<const u32x4*>(a.k_pool + ((size_t)pid * kPage + (key & 15)) * D + 8 * c)
                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int qd = tid + u * kImpThreads;
      *reinterpret_cast<u32x4*>(&ks[(qd / KCH) * kStride + 8 * (qd % KCH)]) = kr[u];
    }
  }
  __syncthreads();

  const int cls = v.cls, W = v.W;
  const bool pages_full = s_pid[0] >= 0 && s_pid[1] >= 0 && s_pid[2] >= 0 && s_pid[3] >= 0;
  const int pa = s_pid[lrow >> 4], pb = s_pid[2 + (lrow >> 4)];
  const int j0 = pa < 0 ? INT_MAX : kb0 + lrow;
  const int j1 = pb < 0 ? INT_MAX : kb0 + 32 + lrow;

  float acc0 = 0.f, acc1 = 0.f;  // keys lrow and 32 + lrow, this lane's rows
  // unit uu with Q in qa; once its MFMAs have read qa, the next unit's Q is
  // requested into qa, so that load overlaps this unit's exponentials
  auto unit = [&](int uu) {
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
#pragma unroll
    for (int k8 = 0; k8 < KS; ++k8) {  // B operand: key 32 kb + lrow, dims 16 k8 + 8 lg .. + 8
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(&ks[lrow * kStride + 16 * k8 + 8 * lg]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(&ks[(32 + lrow) * kStride + 16 * k8 + 8 * lg]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[k8], k0, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[k8], k1, s1, 0, 0, 0);
    }
    if (uu + 1 < u_hi) q_load(qa, uu + 1);
    // lane holds keys (j0, j1) for rows t = tb + 8(i/4) + 4 lg + i%4 of query head hg
    const int hg = uu / nb_head, tb = (uu % nb_head) * 32;
    const float* lse_h = &s_lse[hg * NP + tb + 4 * lg];
    f32x4 l2[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) l2[c] = *reinterpret_cast<const f32x4*>(lse_h + 8 * c);
    const int pos0 = pos_base + tb;  // position of row tb
    const bool full = pages_full && tb + 32 <= n && kb0 + kTileKeys - 1 <= pos0 &&
                      (cls != kClassLocal || kb0 >= local_lo(pos0 + 31, bq, W));
    float p0 = 0.f, p1 = 0.f;
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p0 += __builtin_amdgcn_exp2f(fmaf(s0[i], a.scale_log2, -l2[i >> 2][i & 3]));
        p1 += __builtin_amdgcn_exp2f(fmaf(s1[i], a.scale_log2, -l2[i >> 2][i & 3]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tb + 8 * (i >> 2) + 4 * lg + (i & 3);
        const bool row_ok = t < n;
        const int pos = pos_base + t;
        const int lo = cls == kClassLocal ? local_lo(pos, bq, W) : 0;
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s0[i], a.scale_log2, -l2[i >> 2][i & 3]));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s1[i], a.scale_log2, -l2[i >> 2][i & 3]));
        p0 += (row_ok && j0 <= pos && j0 >= lo) ? e0 : 0.f;
        p1 += (row_ok && j1 <= pos && j1 >= lo) ? e1 : 0.f;
      }
    }
    acc0 += p0;
    acc1 += p1;
  };

  for (int u = u_lo; u < u_hi; ++u) unit(u);
  // lanes lg = 0 / 1 hold different rows of the same keys; then waves in order
  acc0 += __shfl_xor(acc0, 32);
  acc1 += __shfl_xor(acc1, 32);
  if (lg == 0) {
    colsum[wave][lrow] = acc0;
    colsum[wave][32 + lrow] = acc1;
  }
  __syncthreads();
  if (tid < kTileKeys && kb0 + tid < Lk) {
    const int off = reinterpret_cast<const int32_t*>(a.plan + a.L.req_key_off)[r];  // request r's first key
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kImpWaves; ++w) sum += colsum[w][tid];
    a.partial[(size_t)hh * a.total_keys + off + kb0 + tid] = sum;
  }
}

constexpr int kImpMaxHeads = 64;  // kv heads of one request (one 64-bit mask per key block)

// importance[off_r + j] = sum, in head order, of the partials of the heads whose
// tables touch key j's 64-key block (0 when none does); the plan holds one
// head mask per (request, block) and the requests' key offsets.
__global__ __launch_bounds__(256) void importance_reduce_kernel(const char* __restrict__ plan, PlanLayout L,
                                                                const float* __restrict__ partial,
                                                                float* __restrict__ importance, int64_t total_keys,
                                                                int key_blocks) {
  const int r = blockIdx.y;
  const int32_t* req_key = reinterpret_cast<const int32_t*>(plan + L.req_key_off);
  const int off = req_key[r], Lk = req_key[r + 1] - off;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= Lk) return;
  uint64_t mk = reinterpret_cast<const uint64_t*>(plan + L.imp_mask_off)[(size_t)r * key_blocks + j / kTileKeys];
  float sum = 0.f;
  while (mk != 0) {
    const int h = __builtin_ctzll(mk);
    mk &= mk - 1;
    sum += partial[(size_t)h * total_keys + off + j];
  }
  importance[off + j] = sum;
}

// ---- top-k: radix select on order-preserving integer keys ----
//
// One 1024-thread work-group selects the top k of one score vector. Wave w
// owns the contiguous key range [256 S w, 256 S (w + 1)); inside it, sub-block
// u holds keys 256 u + 4 lane + e (e < 4), kept in registers for every pass.
// Four 8-bit digit passes find the k-th largest key; each pass counts the
// candidates' digits in 64 lane-private LDS histograms (bin b of lane l at
// 64 b + l, so a wave's increments never share a bank or an address) and
// picks the digit with a suffix scan. One ordered compaction then writes
// every key above the threshold and the lowest-indexed keys equal to it.
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkSub = 256;  // keys per wave sub-block (64 lanes x 4)
constexpr int kTopkMaxRegSub = 15;  // register-resident up to 15 x 256 x 16 = 61440 keys (no spills)

// fp32 bit pattern -> unsigned integer of the same order (-0 ranks as +0)
__device__ __forceinline__ uint32_t ordered_bits(uint32_t b) {
  b = b == 0x80000000u ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Keys 4 lane + e of sub-block u; positions past n read as 0, below every real key.
__device__ __forceinline__ u32x4 topk_load4(const uint32_t* bits, int j, int n, bool vec) {
  u32x4 x;
  if (vec && j + 3 < n) {
    x = *reinterpret_cast<const u32x4*>(bits + j);
  } else {
    x[0] = j < n ? bits[j] : 0u;
    x[1] = j + 1 < n ? bits[j + 1] : 0u;
    x[2] = j + 2 < n ? bits[j + 2] : 0u;
    x[3] = j + 3 < n ? bits[j + 3] : 0u;
  }
  u32x4 o;
  o[0] = j < n ? ordered_bits(x[0]) : 0u;
  o[1] = j + 1 < n ? ordered_bits(x[1]) : 0u;
  o[2] = j + 2 < n ? ordered_bits(x[2]) : 0u;
  o[3] = j + 3 < n ? ordered_bits(x[3]) : 0u;
  return o;
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// S > 0: S sub-blocks per wave held in registers; S == 0: ns_rt sub-blocks
// re-read from memory in every pass (vectors too long for registers; the
// unroll pragmas below then do not apply).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wpass-failed"
// DPP moves inside rows of 16 lanes; a lane whose source lies outside its row reads 0
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowShl4 = 0x104, kDppRowShl8 = 0x108;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int S>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int32_t* __restrict__ idx_out, int n, int k, int ns_rt) {
  __shared__ uint32_t hist[256 * 64];  // reused to stage the output indices when k <= 16384
  __shared__ uint32_t s_wsum[kTopkWaves];
  __shared__ uint32_t s_sel[3];
  __shared__ int s_tot[kTopkWaves][2];
  constexpr int SR = S > 0 ? S : 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ns = S > 0 ? S : ns_rt;
  const int base = wave * ns * kTopkSub + 4 * lane;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores);
  const bool vec = (reinterpret_cast<uintptr_t>(bits) & 15) == 0;
  u32x4 reg[SR];
  if constexpr (S > 0) {
#pragma unroll
    for (int u = 0; u < S; ++u) reg[u] = topk_load4(bits, base + kTopkSub * u, n, vec);
  }
#define SEGKV_TOPK_KEYS(u) (S > 0 ? reg[(S > 0 ? (u) : 0)] : topk_load4(bits, base + kTopkSub * (u), n, vec))

  for (int x = tid; x < 256 * 64 / 4; x += kTopkThreads) reinterpret_cast<u32x4*>(hist)[x] = u32x4{0, 0, 0, 0};
  __syncthreads();
  uint32_t prefix = 0, eqc = 0;  // eqc: keys equal to the digits fixed so far
  int krem = k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t fixed = pass == 0 ? 0u : 0xFFFFFFFFu << (shift + 8);  // digits chosen by earlier passes
#pragma unroll
    for (int u = 0; u < (S > 0 ? S : ns); ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((x[e] & fixed) == prefix) atomicAdd(&hist[(((x[e] >> shift) & 255u) << 6) + lane], 1u);
    }
    __syncthreads();
    // bin totals: each lane of a quad sums, and clears for the next pass, 16 of
    // the bin's 64 copies; the 16-byte pieces are visited in an order rotated
    // by the bin, so the 16 lanes of a row (4 bins x 4 parts) cover all 64 banks
    const int bin = tid >> 2, part = tid & 3;
    u32x4* hp = reinterpret_cast<u32x4*>(hist + bin * 64 + 16 * part);
    const u32x4 h0 = hp[bin & 3], h1 = hp[(bin + 1) & 3], h2 = hp[(bin + 2) & 3], h3 = hp[(bin + 3) & 3];
    hp[bin & 3] = hp[(bin + 1) & 3] = hp[(bin + 2) & 3] = hp[(bin + 3) & 3] = u32x4{0, 0, 0, 0};
    uint32_t c = ((h0[0] + h0[1]) + (h0[2] + h0[3])) + ((h1[0] + h1[1]) + (h1[2] + h1[3])) +
                 ((h2[0] + h2[1]) + (h2[2] + h2[3])) + ((h3[0] + h3[1]) + (h3[2] + h3[3]));
    c += dpp_move<kDppQuadXor1>(c);
    c += dpp_move<kDppQuadXor2>(c);
    // candidates with digit >= bin: suffix over the 4 bins of a 16-lane row,
    // then the rows above in this wave, then the waves above
    uint32_t sfx = c + dpp_move<kDppRowShl4>(c);
    sfx += dpp_move<kDppRowShl8>(sfx);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 48);
    const int row = lane >> 4;
    sfx += (row < 1 ? r1 : 0u) + (row < 2 ? r2 : 0u) + (row < 3 ? r3 : 0u);
    if (lane == 0) s_wsum[wave] = sfx;  // lane 0 holds the wave's total
    __syncthreads();
    uint32_t above = 0;
#pragma unroll
    for (int v4 = 0; v4 < kTopkWaves / 4; ++v4) {
      const u32x4 w4 = reinterpret_cast<const u32x4*>(s_wsum)[v4];
#pragma unroll
      for (int e = 0; e < 4; ++e) above += 4 * v4 + e > wave ? w4[e] : 0u;
    }
    const uint32_t ge = sfx + above, gt = ge - c;
    if (part == 0 && gt < (uint32_t)krem && (uint32_t)krem <= ge) {
      s_sel[0] = prefix | ((uint32_t)bin << shift);
      s_sel[1] = (uint32_t)krem - gt;
      s_sel[2] = c;
    }
    __syncthreads();
    prefix = s_sel[0];
    krem = (int)s_sel[1];
    eqc = s_sel[2];
  }

  // prefix is the k-th largest key. Output order = index order: waves, then
  // sub-blocks, then lanes, then e. Outputs of up to 16384 indices are staged
  // in LDS (the histogram space) and copied out coalesced.
  const bool stage = k <= 256 * 64;
  uint32_t* s_out = hist;
  if (eqc == (uint32_t)krem) {
    // every key >= prefix is taken
    int g = 0;
#pragma unroll
    for (int u = 0; u < (S > 0 ? S : ns); ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
#pragma unroll
      for (int e = 0; e < 4; ++e) g += __popcll(__ballot(x[e] >= prefix));
    }
    if (lane == 0) s_tot[wave][0] = g;
    __syncthreads();
    int gb = 0;
    for (int v = 0; v < wave; ++v) gb += s_tot[v][0];
#pragma unroll
    for (int u = 0; u < (S > 0 ? S : ns); ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
      uint64_t m[4];
      int pos = gb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = __ballot(x[e] >= prefix);
        pos += lanes_below(m[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (x[e] >= prefix) {
          const int j = base + kTopkSub * u + e;
          if (stage) s_out[pos] = (uint32_t)j;
          else idx_out[pos] = j;
          ++pos;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) gb += __popcll(m[e]);
    }
  } else {
    // keys > prefix, then the first krem keys == prefix
    int g = 0, q = 0;
#pragma unroll
    for (int u = 0; u < (S > 0 ? S : ns); ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g += __popcll(__ballot(x[e] > prefix));
        q += __popcll(__ballot(x[e] == prefix));
      }
    }
    if (lane == 0) {
      s_tot[wave][0] = g;
      s_tot[wave][1] = q;
    }
    __syncthreads();
    int gb = 0, qb = 0;
    for (int v = 0; v < wave; ++v) {
      gb += s_tot[v][0];
      qb += s_tot[v][1];
    }
#pragma unroll
    for (int u = 0; u < (S > 0 ? S : ns); ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
      uint64_t mg[4], mq[4];
      int go = gb, qo = qb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mg[e] = __ballot(x[e] > prefix);
        mq[e] = __ballot(x[e] == prefix);
        go += lanes_below(mg[e]);
        qo += lanes_below(mq[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool isg = x[e] > prefix, isq = x[e] == prefix;
        if (isg || (isq && qo < krem)) {
          const int pos = go + imin(qo, krem), j = base + kTopkSub * u + e;
          if (stage) s_out[pos] = (uint32_t)j;
          else idx_out[pos] = j;
        }
        go += isg ? 1 : 0;
        qo += isq ? 1 : 0;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gb += __popcll(mg[e]);
        qb += __popcll(mq[e]);
      }
    }
  }
  if (stage) {
    __syncthreads();
    for (int x = tid; x < k; x += kTopkThreads) idx_out[x] = (int32_t)s_out[x];
  }
#undef SEGKV_TOPK_KEYS
}
#pragma clang diagnostic pop

int32_t launch_topk(const float* scores, int32_t* idx, int n, int k, hipStream_t s) {
  if (k <= 0) return SEGKV_OK;
  if (n > (1 << 30)) return fail(SEGKV_ERR_UNSUPPORTED, "top-k vectors are limited to 2^30 keys");
  const int ns = cdiv(n, kTopkWaves * kTopkSub);  // sub-blocks per wave
  const dim3 g(1), b(kTopkThreads);
#define SEGKV_TOPK(SV) topk_kernel<SV><<<g, b, 0, s>>>(scores, idx, n, k, ns)
  switch (ns <= kTopkMaxRegSub ? ns : 0) {
    case 1: SEGKV_TOPK(1); break;
    case 2: SEGKV_TOPK(2); break;
    case 3: SEGKV_TOPK(3); break;
    case 4: SEGKV_TOPK(4); break;
    case 5: SEGKV_TOPK(5); break;
    case 6: SEGKV_TOPK(6); break;
    case 7: SEGKV_TOPK(7); break;
    case 8: SEGKV_TOPK(8); break;
    case 9: SEGKV_TOPK(9); break;
    case 10: SEGKV_TOPK(10); break;
    case 11: SEGKV_TOPK(11); break;
    case 12: SEGKV_TOPK(12); break;
    case 13: SEGKV_TOPK(13); break;
    case 14: SEGKV_TOPK(14); break;
    case 15: SEGKV_TOPK(15); break;
    default: SEGKV_TOPK(0); break;
  }
#undef SEGKV_TOPK
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
                                         const void* plan_dev, size_t plan_bytes,
                                         const float* lse_dev, float softmax_scale, int32_t n_last,
                                         const int32_t* k_host, float* importance_dev, int32_t* topk_idx_dev,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  HostPlan hp;
  int32_t st = compute_host_plan(dims, meta_host, &hp);
  if (st != SEGKV_OK) return st;
  if (!meta_dev || !meta_dev->seg_indptr || !cu_q_dev || !q || !k_pool || !page_indptr_dev || !page_ids_dev ||
      !page_pos_dev || !plan_dev || !lse_dev || !importance_dev)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (plan_bytes < hp.plan_bytes) return fail(SEGKV_ERR_WORKSPACE, "plan smaller than plan_bytes from segkv_plan_sizes");
  if (dims->num_kv_heads > kImpMaxHeads) return fail(SEGKV_ERR_UNSUPPORTED, "importance supports num_kv_heads <= 64");
  if (n_last <= 0) return fail(SEGKV_ERR_INVALID_ARG, "n_last must be > 0");
  const int G = dims->num_q_heads / dims->num_kv_heads;
  if (workspace == nullptr || workspace_bytes < importance_workspace_bytes(*dims, hp.total_keys))
    return fail(SEGKV_ERR_WORKSPACE, "workspace smaller than importance_workspace_bytes from segkv_plan_sizes");
  if (!aligned16(workspace)) return fail(SEGKV_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if ((int64_t)dims->num_q_heads * 32 * cdiv(n_last, 32) > kImpMaxLse)
    return fail(SEGKV_ERR_UNSUPPORTED, "num_q_heads * (n_last rounded up to 32) must be <= 4096");
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
  a.partial = static_cast<float*>(workspace);
  a.plan = static_cast<const char*>(plan_dev);
  a.L = host_plan_layout(*dims, hp);
  a.total_keys = hp.total_keys;
  a.scale_log2 = softmax_scale * kLog2e;
  a.R = R;
  a.Hq = dims->num_q_heads;
  a.Hkv = dims->num_kv_heads;
  a.G = G;
  a.n_last = n_last;
  if (R > 65535) return fail(SEGKV_ERR_UNSUPPORTED, "importance supports at most 65535 requests");
  if (hp.n_imp_items > 0) {
    if (dims->head_dim == 128)
      importance_kernel<128><<<hp.n_imp_items, kImpThreads, 0, s>>>(a);
    else
      importance_kernel<64><<<hp.n_imp_items, kImpThreads, 0, s>>>(a);
    SEGKV_LAUNCH_CHECK();
  }
  importance_reduce_kernel<<<dim3(cdiv(max_lk, 256), R), 256, 0, s>>>(a.plan, a.L, a.partial, importance_dev,
                                                                      hp.total_keys, hp.key_blocks);
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
