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
#include <type_traits>

#include "common.h"

namespace segkv {
namespace {

SEGKV_DEVICE_FLAG(g_imp_check);  // bit 1: a table page id outside the pool

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
// in a fixed order with no float atomics. The K tile is staged in LDS. A
// unit's Q block is fetched whole rows per load instruction (a quarter of the
// cache-line requests that MFMA-order loads would make) and passes through the
// wave's own LDS slot; the next unit's Q is in flight while the current one
// computes. Units whose 32 rows see all 64 keys skip every mask.
template <int D>
__global__ __launch_bounds__(kImpThreads, 3) void importance_kernel(ImpArgs a) {
  constexpr int KS = D / 16;
  constexpr int KCH = D / 8;            // 16-byte chunks per key row
  constexpr int kStride = D + 8;        // padded LDS row (elements)
  constexpr int KLOADS = kTileKeys * KCH / kImpThreads;
  constexpr int CH = D / 8;              // 16-byte chunks per Q row
  __shared__ __attribute__((aligned(16))) uint16_t ks[kTileKeys * kStride];
  __shared__ __attribute__((aligned(16))) uint16_t qs[kImpWaves][32 * D];  // each wave's unit Q, chunks swizzled
  extern __shared__ __attribute__((aligned(16))) float s_lse[];  // G * NP values (size set at launch)
  __shared__ int s_pid[kTilePages];  // this head's page at each page of the key block, -1 if none
  __shared__ float colsum[kImpWaves][kTileKeys];

  const ImpItem* itp = reinterpret_cast<const ImpItem*>(a.plan + a.L.imp_items_off) + blockIdx.x;
  const ImpItem item = *itp;  // indexed below only through itp, so the copy stays in registers
  if (item.pair < 0 || item.pair >= a.R * a.Hkv || item.block < 0) return;  // not a plan of this layout
  const int r = item.pair / a.Hkv, hh = item.pair % a.Hkv;
  const int bq = item.bq, Lq = item.Lq, Lk = bq + Lq;
  const int kb0 = item.block * kTileKeys;
  if (kb0 >= Lk) return;
  const int n = imin(a.n_last, Lq);
  const int nb_head = cdiv(n, 32);  // 32-row blocks per query head
  const int NP = 32 * nb_head;      // staged rows per query head (the last row repeated)
  const int U = a.G * nb_head;      // units of this kv head
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int q_base = item.cu_q + Lq - n;  // first of the last n query rows
  const int pos_base = Lk - n;            // its position
  const int u_lo = U * wave / kImpWaves, u_hi = U * (wave + 1) / kImpWaves;

  // Every load of the prologue is issued before any is waited for: the
  // block's page ids (scalar loads), the LSE of its rows, the K tile, and the
  // wave's first Q fragment (A operand: Q row tb + lrow of query head hg).
  // Addresses are clamped into range and unused values dropped afterwards,
  // so no load sits behind a branch.
  int ent[kTilePages], pid[kTilePages];
#pragma unroll
  for (int u = 0; u < kTilePages; ++u) ent[u] = itp->entry[u];
#pragma unroll
  for (int u = 0; u < kTilePages; ++u) pid[u] = a.page_ids[imax(ent[u], 0)];
  const int pool_pages = a.pool_pages < INT32_MAX ? (int)a.pool_pages : INT32_MAX;
#pragma unroll
  for (int u = 0; u < kTilePages; ++u) {
    SEGKV_DCHECK(g_imp_check, ent[u] < 0 || (pid[u] >= 0 && pid[u] < pool_pages), 1);
    pid[u] = ent[u] < 0 || pid[u] < 0 || pid[u] >= pool_pages ? -1 : pid[u];
  }
  // log2-scaled LSE of the last n rows of this head's G query heads, [g][t]
  // with t < NP (rows past n repeat row n - 1)
  const int n_lse = a.G * NP;
  auto lse_at = [&](int x) { return a.lse[(size_t)(q_base + imin(x % NP, n - 1)) * a.Hq + hh * a.G + x / NP]; };
  float lv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) lv[u] = lse_at(imin(tid + u * kImpThreads, n_lse - 1));
  // K tile rows: qd = tid + u * kImpThreads is 16-byte chunk qd % KCH of key
  // qd / KCH; rows of missing pages are zero
  u32x4 kr[KLOADS];
#pragma unroll
  for (int u = 0; u < KLOADS; ++u) {
    const int qd = tid + u * kImpThreads, key = qd / KCH, c = qd % KCH;
    const int pg = pid[key >> 4];
    kr[u] = *reinterpret_cast<const u32x4*>(a.k_pool + ((size_t)imax(pg, 0) * kPage + (key & 15)) * D + 8 * c);
    if (pg < 0) kr[u] = u32x4{0, 0, 0, 0};
  }
  // A unit's 32 x D block of Q is fetched with 16-byte chunk lane + 64 i per
  // lane (whole rows per instruction), passes through the wave's LDS slot with
  // chunk c of row r at c ^ (r mod CH), and is read back in MFMA A-operand
  // order (row lrow, dims 16 k8 + 8 lg .. + 8).
  u32x4 qr[KS];
  auto q_fetch = [&](int uu) __attribute__((always_inline)) {
    const int hg = uu / nb_head, tb = (uu % nb_head) * 32;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int qc = lane + 64 * i, row = qc / CH, c = qc % CH;
      qr[i] = *reinterpret_cast<const u32x4*>(
          a.q + ((size_t)(q_base + imin(tb + row, n - 1)) * a.Hq + hh * a.G + hg) * D + 8 * c);
    }
  };
  uint16_t* const qw = qs[wave];
  auto q_commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int qc = lane + 64 * i, row = qc / CH, c = qc % CH;
      *reinterpret_cast<u32x4*>(qw + row * D + 8 * (c ^ (row & (CH - 1)))) = qr[i];
    }
  };
  if (u_lo < u_hi) q_fetch(u_lo);

  if (tid == 0) {
#pragma unroll
    for (int u = 0; u < kTilePages; ++u) s_pid[u] = pid[u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int x = tid + u * kImpThreads;
    if (x < n_lse) s_lse[x] = lv[u] * kLog2e;
  }
  for (int x = tid + 4 * kImpThreads; x < n_lse; x += kImpThreads) s_lse[x] = lse_at(x) * kLog2e;
#pragma unroll
  for (int u = 0; u < KLOADS; ++u) {
    const int qd = tid + u * kImpThreads;
    *reinterpret_cast<u32x4*>(&ks[(qd / KCH) * kStride + 8 * (qd % KCH)]) = kr[u];
  }
  __syncthreads();

  const int cls = item.cls, W = item.W;
  const bool pages_full = s_pid[0] >= 0 && s_pid[1] >= 0 && s_pid[2] >= 0 && s_pid[3] >= 0;
  const int pa = s_pid[lrow >> 4], pb = s_pid[2 + (lrow >> 4)];
  const int j0 = pa < 0 ? INT_MAX : kb0 + lrow;
  const int j1 = pb < 0 ? INT_MAX : kb0 + 32 + lrow;

  float acc0 = 0.f, acc1 = 0.f;  // keys lrow and 32 + lrow, this lane's rows
  // unit uu: its Q goes from the fetch registers to the wave's LDS slot; once
  // the MFMAs have read it, the next unit's fetch is issued, so that load
  // overlaps this unit's exponentials
  auto unit = [&](int uu) {
    q_commit();
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
#pragma unroll
    for (int k8 = 0; k8 < KS; ++k8) {  // B operand: key 32 kb + lrow, dims 16 k8 + 8 lg .. + 8
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qw + lrow * D + 8 * ((2 * k8 + lg) ^ (lrow & (CH - 1))));
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(&ks[lrow * kStride + 16 * k8 + 8 * lg]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(&ks[(32 + lrow) * kStride + 16 * k8 + 8 * lg]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qv, k0, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qv, k1, s1, 0, 0, 0);
    }
    // operand reads two k-steps ahead of their MFMAs (bounds the live fragments)
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int k8 = 0; k8 < KS - 2; ++k8) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (uu + 1 < u_hi) q_fetch(uu + 1);
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
    const int off = item.key_off;  // request r's first key
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
  const uint64_t mk = reinterpret_cast<const uint64_t*>(plan + L.imp_mask_off)[(size_t)r * key_blocks + j / kTileKeys];
  const float* pj = partial + off + j;
  // heads in groups of 8: the group's loads are all issued before the adds
  float sum = 0.f;
  for (int h0 = 0; h0 < 64 && (mk >> h0) != 0; h0 += 8) {
    const uint32_t g = (uint32_t)(mk >> h0) & 255u;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = (g >> i) & 1u ? pj[(size_t)(h0 + i) * total_keys] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((g >> i) & 1u) sum += p[i];
  }
  importance[off + j] = sum;
}

// ---- top-k: radix select on order-preserving integer keys ----
//
// One 1024-thread work-group selects the top k of one score vector (one
// work-group per request, all in one launch). Wave w owns the contiguous key
// range [256 S w, 256 S (w + 1)); inside it, sub-block u holds keys
// 256 u + 4 lane + e (e < 4), kept in registers for every pass.
// Up to four 8-bit digit passes find the k-th largest key. Each pass counts
// the candidates' digits in 64 lane-private LDS histograms (bin b of lane l at
// 64 b + l, so a wave's increments never share a bank or an address). Every
// wave then sums the copies of 16 bins, and after one barrier every wave
// scans the 256 bin totals itself, so the chosen digit needs no broadcast.
// Two histogram buffers alternate: the one just summed is cleared while the
// next pass counts into the other. The passes stop as soon as every key
// sharing the chosen digits is needed; the threshold is then those digits
// with zero low bits. One ordered compaction writes every key above the
// threshold and the lowest-indexed keys equal to it.
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkSub = 256;  // keys per wave sub-block (64 lanes x 4)
constexpr int kTopkMaxRegSub = 15;  // register-resident up to 15 x 256 x 16 = 61440 keys (no spills)
constexpr int kTopkSplitLoad = 12;  // sub-blocks up to which all key loads precede their ordering
constexpr int kTopkHist = 256 * 64;  // words of one histogram buffer
constexpr int kTopkSegSub = 9;       // up to 9 sub-blocks per wave, every wave's selection fits its own LDS segment
constexpr int kTopkLdsWords = kTopkWaves * kTopkSub * kTopkSegSub + 64;  // >= both histogram buffers
constexpr int kTopkStageMax = kTopkLdsWords - 64;  // staged output indices; the last 64 words take unselected writes
static_assert(kTopkStageMax >= 2 * kTopkHist, "the LDS array must hold both histogram buffers");
constexpr int kTopkMaxJobs = 64;  // score vectors per launch

// The score vectors of one launch: vector j has n[j] keys at scores + off[j]
// and writes its k[j] indices at idx + koff[j].
struct TopkJobs {
  int64_t off[kTopkMaxJobs], koff[kTopkMaxJobs];
  int n[kTopkMaxJobs], k[kTopkMaxJobs];
};

// fp32 bit pattern -> unsigned integer of the same order (-0 ranks as +0)
__device__ __forceinline__ uint32_t ordered_bits(uint32_t b) {
  b = b == 0x80000000u ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Keys j .. j + 3 (4 lane + e of a sub-block): the raw fp32 bits, then their
// ordered form; positions past n read as 0, below every real key.
__device__ __forceinline__ u32x4 topk_load_raw4(const uint32_t* bits, int j, int n, bool vec) {
  u32x4 x;
  if (vec && j + 3 < n) {
    x = *reinterpret_cast<const u32x4*>(bits + j);
  } else {
    x[0] = j < n ? bits[j] : 0u;
    x[1] = j + 1 < n ? bits[j + 1] : 0u;
    x[2] = j + 2 < n ? bits[j + 2] : 0u;
    x[3] = j + 3 < n ? bits[j + 3] : 0u;
  }
  return x;
}
__device__ __forceinline__ u32x4 topk_order4(const u32x4& x, int j, int n) {
  u32x4 o;
  o[0] = j < n ? ordered_bits(x[0]) : 0u;
  o[1] = j + 1 < n ? ordered_bits(x[1]) : 0u;
  o[2] = j + 2 < n ? ordered_bits(x[2]) : 0u;
  o[3] = j + 3 < n ? ordered_bits(x[3]) : 0u;
  return o;
}
__device__ __forceinline__ u32x4 topk_load4(const uint32_t* bits, int j, int n, bool vec) {
  return topk_order4(topk_load_raw4(bits, j, n, vec), j, n);
}

// Lanes below this one whose bit is set in m, plus acc.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m, uint32_t acc) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, acc));
}

// S > 0: S sub-blocks per wave held in registers; S == 0: ns_rt sub-blocks
// re-read from memory in every pass (vectors too long for registers; the
// unroll pragmas below then do not apply).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wpass-failed"
// DPP moves inside rows of 16 lanes; a lane whose source lies outside its row reads 0
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E;
constexpr int kDppRowShl1 = 0x101, kDppRowShl2 = 0x102, kDppRowShl4 = 0x104, kDppRowShl8 = 0x108;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int S>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores_all,
                                                            int32_t* __restrict__ idx_all, const TopkJobs jobs,
                                                            int ns_rt) {
  __shared__ uint32_t hist[kTopkLdsWords];  // two histogram buffers; afterwards the staged output
  __shared__ u32x4 s_bins[64];              // bin totals of the current pass
  __shared__ int s_tot[kTopkWaves][2];
  constexpr int SR = S > 0 ? S : 1;
  const int n = jobs.n[blockIdx.x], k = jobs.k[blockIdx.x];
  if (k <= 0) return;
  const float* scores = scores_all + jobs.off[blockIdx.x];
  int32_t* idx_out = idx_all + jobs.koff[blockIdx.x];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ns = S > 0 ? S : ns_rt;
  const int base = wave * ns * kTopkSub + 4 * lane;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores);
  const bool vec = (reinterpret_cast<uintptr_t>(bits) & 15) == 0;
  // Up to kTopkSplitLoad sub-blocks, the key loads are issued first, one
  // 16-byte load per lane and sub-block wherever the 4 keys lie inside the
  // vector (no branch between them, so no load waits for another); both
  // histogram buffers are cleared while they are in flight. Then a partial
  // last quad (or a vector that is not 16-byte aligned) is read key by key,
  // and the keys take their ordered form. With more sub-blocks the fix-up's
  // registers would spill, so each quad is loaded and ordered at once.
  constexpr bool kSplit = S > 0 && S <= kTopkSplitLoad;
  u32x4 reg[SR];
  if constexpr (kSplit) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int j = base + kTopkSub * u;
      reg[u] = u32x4{0, 0, 0, 0};
      if (vec && j + 3 < n) reg[u] = *reinterpret_cast<const u32x4*>(bits + j);
    }
  } else if constexpr (S > 0) {
#pragma unroll
    for (int u = 0; u < S; ++u) reg[u] = topk_load4(bits, base + kTopkSub * u, n, vec);
  }
#define SEGKV_TOPK_KEYS(u) (S > 0 ? reg[(S > 0 ? (u) : 0)] : topk_load4(bits, base + kTopkSub * (u), n, vec))

  // Byte address of a key's counter in buffer bf: byte 0 = 4 lane, byte 1 =
  // the digit (byte 3 - pass of the key), byte 2 = the buffer; one v_perm.
  const uint32_t lane4 = 4u * (uint32_t)lane;
  char* const hbytes = reinterpret_cast<char*>(hist);
#pragma unroll
  for (int x = tid; x < 2 * kTopkHist / 4; x += kTopkThreads) reinterpret_cast<u32x4*>(hist)[x] = u32x4{0, 0, 0, 0};
  if constexpr (kSplit) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int j = base + kTopkSub * u;
      if (!(vec && j + 3 < n) && j < n) reg[u] = topk_load_raw4(bits, j, n, false);
      reg[u] = topk_order4(reg[u], j, n);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (S > 0 ? S : ns); ++u) {
    const u32x4 x = SEGKV_TOPK_KEYS(u);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      atomicAdd(reinterpret_cast<uint32_t*>(hbytes + __builtin_amdgcn_perm(x[e], lane4, 0x0C0C0700u)), 1u);
  }

  uint32_t prefix = 0, eqc = 0;  // eqc: keys equal to the digits fixed so far
  int krem = k;
  // bin totals: lane q of a quad sums copies 16 q .. 16 q + 15 of bin
  // 16 wave + lane / 4; the 16-byte pieces are visited in an order rotated by
  // the bin, so the 16 lanes of a row (4 bins x 4 parts) cover all 64 banks
  const int my_bin = 16 * wave + (lane >> 2), part = lane & 3;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* hb = hist + (pass & 1) * kTopkHist;
    __syncthreads();
    {
      const u32x4* hp = reinterpret_cast<const u32x4*>(hb + my_bin * 64 + 16 * part);
      const u32x4 h0 = hp[my_bin & 3], h1 = hp[(my_bin + 1) & 3], h2 = hp[(my_bin + 2) & 3], h3 = hp[(my_bin + 3) & 3];
      uint32_t c = ((h0[0] + h0[1]) + (h0[2] + h0[3])) + ((h1[0] + h1[1]) + (h1[2] + h1[3])) +
                   ((h2[0] + h2[1]) + (h2[2] + h2[3])) + ((h3[0] + h3[1]) + (h3[2] + h3[3]));
      c += dpp_move<kDppQuadXor1>(c);
      c += dpp_move<kDppQuadXor2>(c);
      if (part == 0) reinterpret_cast<uint32_t*>(s_bins)[my_bin] = c;
    }
    __syncthreads();
    {
      // every wave: lane L holds bins 4 L + i; candidates with digit >= 4 L
      // by a suffix over the lanes of a 16-lane row, then the rows above
      const u32x4 t = s_bins[lane];
      const uint32_t tl = (t[0] + t[1]) + (t[2] + t[3]);
      uint32_t sfx = tl + dpp_move<kDppRowShl1>(tl);
      sfx += dpp_move<kDppRowShl2>(sfx);
      sfx += dpp_move<kDppRowShl4>(sfx);
      sfx += dpp_move<kDppRowShl8>(sfx);
      const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 16);
      const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 32);
      const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 48);
      const int row = lane >> 4;
      sfx += (row < 1 ? r1 : 0u) + (row < 2 ? r2 : 0u) + (row < 3 ? r3 : 0u);
      // the one (lane, i) with gt < krem <= gt + t[i] holds the k-th largest candidate
      uint32_t gt = sfx - tl, hit_bin = 0, hit_rem = 0, hit_c = 0;
      bool hit = false;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const bool h = gt < (uint32_t)krem && (uint32_t)krem <= gt + t[i];
        hit_bin = h ? (uint32_t)(4 * lane + i) : hit_bin;
        hit_rem = h ? (uint32_t)krem - gt : hit_rem;
        hit_c = h ? t[i] : hit_c;
        hit = hit || h;
        gt += t[i];
      }
      const int src = (int)__builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(hit) | (1ull << 63)));
      prefix |= (uint32_t)__builtin_amdgcn_readlane((int)hit_bin, src) << shift;
      krem = __builtin_amdgcn_readlane((int)hit_rem, src);
      eqc = (uint32_t)__builtin_amdgcn_readlane((int)hit_c, src);
    }
    if (eqc == (uint32_t)krem || pass == 3) break;  // every key with these digits is taken, or all digits fixed
    if (pass < 2) {  // clear this buffer for pass + 2; every wave has summed its bins
      uint32_t* hz = hb + my_bin * 64 + 16 * part;
#pragma unroll
      for (int c = 0; c < 4; ++c) reinterpret_cast<u32x4*>(hz)[c] = u32x4{0, 0, 0, 0};
    }
    // count the next digit of the keys that match the digits fixed so far
    const uint32_t span = 0xFFFFFFFFu >> (8 * (pass + 1));  // x matches iff x - prefix <= span
    const uint32_t psel = 0x0C000000u | (((pass + 1) & 1) ? 0x00020000u : 0x000C0000u) | ((uint32_t)(6 - pass) << 8);
    const uint32_t lanebuf = lane4 | 0x00010000u;  // byte 2 = 1 selects the second buffer
#pragma unroll
    for (int u = 0; u < (S > 0 ? S : ns); ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (x[e] - prefix <= span)
          atomicAdd(reinterpret_cast<uint32_t*>(hbytes + __builtin_amdgcn_perm(x[e], lanebuf, psel)), 1u);
    }
  }
  // prefix is the k-th largest key, or, after an early stop, its leading
  // digits with zero low bits. Output order = index order: waves, then
  // sub-blocks, then lanes, then e. Outputs of up to kTopkStageMax indices
  // are staged in LDS (the histogram space) and copied out coalesced; lanes
  // that select nothing write to a slot of their own past the staged range.
  const bool all_eq = eqc == (uint32_t)krem;  // every key >= prefix is taken
  auto compact = [&](auto staged) __attribute__((always_inline)) {
    constexpr bool kStage = decltype(staged)::value;
    const uint32_t dummy = (uint32_t)(kTopkStageMax + lane);
    auto emit = [&](bool sel, uint32_t pos, int j) __attribute__((always_inline)) {
      if constexpr (kStage) {
        hist[sel ? pos : dummy] = (uint32_t)j;
      } else {
        if (sel) idx_out[pos] = j;
      }
    };
    if (all_eq) {
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
#pragma unroll
      for (int v = 0; v < kTopkWaves; ++v) gb += v < wave ? s_tot[v][0] : 0;
#pragma unroll
      for (int u = 0; u < (S > 0 ? S : ns); ++u) {
        const u32x4 x = SEGKV_TOPK_KEYS(u);
        uint64_t m[4];
        uint32_t pos = (uint32_t)gb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          m[e] = __ballot(x[e] >= prefix);
          pos = lanes_below(m[e], pos);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool sel = x[e] >= prefix;
          emit(sel, pos, base + kTopkSub * u + e);
          pos += sel ? 1u : 0u;
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
#pragma unroll
      for (int v = 0; v < kTopkWaves; ++v) {
        gb += v < wave ? s_tot[v][0] : 0;
        qb += v < wave ? s_tot[v][1] : 0;
      }
#pragma unroll
      for (int u = 0; u < (S > 0 ? S : ns); ++u) {
        const u32x4 x = SEGKV_TOPK_KEYS(u);
        uint64_t mg[4], mq[4];
        uint32_t go = (uint32_t)gb, qo = (uint32_t)qb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mg[e] = __ballot(x[e] > prefix);
          mq[e] = __ballot(x[e] == prefix);
          go = lanes_below(mg[e], go);
          qo = lanes_below(mq[e], qo);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool isg = x[e] > prefix, isq = x[e] == prefix;
          emit(isg || (isq && qo < (uint32_t)krem), go + (qo < (uint32_t)krem ? qo : (uint32_t)krem), base + kTopkSub * u + e);
          go += isg ? 1u : 0u;
          qo += isq ? 1u : 0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gb += __popcll(mg[e]);
          qb += __popcll(mq[e]);
        }
      }
    }
    if constexpr (kStage) {
      __syncthreads();
      if ((reinterpret_cast<uintptr_t>(idx_out) & 15) == 0) {
        const int k4 = k >> 2;
        for (int x = tid; x < k4; x += kTopkThreads)
          reinterpret_cast<u32x4*>(idx_out)[x] = reinterpret_cast<const u32x4*>(hist)[x];
        for (int x = 4 * k4 + tid; x < k; x += kTopkThreads) idx_out[x] = (int32_t)hist[x];
      } else {
        for (int x = tid; x < k; x += kTopkThreads) idx_out[x] = (int32_t)hist[x];
      }
    }
  };
  if (S > 0 && S <= kTopkSegSub && all_eq) {
    // one sweep: wave w stages its selected indices, in order, in its own
    // segment of 256 S words, then copies them to its place in the output
    uint32_t* seg = hist + wave * (kTopkSub * SR);
    uint32_t pos = 0;
#pragma unroll
    for (int u = 0; u < SR; ++u) {
      const u32x4 x = SEGKV_TOPK_KEYS(u);
      uint64_t m[4];
      uint32_t p = pos;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = __ballot(x[e] >= prefix);
        p = lanes_below(m[e], p);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool sel = x[e] >= prefix;
        if (sel) seg[p] = (uint32_t)(base + kTopkSub * u + e);
        p += sel ? 1u : 0u;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pos += (uint32_t)__popcll(m[e]);
    }
    if (lane == 0) s_tot[wave][0] = (int)pos;
    __syncthreads();
    int off = 0;
#pragma unroll
    for (int v = 0; v < kTopkWaves; ++v) off += v < wave ? s_tot[v][0] : 0;
    int32_t* dst = idx_out + off;
#pragma unroll 4
    for (int x = lane; x < (int)pos; x += 64) dst[x] = (int32_t)seg[x];
  } else if (k <= kTopkStageMax) {
    compact(std::true_type{});
  } else {
    compact(std::false_type{});
  }
#undef SEGKV_TOPK_KEYS
}
#pragma clang diagnostic pop

// One launch selects up to kTopkMaxJobs vectors, one work-group each; the
// register-resident sub-block count follows the longest vector.
int32_t launch_topk_jobs(const float* scores, int32_t* idx, const TopkJobs& jobs, int n_jobs, hipStream_t s) {
  int max_n = 0;
  for (int j = 0; j < n_jobs; ++j) {
    if (jobs.n[j] > (1 << 30)) return fail(SEGKV_ERR_UNSUPPORTED, "top-k vectors are limited to 2^30 keys");
    max_n = imax(max_n, jobs.n[j]);
  }
  const int ns = imax(1, cdiv(max_n, kTopkWaves * kTopkSub));  // sub-blocks per wave
  const dim3 g(n_jobs), b(kTopkThreads);
#define SEGKV_TOPK(SV) topk_kernel<SV><<<g, b, 0, s>>>(scores, idx, jobs, ns)
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
    const size_t lse_bytes = sizeof(float) * (size_t)G * 32 * (size_t)cdiv(n_last, 32);  // G * NP of any request
    if (dims->head_dim == 128)
      importance_kernel<128><<<hp.n_imp_items, kImpThreads, lse_bytes, s>>>(a);
    else
      importance_kernel<64><<<hp.n_imp_items, kImpThreads, lse_bytes, s>>>(a);
    SEGKV_LAUNCH_CHECK();
  }
  importance_reduce_kernel<<<dim3(cdiv(max_lk, 256), R), 256, 0, s>>>(a.plan, a.L, a.partial, importance_dev,
                                                                      hp.total_keys, hp.key_blocks);
  SEGKV_LAUNCH_CHECK();
  SEGKV_DEVICE_CHECK(g_imp_check, s, "token_importance_topk: a page-table entry is out of range");
  if (topk_idx_dev == nullptr) return SEGKV_OK;
  // the requests' selections, kTopkMaxJobs per launch (host knows every offset)
  TopkJobs jobs;
  int nj = 0;
  int64_t off = 0, koff = 0;
  for (int r = 0; r < R; ++r) {
    const int sq = meta_host->seg_indptr[r + 1] - 1;
    const int lk = meta_host->seg_start[sq] + meta_host->seg_len[sq];
    jobs.off[nj] = off;
    jobs.koff[nj] = koff;
    jobs.n[nj] = lk;
    jobs.k[nj] = k_host[r];
    ++nj;
    off += lk;
    koff += k_host[r];
    if (nj == kTopkMaxJobs || r == R - 1) {
      st = launch_topk_jobs(importance_dev, topk_idx_dev, jobs, nj, s);
      if (st != SEGKV_OK) return st;
      nj = 0;
    }
  }
  return SEGKV_OK;
}

extern "C" int32_t segkv_topk_select(const float* scores_dev, int32_t n, int32_t k, int32_t* idx_dev,
                                     void* stream) {
  clear_error();
  if (n < 0 || k < 0 || k > n) return fail(SEGKV_ERR_INVALID_ARG, "need 0 <= k <= n");
  if (k == 0) return SEGKV_OK;
  if (!scores_dev || !idx_dev) return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  TopkJobs jobs;
  jobs.off[0] = 0;
  jobs.koff[0] = 0;
  jobs.n[0] = n;
  jobs.k[0] = k;
  return launch_topk_jobs(scores_dev, idx_dev, jobs, 1, static_cast<hipStream_t>(stream));
}
