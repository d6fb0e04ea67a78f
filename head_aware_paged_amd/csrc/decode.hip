// Decode-phase attention: one new query row per request, over the per-head
// page tables that segkv_build_pages wrote for the prefill of the same layout.
//
// The pages (arXiv abstract; paooo.com "如何使用RedKnot": EXECUTE over the
// visible state chosen per head; README "About": per-head page tables and
// per-class visible windows) describe the prefill. The decode step applies the
// same class rule to the new token at position i = L_k(r): GLOBAL and DENSE
// heads see every key, LOCAL heads their query segment and the W-token window
// ending at i, RETRIEVAL heads their query segment and the two reused
// segments; every set holds the new token itself (k_new, v_new). Each of those
// sets lies inside the table of the prefill's last row, so the tables serve
// unchanged.
//
// Split over pages: one work-group per (request, kv head, run of 8 table
// entries) computes, for the kv head's G query heads, the run's max, sum and
// unnormalised output; a second kernel merges the runs and the new token.
#include "common.h"

namespace segkv {
namespace {

SEGKV_DEVICE_FLAG(g_dec_check);  // bit 1: a table page id outside the pool

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecPagesPerWave = 1;
constexpr int kDecChunk = kDecWaves * kDecPagesPerWave;  // table entries per work-group
constexpr int kDecMaxG = 16;                             // query heads per kv head (MFMA columns)
constexpr float kDecLog2e = 1.4426950408889634f;
constexpr float kDecLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

struct DecArgs {
  segkv_meta m;
  const uint16_t* q_new;   // [R][Hq][D]
  const uint16_t* k_new;   // [R][Hkv][D]
  const uint16_t* v_new;   // [R][Hkv][D]
  const uint16_t* k_pool;  // [pages][P][D]
  const uint16_t* v_pool;  // [pages][D][P]
  int64_t pool_pages;
  const int32_t* page_indptr;
  const int32_t* page_ids;
  const int32_t* page_pos;
  float* ws;  // [R*Hkv][max_chunks][G][D + 2]: unnormalised O, then m (log2 units), l
  uint16_t* out;
  float* lse;
  float scale_log2;
  int R, Hq, Hkv, G, max_chunks;
};

// The new token at position i = L_k sees key j < L_k of (r, h) when:
__device__ __forceinline__ bool dec_visible(const HeadView& v, int j) {
  if (j < 0 || j >= v.Lk) return false;
  if (v.cls == kClassLocal) return j >= local_lo(v.Lk, v.bq, v.W);
  if (v.cls == kClassRetrieval) return j >= v.bq || (j >= v.rlo[0] && j < v.rhi[0]) || (j >= v.rlo[1] && j < v.rhi[1]);
  return true;
}

// Work-group (run c of the table of pair k): wave w of the 8 takes entry
// 8 c + w, so each wave's page loads are all in flight at once and the
// run's eight pages arrive together. Per page, S = K Q^T on the 16x16x32 MFMA
// (A: 16 keys x 32 dims of the token-major K page; B: the G query rows,
// columns G..15 zero), so lane l holds S[key 4 (l / 16) + i][head l % 16];
// that is exactly the A operand of the 16x16x16 PV product (rows = heads,
// k = keys), whose B operand is 4 keys of one d from the d-major V page.
// The run's max per head is taken before any exponential (two passes over
// the S registers), so no rescaling is needed; the run writes O unnormalised.
template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_main_kernel(DecArgs a) {
  constexpr int KST = D / 32;  // 32-dim steps of the QK product
  constexpr int DB = D / 16;   // 16-dim blocks of the PV product
  __shared__ float s_max[kDecWaves][16];
  __shared__ float s_sum[kDecWaves][16];
  __shared__ float s_o[kDecWaves][kDecMaxG][D];

  const int k = blockIdx.y, c = blockIdx.x;
  const int r = k / a.Hkv, h = k % a.Hkv;
  const int e0 = a.page_indptr[k], e1 = a.page_indptr[k + 1];
  if (e0 + c * kDecChunk >= e1) return;  // past the pair's table
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const HeadView v = head_view_dev(a.m, a.Hkv, r, h);

  // B operand of QK: query head h G + col, dims 32 s + 8 grp .. + 8
  bf16x8 qf[KST];
  const uint16_t* qrow = a.q_new + ((size_t)r * a.Hq + h * a.G + (col < a.G ? col : 0)) * D + 8 * grp;
#pragma unroll
  for (int s = 0; s < KST; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
    if (col >= a.G) qf[s] = bf16x8{};
  }
  // the wave's pages: K fragments and V fragments, all loads issued first
  int pos0[kDecPagesPerWave];
  bool have[kDecPagesPerWave];
  bf16x8 kf[kDecPagesPerWave][KST];
  s16x4 vf[kDecPagesPerWave][DB];
#pragma unroll
  for (int p = 0; p < kDecPagesPerWave; ++p) {
    const int e = e0 + c * kDecChunk + kDecPagesPerWave * wave + p;
    have[p] = e < e1;
    const int ec = have[p] ? e : e0;
    int pid = a.page_ids[ec];
    pos0[p] = a.page_pos[ec];
    SEGKV_DCHECK(g_dec_check, !have[p] || (pid >= 0 && pid < a.pool_pages), 1);
    if (pid < 0 || pid >= a.pool_pages) {
      have[p] = false;
      pid = 0;
    }
    const uint16_t* kp = a.k_pool + (size_t)pid * kPage * D + col * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < KST; ++s) kf[p][s] = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
    const uint16_t* vp = a.v_pool + (size_t)pid * D * kPage + col * kPage + 4 * grp;
#pragma unroll
    for (int b = 0; b < DB; ++b) vf[p][b] = *reinterpret_cast<const s16x4*>(vp + 16 * b * kPage);
  }
  // S, masked, in log2 units
  f32x4 sc[kDecPagesPerWave];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < kDecPagesPerWave; ++p) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KST; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[p][s], qf[s], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool vis = have[p] && dec_visible(v, pos0[p] + 4 * grp + i);
      sc[p][i] = vis ? acc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[p][i]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (grp == 0) s_max[wave][col] = mx;
  __syncthreads();
  float m = s_max[0][col];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) m = fmaxf(m, s_max[w][col]);
  const float m_use = m == -INFINITY ? 0.f : m;
  // P, the row sums, and O^T += V^T P^T page by page
  f32x4 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ls = 0.f;
#pragma unroll
  for (int p = 0; p < kDecPagesPerWave; ++p) {
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = sc[p][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[p][i] - m_use);
      ls += pv[i];
    }
    s16x4 pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[i] = (short)float_to_bf16_bits(pv[i]);
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vf[p][b], o[b], 0, 0, 0);
  }
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  if (grp == 0) s_sum[wave][col] = ls;
  // lane holds O[head 4 grp + i][d = 16 b + col]
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i < a.G) s_o[wave][4 * grp + i][16 * b + col] = o[b][i];
  __syncthreads();
  float* slot = a.ws + ((size_t)k * a.max_chunks + c) * a.G * (D + 2);
  for (int x = tid; x < a.G * D; x += kDecThreads) {
    const int g = x / D, d = x % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) sum += s_o[w][g][d];
    slot[g * (D + 2) + d] = sum;
  }
  if (tid < a.G) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) l += s_sum[w][tid];
    float mm = s_max[0][tid];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) mm = fmaxf(mm, s_max[w][tid]);
    slot[tid * (D + 2) + D] = mm;
    slot[tid * (D + 2) + D + 1] = l;
  }
}

// Work-group (request, query head, 16-dim slice of the head): merges the runs
// of its kv head's table and the new token:
//   m* = max(m_new, max_c m_c), L = 2^(m_new - m*) + sum_c 2^(m_c - m*) l_c,
//   O = (2^(m_new - m*) v_new + sum_c 2^(m_c - m*) O_c) / L, LSE = (m* + log2 L) ln 2,
// with m_new = scale log2(e) q . k_new. Thread (d, q) adds runs q, q + 64, ...
// into four accumulators (loads of four runs in flight); the partial sums are
// combined in a fixed order, so the result does not depend on timing.
constexpr int kDecCombThreads = 1024;
constexpr int kDecCombDims = 16;                                // dims per work-group
constexpr int kDecCombGroups = kDecCombThreads / kDecCombDims;  // run groups

__device__ __forceinline__ float dec_wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float dec_wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <int D>
__global__ __launch_bounds__(kDecCombThreads) void decode_combine_kernel(DecArgs a) {
  constexpr int NG = kDecCombGroups;
  constexpr int NW = kDecCombThreads / 64;
  __shared__ float s_wd[NW], s_wm[NW];
  __shared__ float s_acc[NG][kDecCombDims];
  __shared__ float s_l[NG];
  const int rg = blockIdx.x, r = rg / a.Hq, gq = rg % a.Hq, h = gq / a.G, g = gq % a.G;
  const int d0 = blockIdx.y * kDecCombDims;
  const int k = r * a.Hkv + h;
  const int nc = (a.page_indptr[k + 1] - a.page_indptr[k] + kDecChunk - 1) / kDecChunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* base = a.ws + (size_t)k * a.max_chunks * a.G * (D + 2) + (size_t)g * (D + 2);
  const size_t cstride = (size_t)a.G * (D + 2);
  // q . k_new over the whole head and the largest run max: wave sums, then waves in order
  const float prod = tid < D ? bf16_bits_to_float(a.q_new[((size_t)r * a.Hq + gq) * D + tid]) *
                                   bf16_bits_to_float(a.k_new[((size_t)r * a.Hkv + h) * D + tid])
                             : 0.f;
  float mx = -INFINITY;
  for (int cc = tid; cc < nc; cc += kDecCombThreads) mx = fmaxf(mx, base[cc * cstride + D]);
  const float wd = dec_wave_sum(prod), wm = dec_wave_max(mx);
  if (lane == 0) {
    s_wd[wave] = wd;
    s_wm[wave] = wm;
  }
  __syncthreads();
  float dot = 0.f, mruns = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    dot += s_wd[w];
    mruns = fmaxf(mruns, s_wm[w]);
  }
  const float m_new = dot * a.scale_log2;
  const float mstar = fmaxf(m_new, mruns);
  const int dl = tid % kDecCombDims, q = tid / kDecCombDims, d = d0 + dl;
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, ls[4] = {0.f, 0.f, 0.f, 0.f};
  int cc = q;
  for (; cc + 3 * NG < nc; cc += 4 * NG) {
    float mc[4], lc[4], oc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* sl = base + (cc + u * NG) * cstride;
      mc[u] = sl[D];
      lc[u] = sl[D + 1];
      oc[u] = sl[d];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = mc[u] == -INFINITY ? 0.f : exp2f(mc[u] - mstar);
      acc[u] += wgt * oc[u];
      ls[u] += wgt * lc[u];
    }
  }
#pragma unroll
  for (int u = 0; u < 3; ++u) {  // at most three runs left
    if (cc + u * NG < nc) {
      const float* sl = base + (cc + u * NG) * cstride;
      const float mc = sl[D];
      const float wgt = mc == -INFINITY ? 0.f : exp2f(mc - mstar);
      acc[u] += wgt * sl[d];
      ls[u] += wgt * sl[D + 1];
    }
  }
  s_acc[q][dl] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (dl == 0) s_l[q] = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  __syncthreads();
  if (tid < kDecCombDims) {
    const float wn = exp2f(m_new - mstar);
    float o = wn * bf16_bits_to_float(a.v_new[((size_t)r * a.Hkv + h) * D + d0 + tid]);
    float L = wn;
#pragma unroll
    for (int qq = 0; qq < NG; ++qq) {
      o += s_acc[qq][tid];
      L += s_l[qq];
    }
    a.out[((size_t)r * a.Hq + gq) * D + d0 + tid] = float_to_bf16_bits(o / L);
    if (tid == 0 && blockIdx.y == 0 && a.lse != nullptr) a.lse[(size_t)r * a.Hq + gq] = (mstar + log2f(L)) * kDecLn2;
  }
}

// Runs (of kDecChunk entries) of the longest table; 0 when every table is empty.
int32_t decode_max_chunks(const segkv_dims* dims, const segkv_meta* meta, int* max_chunks) {
  int32_t st = validate_layout(dims, meta);
  if (st != SEGKV_OK) return st;
  int mc = 0;
  for (int r = 0; r < dims->num_requests; ++r)
    for (int h = 0; h < dims->num_kv_heads; ++h) {
      const HeadView v = head_view_host(*dims, *meta, r, h);
      mc = imax(mc, cdiv(runs_count(head_page_runs(v)), kDecChunk));
    }
  *max_chunks = mc;
  return SEGKV_OK;
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" int32_t segkv_decode_workspace_size(const segkv_dims* dims, const segkv_meta* meta_host,
                                               size_t* bytes) {
  clear_error();
  if (!dims || !meta_host || !bytes) return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  int mc = 0;
  const int32_t st = decode_max_chunks(dims, meta_host, &mc);
  if (st != SEGKV_OK) return st;
  const int G = dims->num_q_heads / dims->num_kv_heads;
  *bytes = sizeof(float) * (size_t)dims->num_requests * dims->num_kv_heads * (size_t)imax(mc, 1) * G *
           (size_t)(dims->head_dim + 2);
  return SEGKV_OK;
}

extern "C" int32_t segpaged_attn_decode(const segkv_dims* dims, const segkv_meta* meta_host,
                                        const segkv_meta* meta_dev, const void* q_new, const void* k_new,
                                        const void* v_new, const void* k_pool, const void* v_pool,
                                        int64_t pool_pages, const int32_t* page_indptr_dev,
                                        const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                        float softmax_scale, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  clear_error();
  if (!dims || !meta_host || !meta_dev || !meta_dev->seg_indptr || !q_new || !k_new || !v_new || !k_pool ||
      !v_pool || !page_indptr_dev || !page_ids_dev || !page_pos_dev || !out)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  int mc = 0;
  int32_t st = decode_max_chunks(dims, meta_host, &mc);
  if (st != SEGKV_OK) return st;
  const int D = dims->head_dim, G = dims->num_q_heads / dims->num_kv_heads;
  if (D != 64 && D != 128) return fail(SEGKV_ERR_UNSUPPORTED, "decode supports head_dim 64 or 128");
  if (G > kDecMaxG) return fail(SEGKV_ERR_UNSUPPORTED, "decode supports at most 16 query heads per kv head");
  if (dims->page_size != kPage) return fail(SEGKV_ERR_UNSUPPORTED, "decode supports page_size 16");
  if (!(softmax_scale > 0.f)) return fail(SEGKV_ERR_INVALID_ARG, "softmax_scale must be > 0");
  if (pool_pages <= 0) return fail(SEGKV_ERR_INVALID_ARG, "pool_pages must be > 0");
  if (!aligned16(q_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(SEGKV_ERR_ALIGNMENT, "q_new, k_pool and v_pool must be 16-byte aligned");
  size_t need = 0;
  st = segkv_decode_workspace_size(dims, meta_host, &need);
  if (st != SEGKV_OK) return st;
  if (mc > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SEGKV_ERR_WORKSPACE, "workspace smaller than segkv_decode_workspace_size");
  if (dims->num_requests > 65535) return fail(SEGKV_ERR_UNSUPPORTED, "decode supports at most 65535 requests");
  DecArgs a;
  a.m = *meta_dev;
  a.q_new = static_cast<const uint16_t*>(q_new);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.pool_pages = pool_pages;
  a.page_indptr = page_indptr_dev;
  a.page_ids = page_ids_dev;
  a.page_pos = page_pos_dev;
  a.ws = static_cast<float*>(workspace);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.scale_log2 = softmax_scale * kDecLog2e;
  a.R = dims->num_requests;
  a.Hq = dims->num_q_heads;
  a.Hkv = dims->num_kv_heads;
  a.G = G;
  a.max_chunks = mc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mc > 0) {
    const dim3 grid(mc, a.R * a.Hkv);
    if (D == 128)
      decode_main_kernel<128><<<grid, kDecThreads, 0, s>>>(a);
    else
      decode_main_kernel<64><<<grid, kDecThreads, 0, s>>>(a);
    SEGKV_LAUNCH_CHECK();
  }
  if (D == 128)
    decode_combine_kernel<128><<<dim3(a.R * a.Hq, 128 / kDecCombDims), kDecCombThreads, 0, s>>>(a);
  else
    decode_combine_kernel<64><<<dim3(a.R * a.Hq, 64 / kDecCombDims), kDecCombThreads, 0, s>>>(a);
  SEGKV_LAUNCH_CHECK();
  SEGKV_DEVICE_CHECK(g_dec_check, s, "segpaged_attn_decode: a page-table entry is out of range");
  return SEGKV_OK;
}
