// BUILDSTATE relocation + page gather: cached segment K rotated to its new
// positions, V copied alongside so K and V share one page table.
//
// RedKnot README ("About": offline KV reuse with RoPE relocation that keeps
// the reused KV numerically aligned; "Key Ideas": offline KV cache + RoPE
// relocation); aitrends.kr "주요 기능" (stored KV re-aligned to the current
// context's positions). Rotate-half RoPE with omega_j = theta^(-2j/D): moving
// a key by delta positions rotates pair (j, j + D/2) by delta * omega_j.
//
// Bandwidth-bound: every move reads and writes one K page (and one V page).
// A work-group takes a batch of 1 (D = 128) or 2 (D = 64) moves, so that a
// layer's few thousand moves spread over many work-groups per CU; it keeps all
// 16-byte loads of the batch in flight and computes the batch's cos/sin table
// (angle reduced in fp64, cos/sin in fp32, in LDS) while they fly.
#include <cmath>

#include "common.h"

namespace segkv {
namespace {

SEGKV_DEVICE_FLAG(g_reloc_check);  // bit 1: a move's source or destination page outside its pool

constexpr int kRelocThreads = 128;
template <int D>
constexpr int moves_per_batch() { return D == 128 ? 1 : 2; }

template <int D>
__global__ __launch_bounds__(kRelocThreads) void relocate_kernel(
    const uint16_t* __restrict__ k_src, uint16_t* __restrict__ k_dst, const uint16_t* __restrict__ v_src,
    uint16_t* __restrict__ v_dst, int64_t src_pages, int64_t dst_pages, const int32_t* __restrict__ src_page,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ delta, int n_moves, double log2_theta) {
  constexpr int kMovesPerBatch = moves_per_batch<D>();
  constexpr int kHalf = D / 2;
  constexpr int kChunksPerHalf = kHalf / 8;          // 16-byte chunks in one half row
  constexpr int kPairsPerPage = kPage * kChunksPerHalf;
  constexpr int kKPairs = kMovesPerBatch * kPairsPerPage;
  constexpr int kKPerThread = kKPairs / kRelocThreads;
  constexpr int kVChunks = kMovesPerBatch * kPage * D / 8;
  constexpr int kVPerThread = kVChunks / kRelocThreads;
  static_assert(kKPairs % kRelocThreads == 0 && kVChunks % kRelocThreads == 0, "batch shape");

  __shared__ double inv_freq[kHalf];
  __shared__ float cs[kMovesPerBatch][kHalf][2];
  __shared__ int s_src[kMovesPerBatch], s_dst[kMovesPerBatch], s_ok[kMovesPerBatch], s_delta[kMovesPerBatch];

  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kMovesPerBatch;
  if (tid < kMovesPerBatch) {
    const int m = m0 + tid;
    int s = -1, d = -1, ok = 0, dl = 0;
    if (m < n_moves) {
      s = src_page[m];
      d = dst_page[m];
      dl = delta[m];
      ok = (s >= 0 && s < src_pages && d >= 0 && d < dst_pages) ? 1 : 0;
      SEGKV_DCHECK(g_reloc_check, ok, 1);
    }
    s_src[tid] = s;
    s_dst[tid] = d;
    s_ok[tid] = ok;
    s_delta[tid] = dl;
  }
  __syncthreads();
  // issue every load of the batch first; the cos/sin table is computed while they fly
  u32x4 kx[kKPerThread], ky[kKPerThread], vv[kVPerThread];
#pragma unroll
  for (int u = 0; u < kKPerThread; ++u) {
    const int q = tid + u * kRelocThreads;
    const int b = q / kPairsPerPage, w = q % kPairsPerPage;
    const int t = w / kChunksPerHalf, c = w % kChunksPerHalf;
    if (s_ok[b]) {
      const u32x4* row = reinterpret_cast<const u32x4*>(k_src + ((size_t)s_src[b] * kPage + t) * D);
      kx[u] = __builtin_nontemporal_load(row + c);  // the cached segment is read once
      ky[u] = __builtin_nontemporal_load(row + c + kChunksPerHalf);
    }
  }
  if (v_src != nullptr) {
#pragma unroll
    for (int u = 0; u < kVPerThread; ++u) {
      const int q = tid + u * kRelocThreads;
      const int b = q / (kPage * D / 8), w = q % (kPage * D / 8);
      if (s_ok[b]) vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_src + (size_t)s_src[b] * kPage * D) + w);
    }
  }
  if (tid < kHalf) inv_freq[tid] = exp2(-2.0 * (double)tid / (double)D * log2_theta);
  __syncthreads();
  for (int e = tid; e < kMovesPerBatch * kHalf; e += kRelocThreads) {
    const int b = e / kHalf, j = e % kHalf;
    float sn = 0.f, cn = 1.f;
    if (s_ok[b]) {
      // angle in fp64, reduced to [-pi, pi] in fp64 by Cody-Waite reduction
      // (x - n C1 - n C2 with 2 pi = C1 + C2, C1 the fp64 value of 2 pi and C2
      // its remainder), then cos/sin in fp32
      const double ang = (double)s_delta[b] * inv_freq[j];
      const double n = rint(ang * 0.15915494309189535);
      sincosf((float)fma(-n, 2.4492935982947064e-16, fma(-n, 6.283185307179586, ang)), &sn, &cn);
    }
    cs[b][j][0] = cn;
    cs[b][j][1] = sn;
  }

  __syncthreads();

#pragma unroll
  for (int u = 0; u < kKPerThread; ++u) {
    const int q = tid + u * kRelocThreads;
    const int b = q / kPairsPerPage, w = q % kPairsPerPage;
    const int t = w / kChunksPerHalf, c = w % kChunksPerHalf;
    if (!s_ok[b]) continue;
    u32x4 ox, oy;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t outx = 0, outy = 0;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int j = c * 8 + e * 2 + hlf;
        const float co = cs[b][j][0], si = cs[b][j][1];
        const float x = bf16_bits_to_float((uint16_t)(kx[u][e] >> (16 * hlf)));
        const float y = bf16_bits_to_float((uint16_t)(ky[u][e] >> (16 * hlf)));
        const float rx = fmaf(x, co, -y * si);
        const float ry = fmaf(x, si, y * co);
        outx |= (uint32_t)float_to_bf16_bits(rx) << (16 * hlf);
        outy |= (uint32_t)float_to_bf16_bits(ry) << (16 * hlf);
      }
      ox[e] = outx;
      oy[e] = outy;
    }
    u32x4* row = reinterpret_cast<u32x4*>(k_dst + ((size_t)s_dst[b] * kPage + t) * D);
    row[c] = ox;
    row[c + kChunksPerHalf] = oy;
  }
  if (v_src != nullptr) {
#pragma unroll
    for (int u = 0; u < kVPerThread; ++u) {
      const int q = tid + u * kRelocThreads;
      const int b = q / (kPage * D / 8), w = q % (kPage * D / 8);
      if (s_ok[b]) reinterpret_cast<u32x4*>(v_dst + (size_t)s_dst[b] * kPage * D)[w] = vv[u];
    }
  }
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" int32_t rope_relocate(const void* k_src, void* k_dst, const void* v_src, void* v_dst,
                                 int64_t src_pool_pages, int64_t dst_pool_pages, const int32_t* src_page_dev,
                                 const int32_t* dst_page_dev, const int32_t* delta_dev, int32_t n_moves,
                                 int32_t page_size, int32_t head_dim, double rope_theta, void* stream) {
  clear_error();
  if (n_moves < 0) return fail(SEGKV_ERR_INVALID_ARG, "n_moves must be >= 0");
  if (page_size != kPage) return fail(SEGKV_ERR_UNSUPPORTED, "page_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(SEGKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(rope_theta > 0.0)) return fail(SEGKV_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (src_pool_pages < 0 || dst_pool_pages < 0) return fail(SEGKV_ERR_INVALID_ARG, "pool sizes must be >= 0");
  if (n_moves == 0) return SEGKV_OK;
  if (!k_src || !k_dst || !src_page_dev || !dst_page_dev || !delta_dev)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((v_src == nullptr) != (v_dst == nullptr))
    return fail(SEGKV_ERR_INVALID_ARG, "v_src and v_dst must both be given or both be NULL");
  if (!aligned16(k_src) || !aligned16(k_dst) || (v_src && (!aligned16(v_src) || !aligned16(v_dst))))
    return fail(SEGKV_ERR_ALIGNMENT, "pools must be 16-byte aligned");
  const int grid = cdiv(n_moves, head_dim == 128 ? moves_per_batch<128>() : moves_per_batch<64>());
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto ks = static_cast<const uint16_t*>(k_src);
  auto kd = static_cast<uint16_t*>(k_dst);
  auto vs = static_cast<const uint16_t*>(v_src);
  auto vd = static_cast<uint16_t*>(v_dst);
  if (head_dim == 128)
    relocate_kernel<128><<<grid, kRelocThreads, 0, s>>>(ks, kd, vs, vd, src_pool_pages, dst_pool_pages,
                                                        src_page_dev, dst_page_dev, delta_dev, n_moves, std::log2(rope_theta));
  else
    relocate_kernel<64><<<grid, kRelocThreads, 0, s>>>(ks, kd, vs, vd, src_pool_pages, dst_pool_pages,
                                                       src_page_dev, dst_page_dev, delta_dev, n_moves, std::log2(rope_theta));
  SEGKV_LAUNCH_CHECK();
  SEGKV_DEVICE_CHECK(g_reloc_check, s, "rope_relocate: a move's page id is outside its pool");
  return SEGKV_OK;
}
