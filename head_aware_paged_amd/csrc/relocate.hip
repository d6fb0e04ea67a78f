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
// A 256-thread work-group takes a batch of 2 (D = 128) or 4 (D = 64) moves,
// 16 KiB of K and V. The chunks a wave copies always lie in one move, so the
// page ids come in by scalar loads with no barrier before the page loads; all 16-byte
// loads of the batch are issued first (V, then K), the batch's cos/sin table
// (angle reduced in fp64, cos/sin in fp32, in LDS) is computed while they fly,
// V is stored as soon as it lands, then K is rotated and stored. Pages are
// read once and written once, so loads and stores are non-temporal (on random
// 4 KiB pages this gets within a few per cent of a plain copy of the same
// pages).
#include <cmath>

#include "common.h"

namespace segkv {
namespace {

SEGKV_DEVICE_FLAG(g_reloc_check);  // bit 1: a move's source or destination page outside its pool

constexpr int kRelocThreads = 256;
template <int D>
constexpr int moves_per_batch() { return D == 128 ? 2 : 4; }

template <int D>
__global__ __launch_bounds__(kRelocThreads) void relocate_kernel(
    const uint16_t* __restrict__ k_src, uint16_t* __restrict__ k_dst, const uint16_t* __restrict__ v_src,
    uint16_t* __restrict__ v_dst, int64_t src_pages, int64_t dst_pages, const int32_t* __restrict__ src_page,
    const int32_t* __restrict__ dst_page, const int32_t* __restrict__ delta, int n_moves, double log2_theta) {
  constexpr int kMovesPerBatch = moves_per_batch<D>();
  constexpr int kHalf = D / 2;
  constexpr int kChunksPerHalf = kHalf / 8;          // 16-byte chunks in one half row
  constexpr int kPairsPerPage = kPage * kChunksPerHalf;
  constexpr int kVChunksPerPage = kPage * D / 8;
  constexpr int kKPerThread = kMovesPerBatch * kPairsPerPage / kRelocThreads;
  constexpr int kVPerThread = kMovesPerBatch * kVChunksPerPage / kRelocThreads;
  static_assert(kKPerThread * kRelocThreads == kMovesPerBatch * kPairsPerPage &&
                kVPerThread * kRelocThreads == kMovesPerBatch * kVChunksPerPage, "batch shape");
  static_assert(kPairsPerPage % 64 == 0 && kVChunksPerPage % 64 == 0, "a wave's chunks must lie in one move");

  __shared__ double inv_freq[kHalf];
  __shared__ float cs[kMovesPerBatch][kHalf][2];

  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kMovesPerBatch;
  // the move of a wave's chunk, its page ids (scalar loads) and whether both ids are in range
  auto move_of = [&](int b, int& s, int& d) {
    const int m = m0 + b;
    s = -1;
    d = -1;
    if (m < n_moves) {
      const int s_ = src_page[m], d_ = dst_page[m];
      const bool ok = s_ >= 0 && s_ < src_pages && d_ >= 0 && d_ < dst_pages;
      SEGKV_DCHECK(g_reloc_check, ok, 1);
      if (ok) {
        s = s_;
        d = d_;
      }
    }
  };
  u32x4 kx[kKPerThread], ky[kKPerThread], vv[kVPerThread];
  int kd[kKPerThread], vd[kVPerThread];
  if (v_src != nullptr) {
#pragma unroll
    for (int u = 0; u < kVPerThread; ++u) {
      const int q = tid + u * kRelocThreads;
      int s_, d_;
      move_of(__builtin_amdgcn_readfirstlane(q / kVChunksPerPage), s_, d_);
      vd[u] = d_;
      if (s_ >= 0)
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_src + (size_t)s_ * kPage * D) +
                                           q % kVChunksPerPage);  // the cached segment is read once
    }
  }
#pragma unroll
  for (int u = 0; u < kKPerThread; ++u) {
    const int q = tid + u * kRelocThreads;
    const int w = q % kPairsPerPage, t = w / kChunksPerHalf, c = w % kChunksPerHalf;
    int s_, d_;
    move_of(__builtin_amdgcn_readfirstlane(q / kPairsPerPage), s_, d_);
    kd[u] = d_;
    if (s_ >= 0) {
      const u32x4* row = reinterpret_cast<const u32x4*>(k_src + ((size_t)s_ * kPage + t) * D);
      kx[u] = __builtin_nontemporal_load(row + c);
      ky[u] = __builtin_nontemporal_load(row + c + kChunksPerHalf);
    }
  }
  if (tid < kHalf) inv_freq[tid] = exp2(-2.0 * (double)tid / (double)D * log2_theta);
  __syncthreads();
  for (int e = tid; e < kMovesPerBatch * kHalf; e += kRelocThreads) {
    const int b = e / kHalf, j = e % kHalf;
    float sn = 0.f, cn = 1.f;
    if (m0 + b < n_moves) {
      // angle in fp64, reduced to [-pi, pi] in fp64 by Cody-Waite reduction
      // (x - n C1 - n C2 with 2 pi = C1 + C2, C1 the fp64 value of 2 pi and C2
      // its remainder), then cos/sin in fp32
      const double ang = (double)delta[m0 + b] * inv_freq[j];
      const double n = rint(ang * 0.15915494309189535);
      sincosf((float)fma(-n, 2.4492935982947064e-16, fma(-n, 6.283185307179586, ang)), &sn, &cn);
    }
    cs[b][j][0] = cn;
    cs[b][j][1] = sn;
  }
  if (v_src != nullptr) {
#pragma unroll
    for (int u = 0; u < kVPerThread; ++u) {
      const int q = tid + u * kRelocThreads;
      if (vd[u] >= 0)
        __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(v_dst + (size_t)vd[u] * kPage * D) + q % kVChunksPerPage);
    }
  }
  __syncthreads();

#pragma unroll
  for (int u = 0; u < kKPerThread; ++u) {
    const int q = tid + u * kRelocThreads;
    const int b = q / kPairsPerPage, w = q % kPairsPerPage;
    const int t = w / kChunksPerHalf, c = w % kChunksPerHalf;
    if (kd[u] < 0) continue;
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
    u32x4* row = reinterpret_cast<u32x4*>(k_dst + ((size_t)kd[u] * kPage + t) * D);
    __builtin_nontemporal_store(ox, row + c);
    __builtin_nontemporal_store(oy, row + c + kChunksPerHalf);
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
