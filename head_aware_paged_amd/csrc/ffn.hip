// Token-selective (sparse) SwiGLU FFN.
//
// paooo.com "RedKnot的主要功能" (dense FFN on the top-k tokens by attention
// score, identity residual for the rest) and "RedKnot的技术原理" (FFN and
// attention optimised orthogonally); RedKnot README "About" (Elastic
// Sparsity). The selected rows are gathered straight into the first GEMM's
// operand tiles, the SwiGLU activation is formed in that GEMM's epilogue and
// stored once in bf16, and the second GEMM adds its result onto the selected
// rows of the residual stream in place. Unselected rows are never touched.
//
// Both GEMMs compute C^T = W X^T with the gfx950 32x32x16 bf16 MFMA (A = weight
// rows, B = token rows), so each lane ends up holding one token row and 4-wide
// runs of output features, which the epilogues store as 8-byte bf16 groups.
#include "common.h"

namespace segkv {
namespace {

constexpr int kFfnThreads = 256;
constexpr int kBK = 64;                // reduction depth per LDS stage
constexpr int kLdsStride = kBK + 8;    // padded row (elements)
constexpr int kRowsA = 128, kRowsB = 128;

enum { kModeSwiglu = 0, kModeResidual = 1 };

struct FfnArgs {
  const uint16_t* a0;   // weights: gate (SwiGLU) or down (residual)
  const uint16_t* a1;   // up weights (SwiGLU only)
  const uint16_t* x;    // token rows: hidden (gathered through idx) or the activation
  uint16_t* out;        // activation (SwiGLU) or hidden (residual, in place)
  const int32_t* idx;
  int k_tokens, K, out_ld, n_rows;
};

template <int MODE>
__global__ __launch_bounds__(kFfnThreads, 2) void ffn_gemm_kernel(FfnArgs a) {
  __shared__ uint16_t sa[kRowsA * kLdsStride];
  __shared__ uint16_t sb[kRowsB * kLdsStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  // SwiGLU: a block covers 64 activation features (gate rows 0..63, up rows 64..127 of the A tile)
  const int n0 = blockIdx.x * (MODE == kModeSwiglu ? 64 : kRowsA);
  const int m0 = blockIdx.y * kRowsB;

  // source rows of this thread's 16-byte loads (4 A chunks + 4 B chunks per stage)
  const uint16_t* arow[4];
  const uint16_t* brow[4];
  int lds_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int qd = tid + u * kFfnThreads;
    const int row = qd >> 3, c = qd & 7;
    lds_off[u] = row * kLdsStride + 8 * c;
    if (MODE == kModeSwiglu)
      arow[u] = (row < 64 ? a.a0 + (size_t)(n0 + row) * a.K : a.a1 + (size_t)(n0 + row - 64) * a.K) + 8 * c;
    else
      arow[u] = a.a0 + (size_t)(n0 + row) * a.K + 8 * c;
    const int m = m0 + row;
    const int src = m < a.k_tokens ? (MODE == kModeSwiglu ? a.idx[m] : m) : -1;
    if (src >= 0 && (MODE != kModeSwiglu || src < a.n_rows)) {
      brow[u] = a.x + (size_t)src * a.K + 8 * c;
    } else {
      brow[u] = nullptr;
    }
  }
  u32x4 ra[4], rb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = *reinterpret_cast<const u32x4*>(arow[u] + k0);
      rb[u] = brow[u] ? *reinterpret_cast<const u32x4*>(brow[u] + k0) : u32x4{0, 0, 0, 0};
    }
  };

  // wave's A rows: SwiGLU -> gate block wn and up block wn; residual -> blocks 2wn, 2wn+1
  const int arow0 = MODE == kModeSwiglu ? 32 * wn : 64 * wn;
  const int arow1 = MODE == kModeSwiglu ? 64 + 32 * wn : 64 * wn + 32;
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[x][y][i] = 0.f;

  fetch(0);
  for (int k0 = 0; k0 < a.K; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4*>(&sa[lds_off[u]]) = ra[u];
      *reinterpret_cast<u32x4*>(&sb[lds_off[u]]) = rb[u];
    }
    __syncthreads();
    if (k0 + kBK < a.K) fetch(k0 + kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int col = 16 * ks + 8 * lg;
      const bf16x8 fa0 = *reinterpret_cast<const bf16x8*>(&sa[(arow0 + lrow) * kLdsStride + col]);
      const bf16x8 fa1 = *reinterpret_cast<const bf16x8*>(&sa[(arow1 + lrow) * kLdsStride + col]);
      const bf16x8 fb0 = *reinterpret_cast<const bf16x8*>(&sb[(64 * wm + lrow) * kLdsStride + col]);
      const bf16x8 fb1 = *reinterpret_cast<const bf16x8*>(&sb[(64 * wm + 32 + lrow) * kLdsStride + col]);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb1, acc[1][1], 0, 0, 0);
    }
  }

  // lane holds token row m = m0 + 64 wm + 32 mb + lrow and features 8(i/4) + 4 lg + i%4 of each block
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + 64 * wm + 32 * mb + lrow;
    if (m >= a.k_tokens) continue;
    if (MODE == kModeSwiglu) {
      uint16_t* orow = a.out + (size_t)m * a.out_ld + n0 + 32 * wn;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint32_t pk = 0;
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const int i = 4 * g4 + 2 * e + hl;
            const float g = acc[0][mb][i], u = acc[1][mb][i];
            const float act = g / (1.f + __expf(-g)) * u;
            pk |= (uint32_t)float_to_bf16_bits(act) << (16 * hl);
          }
          w[e] = pk;
        }
        *reinterpret_cast<u32x2*>(orow + 8 * g4 + 4 * lg) = u32x2{w[0], w[1]};
      }
    } else {
      const int dst = a.idx[m];
      if (dst < 0 || dst >= a.n_rows) continue;  // out-of-range index: row skipped
      uint16_t* orow = a.out + (size_t)dst * a.out_ld + n0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint16_t* p = orow + 64 * wn + 32 * nb + 8 * g4 + 4 * lg;
          const u32x2 old = *reinterpret_cast<const u32x2*>(p);
          uint32_t w[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            uint32_t pk = 0;
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
              const int i = 4 * g4 + 2 * e + hl;
              const float h = bf16_bits_to_float((uint16_t)(old[e] >> (16 * hl)));
              pk |= (uint32_t)float_to_bf16_bits(h + acc[nb][mb][i]) << (16 * hl);
            }
            w[e] = pk;
          }
          *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
        }
    }
  }
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" size_t sparse_ffn_workspace_size(int32_t k, int32_t inter) {
  if (k <= 0 || inter <= 0) return 0;
  return (size_t)k * (size_t)inter * sizeof(uint16_t);
}

extern "C" int32_t sparse_ffn_swiglu(void* hidden, int32_t n_rows, int32_t hidden_size, int32_t inter,
                                     const int32_t* idx_dev, int32_t k, const void* w_gate, const void* w_up,
                                     const void* w_down, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (n_rows <= 0 || hidden_size <= 0 || inter <= 0 || k < 0 || k > n_rows)
    return fail(SEGKV_ERR_INVALID_ARG, "need n_rows, hidden_size, inter > 0 and 0 <= k <= n_rows");
  if (hidden_size % 128 != 0 || inter % 128 != 0)
    return fail(SEGKV_ERR_UNSUPPORTED, "hidden_size and inter must be multiples of 128");
  if (k == 0) return SEGKV_OK;
  if (!hidden || !idx_dev || !w_gate || !w_up || !w_down || !workspace)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (workspace_bytes < sparse_ffn_workspace_size(k, inter))
    return fail(SEGKV_ERR_WORKSPACE, "workspace smaller than sparse_ffn_workspace_size(k, inter)");
  if (!aligned16(hidden) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(workspace))
    return fail(SEGKV_ERR_ALIGNMENT, "tensors must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  FfnArgs g1;
  g1.a0 = static_cast<const uint16_t*>(w_gate);
  g1.a1 = static_cast<const uint16_t*>(w_up);
  g1.x = static_cast<const uint16_t*>(hidden);
  g1.out = static_cast<uint16_t*>(workspace);
  g1.idx = idx_dev;
  g1.k_tokens = k;
  g1.K = hidden_size;
  g1.out_ld = inter;
  g1.n_rows = n_rows;
  ffn_gemm_kernel<kModeSwiglu><<<dim3(inter / 64, cdiv(k, kRowsB)), kFfnThreads, 0, s>>>(g1);
  SEGKV_LAUNCH_CHECK();
  FfnArgs g2;
  g2.a0 = static_cast<const uint16_t*>(w_down);
  g2.a1 = nullptr;
  g2.x = static_cast<const uint16_t*>(workspace);
  g2.out = static_cast<uint16_t*>(hidden);
  g2.idx = idx_dev;
  g2.k_tokens = k;
  g2.K = inter;
  g2.out_ld = hidden_size;
  g2.n_rows = n_rows;
  ffn_gemm_kernel<kModeResidual><<<dim3(hidden_size / kRowsA, cdiv(k, kRowsB)), kFfnThreads, 0, s>>>(g2);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}
