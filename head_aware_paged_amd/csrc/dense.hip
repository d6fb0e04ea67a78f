// Masked-dense attention: the comparator of the paged, head-aware layout.
//
// paooo.com "RedKnot的技术原理" and "RedKnot的核心优势": the fused
// variable-length kernel replaces the general path of a dense [heads][keys]
// layout plus an attention mask, which the pages quote as several times
// slower. This is that general path on MI355X: every kv head's keys stored
// densely, one byte of mask per (kv head, query row, key), and every key of
// every row computed; the mask only decides which scores enter the softmax.
//
// Work split: wave = 16 query positions x HW query heads of one kv head (each
// K/V fragment feeds HW heads); work-group = 4 independent waves; grid z =
// runs of key tiles (split-KV), merged by a second kernel in a fixed order.
// Per step of 32 or 64 keys: S^T = K Q^T with the 16x16x32 bf16 MFMA (A = K rows,
// B = Q rows), whose accumulator layout (4 keys x 1 row per lane) is the A
// layout of the 16x16x16 MFMA for O = P V, so P stays in registers.
#include <algorithm>
#include <climits>

#include "common.h"

namespace segkv {
namespace {

constexpr int kDenThreads = 256;
constexpr int kDenWaves = kDenThreads / 64;
constexpr int kDenKeys = 64;          // keys per tile
constexpr int kDenRows = 16;          // query positions per wave
constexpr int kDenTargetGroups = 2048;
constexpr float kDenLn2 = 0.69314718055994530942f;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

struct DenArgs {
  const uint16_t* q;     // [T][Hq][D]
  const uint16_t* k;     // [Hkv][L][D]
  const uint16_t* vt;    // [Hkv][D][L]
  const uint8_t* mask;   // [Hkv][T][L]
  float* ws;             // [chunks][T][Hq][D + 2]: O (unnormalised), m (log2 units), l
  uint16_t* out;         // [T][Hq][D]
  float* lse;            // [T][Hq] natural log, or null
  float scale_log2;
  int T, Hq, Hkv, G, L, units, tiles_per_chunk;
};

template <int D, int HW>
__global__ __launch_bounds__(kDenThreads, 2) void dense_main_kernel(DenArgs a) {
  constexpr int KST = D / 32;  // 32-dim steps of QK
  constexpr int DB = D / 16;   // 16-dim blocks of PV
  // 16-key blocks per softmax step: 2 where the fragments of 4 would not fit the registers
  constexpr int SB = D == 128 && HW == 2 ? 2 : 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, c = blockIdx.z;
  const int u = blockIdx.x * kDenWaves + wave;
  if (u >= a.units) return;  // waves share no LDS and no barrier
  const int hpg = a.G / HW;
  const int t0 = (u / hpg) * kDenRows, g0 = h * a.G + (u % hpg) * HW;
  const int trow = min(t0 + col, a.T - 1);  // this lane's query row (clamped; rows >= T are not written)

  bf16x8 qf[HW][KST];
#pragma unroll
  for (int hh = 0; hh < HW; ++hh)
#pragma unroll
    for (int s = 0; s < KST; ++s)
      qf[hh][s] = *reinterpret_cast<const bf16x8*>(a.q + ((size_t)trow * a.Hq + g0 + hh) * D + 32 * s + 8 * grp);
  f32x4 o[HW][DB];
  float m[HW], l[HW];
#pragma unroll
  for (int hh = 0; hh < HW; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) o[hh][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint8_t* mrow = a.mask + ((size_t)h * a.T + trow) * a.L;
  const uint16_t* kh = a.k + (size_t)h * a.L * D;
  const uint16_t* vh = a.vt + (size_t)h * D * a.L;
  const int kt0 = c * a.tiles_per_chunk;
  const int kt1 = min(kt0 + a.tiles_per_chunk, a.L / kDenKeys);
  for (int j0 = kt0 * kDenKeys; j0 < kt1 * kDenKeys; j0 += 16 * SB) {
    bf16x8 kf[SB][KST];
    uint32_t mk[SB];
    s16x4 vf[SB][DB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const uint16_t* kp = kh + (size_t)(j0 + 16 * sb + col) * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < KST; ++s) kf[sb][s] = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
      mk[sb] = *reinterpret_cast<const uint32_t*>(mrow + j0 + 16 * sb + 4 * grp);
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int b = 0; b < DB; ++b)
        vf[sb][b] = *reinterpret_cast<const s16x4*>(vh + (size_t)(16 * b + col) * a.L + j0 + 16 * sb + 4 * grp);
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      // lane: keys j0 + 16 sb + 4 grp + i of row `col`, log2 units, masked
      f32x4 sc[SB];
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KST; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[sb][s], qf[hh][s], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[sb][i] = (mk[sb] >> (8 * i)) & 0xffu ? acc[i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[sb][i]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m[hh], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mu);
      m[hh] = mn;
      l[hh] *= alpha;
      // O rows are 4 grp + i; the scale of row r sits in lane r
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ar = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int b = 0; b < DB; ++b) o[hh][b][i] *= ar;
      }
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        s16x4 pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = sc[sb][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[sb][i] - mu);
          l[hh] += p;
          pa[i] = (short)float_to_bf16_bits(p);
        }
#pragma unroll
        for (int b = 0; b < DB; ++b) o[hh][b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vf[sb][b], o[hh][b], 0, 0, 0);
      }
    }
  }
  // partial of this run of tiles: O rows 4 grp + i, dims 16 b + col; (m, l) of row `col`
#pragma unroll
  for (int hh = 0; hh < HW; ++hh) {
    float ls = l[hh];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    float* base = a.ws + ((size_t)c * a.T * a.Hq + g0 + hh) * (D + 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * grp + i;
      if (t < a.T) {
        float* row = base + (size_t)t * a.Hq * (D + 2);
#pragma unroll
        for (int b = 0; b < DB; ++b) row[16 * b + col] = o[hh][b][i];
      }
    }
    if (grp == 0 && t0 + col < a.T) {
      float* row = base + (size_t)(t0 + col) * a.Hq * (D + 2);
      row[D] = m[hh];
      row[D + 1] = ls;
    }
  }
}

// One work-group per (query row, query head): merges the runs in order.
template <int D>
__global__ __launch_bounds__(D) void dense_combine_kernel(DenArgs a, int chunks) {
  const int rg = blockIdx.x, d = threadIdx.x;
  const size_t stride = (size_t)a.T * a.Hq * (D + 2);
  const float* base = a.ws + (size_t)rg * (D + 2);
  float mstar = -INFINITY;
  for (int c = 0; c < chunks; ++c) mstar = fmaxf(mstar, base[c * stride + D]);
  float L = 0.f, o = 0.f;
  if (mstar != -INFINITY) {
    for (int c = 0; c < chunks; ++c) {
      const float mc = base[c * stride + D];
      const float w = mc == -INFINITY ? 0.f : exp2f(mc - mstar);
      L += w * base[c * stride + D + 1];
      o += w * base[c * stride + d];
    }
    o /= L;
  }
  a.out[(size_t)rg * D + d] = float_to_bf16_bits(o);
  if (d == 0 && a.lse != nullptr) a.lse[rg] = mstar == -INFINITY ? -INFINITY : (mstar + log2f(L)) * kDenLn2;
}

struct DenPlan {
  int hw, units, tiles_per_chunk, chunks, groups;
};

DenPlan dense_plan(int T, int Hq, int Hkv, int L) {
  DenPlan p;
  const int G = Hq / Hkv;
  p.hw = G % 2 == 0 ? 2 : 1;
  p.units = cdiv(T, kDenRows) * (G / p.hw);
  p.groups = cdiv(p.units, kDenWaves);
  const int tiles = L / kDenKeys;
  const int want = std::max(1, std::min(tiles, cdiv(kDenTargetGroups, p.groups * Hkv)));
  p.tiles_per_chunk = cdiv(tiles, want);
  p.chunks = cdiv(tiles, p.tiles_per_chunk);
  return p;
}

int32_t dense_check(int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t L) {
  if (T <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || Hq % Hkv != 0)
    return fail(SEGKV_ERR_INVALID_ARG, "need T, Hq, Hkv, L > 0 and Hq a multiple of Hkv");
  if (D != 64 && D != 128) return fail(SEGKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (L % kDenKeys != 0) return fail(SEGKV_ERR_UNSUPPORTED, "L must be a multiple of 64 (pad with masked keys)");
  if ((int64_t)Hkv * T * L > (int64_t)1 << 40) return fail(SEGKV_ERR_UNSUPPORTED, "mask too large");
  if ((int64_t)T * Hq > INT32_MAX) return fail(SEGKV_ERR_UNSUPPORTED, "T * Hq must fit in 31 bits");
  return SEGKV_OK;
}

size_t dense_ws_bytes(int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t L) {
  const DenPlan p = dense_plan(T, Hq, Hkv, L);
  return (size_t)p.chunks * T * Hq * (D + 2) * sizeof(float);
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" int32_t segkv_masked_dense_workspace_size(int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t L,
                                                     size_t* bytes) {
  clear_error();
  if (!bytes) return fail(SEGKV_ERR_INVALID_ARG, "bytes is NULL");
  const int32_t st = dense_check(T, Hq, Hkv, D, L);
  if (st != SEGKV_OK) return st;
  *bytes = dense_ws_bytes(T, Hq, Hkv, D, L);
  return SEGKV_OK;
}

extern "C" int32_t masked_dense_attn(const void* q, const void* k, const void* v_t, const uint8_t* mask, int32_t T,
                                     int32_t Hq, int32_t Hkv, int32_t D, int32_t L, float softmax_scale, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const int32_t st = dense_check(T, Hq, Hkv, D, L);
  if (st != SEGKV_OK) return st;
  if (!q || !k || !v_t || !mask || !out || !workspace) return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(softmax_scale > 0.f)) return fail(SEGKV_ERR_INVALID_ARG, "softmax_scale must be > 0");
  if (workspace_bytes < dense_ws_bytes(T, Hq, Hkv, D, L))
    return fail(SEGKV_ERR_WORKSPACE, "workspace smaller than segkv_masked_dense_workspace_size");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v_t) || !aligned16(mask) || !aligned16(out) ||
      !aligned16(workspace) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(SEGKV_ERR_ALIGNMENT, "tensors must be 16-byte aligned");
  const DenPlan p = dense_plan(T, Hq, Hkv, L);
  DenArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.vt = static_cast<const uint16_t*>(v_t);
  a.mask = mask;
  a.ws = static_cast<float*>(workspace);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.L = L;
  a.units = p.units;
  a.tiles_per_chunk = p.tiles_per_chunk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(p.groups, Hkv, p.chunks);
  if (D == 128) {
    if (p.hw == 2)
      dense_main_kernel<128, 2><<<grid, kDenThreads, 0, s>>>(a);
    else
      dense_main_kernel<128, 1><<<grid, kDenThreads, 0, s>>>(a);
  } else {
    if (p.hw == 2)
      dense_main_kernel<64, 2><<<grid, kDenThreads, 0, s>>>(a);
    else
      dense_main_kernel<64, 1><<<grid, kDenThreads, 0, s>>>(a);
  }
  SEGKV_LAUNCH_CHECK();
  if (D == 128)
    dense_combine_kernel<128><<<(unsigned)(T * Hq), 128, 0, s>>>(a, p.chunks);
  else
    dense_combine_kernel<64><<<(unsigned)(T * Hq), 64, 0, s>>>(a, p.chunks);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}
