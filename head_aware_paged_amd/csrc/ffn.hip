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
#include <climits>
#include <mutex>

#include <cmath>

#include "common.h"
#include "plan.h"

namespace segkv {
namespace {

constexpr int kFfnThreads = 256;
constexpr int kBK = 64;                // reduction depth per LDS stage
constexpr int kLdsStride = kBK + 8;    // padded row (elements)
constexpr int kRowsA = 128, kRowsB = 128;

enum { kModeSwiglu = 0, kModeResidual = 1 };

// 128-row token tiles leave CUs idle when a launch has fewer than two
// work-groups per CU (256 CUs); 64-row tiles double the count.
inline bool small_grid(int n_tiles, int rows) { return (int64_t)n_tiles * cdiv(rows, kRowsB) < 512; }

struct FfnArgs {
  const uint16_t* a0;   // weights: gate (SwiGLU) or down (residual)
  const uint16_t* a1;   // up weights (SwiGLU only)
  const uint16_t* x;    // token rows: hidden (gathered through idx) or the activation
  uint16_t* out;        // activation (SwiGLU) or hidden (residual, in place)
  const int32_t* idx;
  int k_tokens, K, out_ld, n_rows;
};

// Main loop shared by the projections: the work-group's C^T tile (128 weight
// rows x 128 token rows) over the reduction dimension K, staged through LDS in
// kBK-deep slices, each slice's global loads issued kStages slices ahead. Thread u-th
// 16-byte chunks: weight row arow[u], token row brow[u] (NULL: zero row).
// Wave (wn, wm) accumulates weight rows arow0..+31 (acc[0]) and arow1..+31
// (acc[1]) against NB blocks of 32 token rows from 32 NB wm (acc[.][b]); the
// token tile is 64 NB rows (NB = 1 halves it, doubling the work-groups of a
// launch with few token rows).
template <int NB>
__device__ __forceinline__ void gemm_tile(const uint16_t* const (&arow)[4], const uint16_t* const (&brow)[2 * NB],
                                          const int (&lds_off)[4], int K, int arow0, int arow1, int wm,
                                          uint16_t* sa, uint16_t* sb, f32x16 (&acc)[2][NB]) {
  const int lane = threadIdx.x & 63, lrow = lane & 31, lg = lane >> 5;
  // a ring of kStages register sets: slice k is loaded kStages slices ahead of
  // its use. The 64-row token tile (fewer waves per CU's worth of work) takes
  // three; the 128-row tile keeps one, as more stages cost it occupancy.
  constexpr int kStages = NB == 1 ? 3 : 1;
  u32x4 ra[kStages][4], rb[kStages][2 * NB];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[x][y][i] = 0.f;
#pragma unroll
  for (int st = 0; st < kStages; ++st)
    if (st * kBK < K) {
#pragma unroll
      for (int u = 0; u < 4; ++u) ra[st][u] = *reinterpret_cast<const u32x4*>(arow[u] + st * kBK);
#pragma unroll
      for (int u = 0; u < 2 * NB; ++u)
        rb[st][u] = brow[u] ? *reinterpret_cast<const u32x4*>(brow[u] + st * kBK) : u32x4{0, 0, 0, 0};
    }
  for (int k0 = 0; k0 < K; k0 += kStages * kBK) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int kk = k0 + st * kBK;
      if (kk >= K) break;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(&sa[lds_off[u]]) = ra[st][u];
#pragma unroll
      for (int u = 0; u < 2 * NB; ++u) *reinterpret_cast<u32x4*>(&sb[lds_off[u]]) = rb[st][u];
      __syncthreads();
      const int kn = kk + kStages * kBK;
      if (kn < K) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ra[st][u] = *reinterpret_cast<const u32x4*>(arow[u] + kn);
#pragma unroll
        for (int u = 0; u < 2 * NB; ++u)
          rb[st][u] = brow[u] ? *reinterpret_cast<const u32x4*>(brow[u] + kn) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        const int col = 16 * ks + 8 * lg;
        const bf16x8 fa0 = *reinterpret_cast<const bf16x8*>(&sa[(arow0 + lrow) * kLdsStride + col]);
        const bf16x8 fa1 = *reinterpret_cast<const bf16x8*>(&sa[(arow1 + lrow) * kLdsStride + col]);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const bf16x8 fb =
              *reinterpret_cast<const bf16x8*>(&sb[(32 * NB * wm + 32 * bb + lrow) * kLdsStride + col]);
          acc[0][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb, acc[0][bb], 0, 0, 0);
          acc[1][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb, acc[1][bb], 0, 0, 0);
        }
      }
    }
  }
}

template <int MODE, int NB>
__global__ __launch_bounds__(kFfnThreads, 2) void ffn_gemm_kernel(FfnArgs a) {
  __shared__ uint16_t sa[kRowsA * kLdsStride];
  __shared__ uint16_t sb[kRowsB * kLdsStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  // SwiGLU: a block covers 64 activation features (gate rows 0..63, up rows 64..127 of the A tile)
  const int n0 = blockIdx.x * (MODE == kModeSwiglu ? 64 : kRowsA);
  const int m0 = blockIdx.y * 64 * NB;

  // source rows of this thread's 16-byte loads (4 A chunks + 2 NB B chunks per stage)
  const uint16_t* arow[4];
  const uint16_t* brow[2 * NB];
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
    if (u >= 2 * NB) continue;
    const int m = m0 + row;
    const int src = m < a.k_tokens ? (MODE == kModeSwiglu ? a.idx[m] : m) : -1;
    if (src >= 0 && (MODE != kModeSwiglu || src < a.n_rows)) {
      brow[u] = a.x + (size_t)src * a.K + 8 * c;
    } else {
      brow[u] = nullptr;
    }
  }
  // wave's A rows: SwiGLU -> gate block wn and up block wn; residual -> blocks 2wn, 2wn+1
  const int arow0 = MODE == kModeSwiglu ? 32 * wn : 64 * wn;
  const int arow1 = MODE == kModeSwiglu ? 64 + 32 * wn : 64 * wn + 32;
  f32x16 acc[2][NB];
  gemm_tile<NB>(arow, brow, lds_off, a.K, arow0, arow1, wm, sa, sb, acc);

  // lane holds token row m = m0 + 32 NB wm + 32 mb + lrow and features 8(i/4) + 4 lg + i%4 of each block
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    const int m = m0 + 32 * NB * wm + 32 * mb + lrow;
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
      const int dst = a.idx ? a.idx[m] : m;  // no index list: row m itself
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

// ---- large-tile projections: the LDS-ring main loop and its kernels ----
//
// Same products and epilogues as ffn_gemm_kernel. A work-group has NA x NB
// waves; each wave computes (32 WA) x (32 WB) outputs, the work-group
// (NA 32 WA) weight rows x (NB 32 WB) token rows. Each 16-byte LDS fragment
// feeds WB (A) or WA (B) MFMAs. The sparse FFN runs 8 waves (two per SIMD,
// so one wave's MFMAs fill the matrix core while the other waits on LDS or a
// barrier) on 256 x 256 and 128 x 256 tiles; the layer glue and launches
// with few token rows run 4 waves on 128 x 128 and 128 x 64 tiles, two
// work-groups per CU. K goes in 32-deep slices through a ring of kBigStages LDS stages,
// filled by buffer loads with the LDS destination (no register staging),
// each slice issued kBigStages - 1 slices ahead. A stage row is 32 bf16 =
// four 16-byte chunks; chunk c of row r sits at slot c ^ ((r / 4) % 4), so
// the 16-byte operand reads of 16 consecutive rows fall in distinct bank
// groups. Rows that do not exist (token rows past k, an out-of-range index,
// weight rows past the last head) read as zeros through the buffer's range
// check.
constexpr int kBigBK = 32;        // reduction depth per slice
constexpr int kBigStages = 4;     // LDS ring depth
constexpr int kBigRowBytes = kBigBK * 2;
constexpr int kBigRowsPerDma = 16;  // rows of one 1 KiB buffer-to-LDS instruction
constexpr uint32_t kBigOob = 0x7FFFFFF0u;  // a source offset past every buffer: reads zeros
// s_waitcnt immediate with lgkmcnt and expcnt at their maximum (not waited
// for) and vmcnt n (gfx9 encoding: vmcnt low bits 3:0, high bits 15:14)
constexpr int big_wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ u32x4 big_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)), bytes, 0x00020000u};
}
__device__ __forceinline__ int big_swz(int row) { return (row >> 2) & 3; }

// Tile shape: NA x NB waves, wave w in wave row w % NA (its 32 WA weight
// rows) and wave column w / NA (its 32 WB token rows). A slice of a tile is
// copied by 1 KiB DMA instructions of 16 rows each, IA (weight) and IB
// (token) per wave.
template <int WA, int WB, int NA, int NB>
struct BigTile {
  static constexpr int kWaves = NA * NB, kThreads = 64 * kWaves;
  static constexpr int TA = NA * 32 * WA, TB = NB * 32 * WB;
  static constexpr int IA = TA / kBigRowsPerDma / kWaves, IB = TB / kBigRowsPerDma / kWaves;
  static_assert(IA * kBigRowsPerDma * kWaves == TA && IB * kBigRowsPerDma * kWaves == TB,
                "every wave issues the same number of DMA instructions");
  static constexpr int kLds = kBigStages * (TA + TB) * kBigRowBytes;
};

// Main loop of the large-tile path: acc[x][y] (wave block x of the A tile,
// block y of the token tile) over K. For each of its DMA instructions (one
// per 16-row group: A groups wave, wave + NA NB, ..., then the token groups
// alike) the wave passes the source buffer and the byte offset at k = 0 of
// the lane's 16-byte chunk (row (wave + NA NB i) * 16 + lane / 4, chunk
// lane % 4 at slot chunk ^ big_swz(row)); kBigOob reads a zero row.
template <int WA, int WB, int NA, int NB>
__device__ __forceinline__ void big_mainloop(const u32x4 (&ra)[BigTile<WA, WB, NA, NB>::IA],
                                             const int (&offa)[BigTile<WA, WB, NA, NB>::IA], const u32x4& rx,
                                             const int (&offb)[BigTile<WA, WB, NA, NB>::IB], int K, char* lds,
                                             f32x16 (&acc)[WA][WB]) {
  using Tile = BigTile<WA, WB, NA, NB>;
  constexpr int TA = Tile::TA, IA = Tile::IA, IB = Tile::IB, NW = Tile::kWaves;
  constexpr int STAGE = (Tile::TA + Tile::TB) * kBigRowBytes;
  constexpr int KSTEPS = kBigBK / 16;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int wa = wave % NA, wb = wave / NA;
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  auto dma = [&](uint32_t lds_byte, const u32x4& rs, int off) __attribute__((always_inline)) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_byte), "v"(off), "s"(rs)
                 : "memory", "m0");
  };
  auto issue = [&](int sl) __attribute__((always_inline)) {  // slice sl into stage sl % kBigStages
    const uint32_t st = lds_base + (uint32_t)((sl % kBigStages) * STAGE);
    const int kb = sl * kBigRowBytes;
#pragma unroll
    for (int i = 0; i < IA; ++i) dma(st + (uint32_t)((wave + NW * i) * 1024), ra[i], offa[i] + kb);
#pragma unroll
    for (int i = 0; i < IB; ++i) dma(st + (uint32_t)(TA * kBigRowBytes + (wave + NW * i) * 1024), rx, offb[i] + kb);
  };
#pragma unroll
  for (int x = 0; x < WA; ++x)
#pragma unroll
    for (int y = 0; y < WB; ++y) acc[x][y] = f32x16{};
  const int nsl = K / kBigBK;
#pragma unroll
  for (int sl = 0; sl < kBigStages - 1; ++sl)
    if (sl < nsl) issue(sl);
  auto rd = [&](const char* base, int row, int c) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(base + row * kBigRowBytes + 16 * (c ^ big_swz(row)));
  };
  constexpr int kVm = (kBigStages - 2) * (IA + IB);  // this wave's DMA of the slices after the next
  static_assert(kVm < 64, "vmcnt immediate");
  for (int sl = 0; sl < nsl; ++sl) {
    // slice sl has landed for this wave (the kBigStages - 2 younger slices may
    // still fly), then for every wave; the barrier also retires the reads of
    // the stage the next issue overwrites
    if (sl + kBigStages - 2 < nsl)
      __builtin_amdgcn_s_waitcnt(big_wait_vm(kVm));
    else
      __builtin_amdgcn_s_waitcnt(big_wait_vm(0));
    __syncthreads();
    if (sl + kBigStages - 1 < nsl) issue(sl + kBigStages - 1);
    const char* st = lds + (sl % kBigStages) * STAGE;
    bf16x8 fa[KSTEPS][WA], fb[KSTEPS][WB];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int x = 0; x < WA; ++x) fa[ks][x] = rd(st, 32 * (WA * wa + x) + lrow, 2 * ks + lg);
#pragma unroll
      for (int y = 0; y < WB; ++y) fb[ks][y] = rd(st + TA * kBigRowBytes, 32 * (WB * wb + y) + lrow, 2 * ks + lg);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int x = 0; x < WA; ++x)
#pragma unroll
        for (int y = 0; y < WB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][x], fb[ks][y], acc[x][y], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, KSTEPS * (WA + WB), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, KSTEPS * WA * WB, 0);
  }
}

// Byte offset at k = 0 of this lane's chunk of token-tile DMA instruction i
// (of IB, in a work-group of NW waves): token row src[i] of x (kBigOob when
// src[i] < 0).
template <int IB, int NW>
__device__ __forceinline__ void big_token_offsets(int (&offb)[IB], int wave, int lane, int K,
                                                  const int (&src)[IB]) {
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int row = (wave + NW * i) * kBigRowsPerDma + lane / 4, slot = lane % 4;
    offb[i] = src[i] >= 0 ? (src[i] * K + 8 * (slot ^ big_swz(row))) * 2 : (int)kBigOob;
  }
}

// MODE kModeSwiglu: WA = 4, NA = 2; the A tile's 256 rows are gate rows
// f0 .. f0+63, up rows f0 .. f0+63, gate rows f0+64 .., up rows f0+64 ..
// (64-row groups), so wave row wa holds gate blocks 0, 1 and the matching up
// blocks 2, 3 of features f0 + 64 wa ... The work-group covers 128 features.
// OCC: work-groups per CU the launch bounds allow.
template <int MODE, int WA, int WB, int NA, int NB, int OCC>
__global__ __launch_bounds__(64 * NA * NB, OCC) void ffn_big_kernel(FfnArgs a, uint32_t a_bytes, uint32_t x_bytes) {
  using Tile = BigTile<WA, WB, NA, NB>;
  constexpr int TA = Tile::TA, TB = Tile::TB, IA = Tile::IA, IB = Tile::IB, NW = Tile::kWaves;
  static_assert(MODE != kModeSwiglu || (WA == 4 && NA == 2), "SwiGLU tile pairs gate and up blocks");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int wa = wave % NA, wb = wave / NA;
  const int f0 = blockIdx.x * (MODE == kModeSwiglu ? 128 : TA);  // first output feature
  const int m0 = blockIdx.y * TB;                                 // first token row
  u32x4 ra[IA];
  int offa[IA], offb[IB], srcb[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int r0 = (wave + NW * i) * kBigRowsPerDma, row = r0 + lane / 4, slot = lane % 4;
    int src;  // weight row of stage row `row`
    if (MODE == kModeSwiglu) {
      const int grp = r0 / 64;  // 0: gate, 1: up, 2: gate + 64, 3: up + 64 (uniform per instruction)
      ra[i] = big_rsrc((grp & 1) ? a.a1 : a.a0, a_bytes);
      src = f0 + 64 * (grp >> 1) + (row - 64 * grp);
    } else {
      ra[i] = big_rsrc(a.a0, a_bytes);
      src = f0 + row;
    }
    offa[i] = (src * a.K + 8 * (slot ^ big_swz(row))) * 2;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int m = m0 + (wave + NW * i) * kBigRowsPerDma + lane / 4;
    const int src = m < a.k_tokens ? (MODE == kModeSwiglu ? a.idx[m] : m) : -1;
    srcb[i] = src >= 0 && (MODE != kModeSwiglu || src < a.n_rows) ? src : -1;
  }
  big_token_offsets<IB, NW>(offb, wave, lane, a.K, srcb);
  f32x16 acc[WA][WB];
  big_mainloop<WA, WB, NA, NB>(ra, offa, big_rsrc(a.x, x_bytes), offb, a.K, lds, acc);

  // lane holds token row m0 + 32 (WB wb + y) + lrow and features 8 (i/4) + 4 lg + i%4 of each block
#pragma unroll
  for (int y = 0; y < WB; ++y) {
    const int m = m0 + 32 * (WB * wb + y) + lrow;
    if (m >= a.k_tokens) continue;
    if (MODE == kModeSwiglu) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        uint16_t* orow = a.out + (size_t)m * a.out_ld + f0 + 64 * wa + 32 * x;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint32_t w[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            uint32_t pk = 0;
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
              const int i = 4 * g4 + 2 * e + hl;
              const float g = acc[x][y][i], u = acc[x + 2][y][i];
              const float act = g / (1.f + __expf(-g)) * u;
              pk |= (uint32_t)float_to_bf16_bits(act) << (16 * hl);
            }
            w[e] = pk;
          }
          *reinterpret_cast<u32x2*>(orow + 8 * g4 + 4 * lg) = u32x2{w[0], w[1]};
        }
      }
    } else {
      const int dst = a.idx ? a.idx[m] : m;  // no index list: row m itself
      if (dst < 0 || dst >= a.n_rows) continue;  // out-of-range index: row skipped
#pragma unroll
      for (int x = 0; x < WA; ++x) {
        uint16_t* orow = a.out + (size_t)dst * a.out_ld + f0 + 32 * (WA * wa + x);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint16_t* p = orow + 8 * g4 + 4 * lg;
          const u32x2 old = *reinterpret_cast<const u32x2*>(p);
          uint32_t w[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            uint32_t pk = 0;
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
              const int i = 4 * g4 + 2 * e + hl;
              const float h = bf16_bits_to_float((uint16_t)(old[e] >> (16 * hl)));
              pk |= (uint32_t)float_to_bf16_bits(h + acc[x][y][i]) << (16 * hl);
            }
            w[e] = pk;
          }
          *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
        }
      }
    }
  }
}

// Dynamic LDS above the default limit, allowed once per kernel and device
// (false: the caller takes its fallback kernel).
template <auto* KERNEL>
bool big_lds_attr(int bytes) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static signed char state[kDevices] = {};  // 0: not yet set, 1: set, -1: refused
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) {
    (void)hipGetLastError();
    return false;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (state[dev] == 0) {
    state[dev] = hipFuncSetAttribute((const void*)KERNEL, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess
                     ? 1
                     : -1;
    if (state[dev] < 0) (void)hipGetLastError();
  }
  return state[dev] > 0;
}

// The 8-wave large-tile path of the sparse FFN (SwiGLU: 256 weight rows =
// 128 features x 256 token rows, 128 x 64 per wave; down projection: 128
// features x 256 token rows, 64 x 64 per wave), when the launch has at least
// one work-group per CU and every buffer fits the 32-bit offsets of a buffer
// load; returns false to let the caller take another kernel.
template <int MODE>
bool launch_ffn_big(const FfnArgs& g, int n_features, int rows, size_t a_bytes, size_t x_bytes, hipStream_t s) {
  constexpr int WA = MODE == kModeSwiglu ? 4 : 2, WB = 2, NA = 2, NB = 4;
  using Tile = BigTile<WA, WB, NA, NB>;
  constexpr int FEAT = MODE == kModeSwiglu ? 128 : Tile::TA;
  if (g.K % kBigBK != 0 || n_features % FEAT != 0) return false;
  if (a_bytes >= (size_t)INT_MAX || x_bytes >= (size_t)INT_MAX) return false;
  const dim3 grid(n_features / FEAT, cdiv(rows, Tile::TB));
  if ((int64_t)grid.x * grid.y < 256) return false;
  if (!big_lds_attr<ffn_big_kernel<MODE, WA, WB, NA, NB, 1>>(Tile::kLds)) return false;
  ffn_big_kernel<MODE, WA, WB, NA, NB, 1><<<grid, Tile::kThreads, Tile::kLds, s>>>(g, (uint32_t)a_bytes,
                                                                                   (uint32_t)x_bytes);
  return true;
}

// ---- layer glue: fused QKV projection + RoPE + append of the query rows' K/V ----
//
// paooo.com "如何使用RedKnot" (EXECUTE recomputes the query segment) and RedKnot
// README "About" (the query segment's KV is produced online into the per-head
// paged store). Q, K and V of a query row come from one GEMM against the
// stacked weights [Hq | Hkv | Hkv heads][D rows]; Q and K are rotated at the
// row's position (rotate-half pairing of dims j and j + D/2, omega_j =
// theta^(-2j/D)) in the epilogue, which also writes K and V straight into the
// query segment's working pages. The wave's two weight blocks are chosen so a
// lane holds both halves of a pair: blocks (32 wn, 64 + 32 wn) of a one-head
// tile for D = 128, blocks (64 wn, 64 wn + 32) = one head per wave for D = 64.

constexpr int kRowThreads = 64;

struct QkvRowArgs {
  const int32_t* cu_q;
  const int32_t* seg_indptr;
  const int32_t* seg_start;
  const int32_t* seg_page_indptr;
  const int32_t* seg_pages;
  float2* rope_cs;     // [T][D/2] (cos, sin) of row t's angle for pair j
  int32_t* row_slot;   // [T][Hkv] page * P + slot of row t's K/V for kv head h, or -1
  int R, T, Hkv, D;
  int64_t pool_pages;
  double log2_theta;  // log2 of the RoPE base, taken on the host
};

// One work-group per query row: its request (largest r with cu_q[r] <= t), its
// position, the cos/sin of its angles (fp64 sincos, rounded to fp32) and the
// page slot its K/V go to for each kv head.
__global__ __launch_bounds__(kRowThreads) void qkv_rows_kernel(QkvRowArgs a) {
  const int t = blockIdx.x, tid = threadIdx.x;
  int lo = 0, hi = a.R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int r = lo, sq = a.seg_indptr[r + 1] - 1, tl = t - a.cu_q[r];
  const int pos = a.seg_start[sq] + tl;
  for (int j = tid; j < a.D / 2; j += kRowThreads) {
    const double w = exp2(-2.0 * (double)j / (double)a.D * a.log2_theta);  // theta^(-2j/D)
    double sn, cn;
    sincos((double)pos * w, &sn, &cn);
    a.rope_cs[(size_t)t * (a.D / 2) + j] = make_float2((float)cn, (float)sn);
  }
  for (int h = tid; h < a.Hkv; h += kRowThreads) {
    const int e = a.seg_page_indptr[sq * a.Hkv + h] + tl / kPage;
    int slot = -1;
    if (e < a.seg_page_indptr[sq * a.Hkv + h + 1]) {
      const int page = a.seg_pages[e];
      if (page >= 0 && page < a.pool_pages) slot = page * kPage + tl % kPage;
    }
    a.row_slot[(size_t)t * a.Hkv + h] = slot;
  }
}

struct QkvArgs {
  const uint16_t* w;        // [(Hq + 2 Hkv) D][K]
  const uint16_t* x;        // [T][K]
  const float2* rope_cs;
  const int32_t* row_slot;
  uint16_t* q_out;          // [T][Hq][D]
  uint16_t* k_pool;         // [pages][P][D]
  uint16_t* v_pool;         // [pages][D][P]
  int T, K, Hq, Hkv, D;
};

template <int NB>
__global__ __launch_bounds__(kFfnThreads, 2) void qkv_rope_append_kernel(QkvArgs a) {
  __shared__ uint16_t sa[kRowsA * kLdsStride];
  __shared__ uint16_t sb[kRowsB * kLdsStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * kRowsA, m0 = blockIdx.y * 64 * NB;
  const int nfeat = (a.Hq + 2 * a.Hkv) * a.D;
  const uint16_t* arow[4];
  const uint16_t* brow[2 * NB];
  int lds_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int qd = tid + u * kFfnThreads;
    const int row = qd >> 3, c = qd & 7;
    lds_off[u] = row * kLdsStride + 8 * c;
    const int nrow = n0 + row < nfeat ? n0 + row : nfeat - 1;  // a half tile past the last head (D = 64)
    arow[u] = a.w + (size_t)nrow * a.K + 8 * c;
    if (u < 2 * NB) brow[u] = m0 + row < a.T ? a.x + (size_t)(m0 + row) * a.K + 8 * c : nullptr;
  }
  const int arow0 = a.D == 128 ? 32 * wn : 64 * wn;
  const int arow1 = a.D == 128 ? 64 + 32 * wn : 64 * wn + 32;
  f32x16 acc[2][NB];
  gemm_tile<NB>(arow, brow, lds_off, a.K, arow0, arow1, wm, sa, sb, acc);

  // acc[0][mb][i] and acc[1][mb][i]: dims j and j + D/2 of head `head`, token row m,
  // with j = j0 + 8 (i/4) + 4 lg + i%4
  const int head = (n0 + arow0) / a.D, j0 = (n0 + arow0) % a.D, half = a.D / 2;
  if (head >= a.Hq + 2 * a.Hkv) return;  // the unused half of the last tile
  const int kind = head < a.Hq ? 0 : head < a.Hq + a.Hkv ? 1 : 2;  // Q, K, V
  const int hk = kind == 1 ? head - a.Hq : head - a.Hq - a.Hkv;
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    const int m = m0 + 32 * NB * wm + 32 * mb + lrow;
    if (m >= a.T) continue;
    const int slot = kind == 0 ? 0 : a.row_slot[(size_t)m * a.Hkv + hk];
    if (slot < 0) continue;  // no page for this row: nothing written
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int j = j0 + 8 * g4 + 4 * lg;
      float lo4[4], hi4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = acc[0][mb][4 * g4 + e], y = acc[1][mb][4 * g4 + e];
        if (kind == 2) {
          lo4[e] = x;
          hi4[e] = y;
        } else {
          const float2 cs = a.rope_cs[(size_t)m * half + j + e];
          lo4[e] = x * cs.x - y * cs.y;
          hi4[e] = x * cs.y + y * cs.x;
        }
      }
      if (kind == 2) {  // d-major page: element (d, slot) at d * P + slot
        uint16_t* vp = a.v_pool + (size_t)(slot / kPage) * a.D * kPage + slot % kPage;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vp[(size_t)(j + e) * kPage] = float_to_bf16_bits(lo4[e]);
          vp[(size_t)(j + e + half) * kPage] = float_to_bf16_bits(hi4[e]);
        }
      } else {
        uint16_t* dst = kind == 0 ? a.q_out + ((size_t)m * a.Hq + head) * a.D : a.k_pool + (size_t)slot * a.D;
        const u32x2 wl = {(uint32_t)float_to_bf16_bits(lo4[0]) | (uint32_t)float_to_bf16_bits(lo4[1]) << 16,
                          (uint32_t)float_to_bf16_bits(lo4[2]) | (uint32_t)float_to_bf16_bits(lo4[3]) << 16};
        const u32x2 wh = {(uint32_t)float_to_bf16_bits(hi4[0]) | (uint32_t)float_to_bf16_bits(hi4[1]) << 16,
                          (uint32_t)float_to_bf16_bits(hi4[2]) | (uint32_t)float_to_bf16_bits(hi4[3]) << 16};
        *reinterpret_cast<u32x2*>(dst + j) = wl;
        *reinterpret_cast<u32x2*>(dst + j + half) = wh;
      }
    }
  }
}

// The QKV projection on the large-tile main loop: 128 weight rows x 64 WB
// token rows per work-group (OCC per CU). The A tile is one head (D = 128)
// or two (D = 64). For D = 128 its middle two 32-row blocks are swapped in
// LDS (stage blocks 0..3 = dims 0-31, 64-95, 32-63, 96-127), so that each
// wave's two blocks are dims j0 .. j0 + 31 and j0 + 64 ..: the rotate-half
// pairs, as in qkv_rope_append_kernel, whose epilogue this one repeats.
template <int WB, int OCC>
__global__ __launch_bounds__(kFfnThreads, OCC) void qkv_big_kernel(QkvArgs a, uint32_t w_bytes, uint32_t x_bytes) {
  constexpr int WA = 2, TB = 64 * WB;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int wa = wave & 1, wb = wave >> 1;
  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * TB;
  const int nfeat = (a.Hq + 2 * a.Hkv) * a.D;
  u32x4 ra[WA];
  int offa[WA], offb[WB], srcb[WB];
#pragma unroll
  for (int i = 0; i < WA; ++i) {
    const int row = (wave + 4 * i) * kBigRowsPerDma + lane / 4, slot = lane % 4;
    const int blk = row / 32, sb = a.D == 128 && (blk == 1 || blk == 2) ? 3 - blk : blk;
    const int f = n0 + 32 * sb + row % 32;  // weight row (feature) of stage row `row`
    ra[i] = big_rsrc(a.w, w_bytes);
    offa[i] = f < nfeat ? (f * a.K + 8 * (slot ^ big_swz(row))) * 2 : (int)kBigOob;
  }
#pragma unroll
  for (int i = 0; i < WB; ++i) {
    const int m = m0 + (wave + 4 * i) * kBigRowsPerDma + lane / 4;
    srcb[i] = m < a.T ? m : -1;
  }
  big_token_offsets<WB, 4>(offb, wave, lane, a.K, srcb);

  // acc[0][y][i] and acc[1][y][i]: dims j and j + D/2 of head `head`, token
  // row m = m0 + 32 (WB wb + y) + lrow, with j = j0 + 8 (i/4) + 4 lg + i%4.
  // The epilogue's page slots and (cos, sin) pairs are loaded before the
  // main loop, so they do not add a memory round trip at its end.
  const int head = (n0 + 64 * wa) / a.D, j0 = a.D == 128 ? 32 * wa : 0, half = a.D / 2;
  const bool head_ok = head < a.Hq + 2 * a.Hkv;  // false: the unused half of the last tile
  const int kind = head < a.Hq ? 0 : head < a.Hq + a.Hkv ? 1 : 2;  // Q, K, V
  const int hk = kind == 1 ? head - a.Hq : head - a.Hq - a.Hkv;
  int slot[WB];
  float4 cs[WB][4][2];  // (cos, sin) of pairs j .. j + 3 per g4: two 16-byte loads (j is a multiple of 4)
#pragma unroll
  for (int y = 0; y < WB; ++y) {
    const int m = m0 + 32 * (WB * wb + y) + lrow;
    const bool row_ok = head_ok && m < a.T;
    slot[y] = row_ok && kind != 0 ? a.row_slot[(size_t)m * a.Hkv + hk] : 0;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      cs[y][g4][0] = cs[y][g4][1] = float4{0.f, 0.f, 0.f, 0.f};
      if (row_ok && kind != 2) {
        const float4* cp = reinterpret_cast<const float4*>(a.rope_cs + (size_t)m * half + j0 + 8 * g4 + 4 * lg);
        cs[y][g4][0] = cp[0];
        cs[y][g4][1] = cp[1];
      }
    }
  }
  f32x16 acc[WA][WB];
  big_mainloop<WA, WB, 2, 2>(ra, offa, big_rsrc(a.x, x_bytes), offb, a.K, lds, acc);

  if (!head_ok) return;
#pragma unroll
  for (int y = 0; y < WB; ++y) {
    const int m = m0 + 32 * (WB * wb + y) + lrow;
    if (m >= a.T || slot[y] < 0) continue;  // no page for this row: nothing written
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int j = j0 + 8 * g4 + 4 * lg;
      float lo4[4], hi4[4];
      const float4 (&cs4)[2] = cs[y][g4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = acc[0][y][4 * g4 + e], yv = acc[1][y][4 * g4 + e];
        if (kind == 2) {
          lo4[e] = x;
          hi4[e] = yv;
        } else {
          const float4 c = cs4[e >> 1];
          const float cx = (e & 1) ? c.z : c.x, sy = (e & 1) ? c.w : c.y;
          lo4[e] = x * cx - yv * sy;
          hi4[e] = x * sy + yv * cx;
        }
      }
      if (kind == 2) {  // d-major page: element (d, slot) at d * P + slot
        uint16_t* vp = a.v_pool + (size_t)(slot[y] / kPage) * a.D * kPage + slot[y] % kPage;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vp[(size_t)(j + e) * kPage] = float_to_bf16_bits(lo4[e]);
          vp[(size_t)(j + e + half) * kPage] = float_to_bf16_bits(hi4[e]);
        }
      } else {
        uint16_t* dst = kind == 0 ? a.q_out + ((size_t)m * a.Hq + head) * a.D : a.k_pool + (size_t)slot[y] * a.D;
        const u32x2 wl = {(uint32_t)float_to_bf16_bits(lo4[0]) | (uint32_t)float_to_bf16_bits(lo4[1]) << 16,
                          (uint32_t)float_to_bf16_bits(lo4[2]) | (uint32_t)float_to_bf16_bits(lo4[3]) << 16};
        const u32x2 wh = {(uint32_t)float_to_bf16_bits(hi4[0]) | (uint32_t)float_to_bf16_bits(hi4[1]) << 16,
                          (uint32_t)float_to_bf16_bits(hi4[2]) | (uint32_t)float_to_bf16_bits(hi4[3]) << 16};
        *reinterpret_cast<u32x2*>(dst + j) = wl;
        *reinterpret_cast<u32x2*>(dst + j + half) = wh;
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
  uint16_t* act = static_cast<uint16_t*>(workspace);  // the activation [k][inter]
  FfnArgs g1;
  g1.a0 = static_cast<const uint16_t*>(w_gate);
  g1.a1 = static_cast<const uint16_t*>(w_up);
  g1.x = static_cast<const uint16_t*>(hidden);
  g1.out = act;
  g1.idx = idx_dev;
  g1.k_tokens = k;
  g1.K = hidden_size;
  g1.out_ld = inter;
  g1.n_rows = n_rows;
  if (launch_ffn_big<kModeSwiglu>(g1, inter, k, (size_t)inter * hidden_size * 2, (size_t)n_rows * hidden_size * 2, s))
    ;
  else if (small_grid(inter / 64, k))
    ffn_gemm_kernel<kModeSwiglu, 1><<<dim3(inter / 64, cdiv(k, 64)), kFfnThreads, 0, s>>>(g1);
  else
    ffn_gemm_kernel<kModeSwiglu, 2><<<dim3(inter / 64, cdiv(k, kRowsB)), kFfnThreads, 0, s>>>(g1);
  SEGKV_LAUNCH_CHECK();
  FfnArgs g2;
  g2.a0 = static_cast<const uint16_t*>(w_down);
  g2.a1 = nullptr;
  g2.x = act;
  g2.out = static_cast<uint16_t*>(hidden);
  g2.idx = idx_dev;
  g2.k_tokens = k;
  g2.K = inter;
  g2.out_ld = hidden_size;
  g2.n_rows = n_rows;
  const size_t w2_bytes = (size_t)hidden_size * inter * 2, x2_bytes = (size_t)k * inter * 2;
  constexpr int kResLds = BigTile<2, 1, 2, 2>::kLds;
  if (launch_ffn_big<kModeResidual>(g2, hidden_size, k, w2_bytes, x2_bytes, s))
    ;
  else if (w2_bytes < (size_t)INT_MAX && x2_bytes < (size_t)INT_MAX &&
           big_lds_attr<ffn_big_kernel<kModeResidual, 2, 1, 2, 2, 2>>(kResLds))  // fewer rows: 128 x 64, 2 per CU
    ffn_big_kernel<kModeResidual, 2, 1, 2, 2, 2><<<dim3(hidden_size / 128, cdiv(k, 64)), kFfnThreads, kResLds, s>>>(
        g2, (uint32_t)w2_bytes, (uint32_t)x2_bytes);
  else if (small_grid(hidden_size / kRowsA, k))
    ffn_gemm_kernel<kModeResidual, 1><<<dim3(hidden_size / kRowsA, cdiv(k, 64)), kFfnThreads, 0, s>>>(g2);
  else
    ffn_gemm_kernel<kModeResidual, 2><<<dim3(hidden_size / kRowsA, cdiv(k, kRowsB)), kFfnThreads, 0, s>>>(g2);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}

namespace {
size_t qkv_ws_bytes(int64_t T, int Hkv, int D) {
  const size_t cs = ((size_t)T * (D / 2) * sizeof(float2) + 255) & ~(size_t)255;
  return cs + (size_t)T * Hkv * sizeof(int32_t);
}
}  // namespace

extern "C" int32_t segkv_qkv_workspace_size(const segkv_dims* dims, const segkv_meta* meta_host, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(SEGKV_ERR_INVALID_ARG, "bytes is NULL");
  const int32_t st = validate_layout(dims, meta_host);
  if (st != SEGKV_OK) return st;
  int64_t T = 0;
  for (int r = 0; r < dims->num_requests; ++r) T += meta_host->seg_len[meta_host->seg_indptr[r + 1] - 1];
  *bytes = qkv_ws_bytes(T, dims->num_kv_heads, dims->head_dim);
  return SEGKV_OK;
}

extern "C" int32_t segkv_qkv_rope_append(const segkv_dims* dims, const segkv_meta* meta_host,
                                         const segkv_meta* meta_dev, const int32_t* cu_q_dev,
                                         const int32_t* seg_page_indptr_dev, const int32_t* seg_pages_dev,
                                         int64_t pool_pages, const void* hidden, int32_t hidden_size,
                                         const void* w_qkv, double rope_theta, void* q_out, void* k_pool,
                                         void* v_pool, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const int32_t st = validate_layout(dims, meta_host);
  if (st != SEGKV_OK) return st;
  const int R = dims->num_requests, Hq = dims->num_q_heads, Hkv = dims->num_kv_heads, D = dims->head_dim;
  if (!meta_dev || !cu_q_dev || !seg_page_indptr_dev || !seg_pages_dev || !hidden || !w_qkv || !q_out ||
      !k_pool || !v_pool || !workspace)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (hidden_size <= 0 || hidden_size % kBK != 0)
    return fail(SEGKV_ERR_UNSUPPORTED, "hidden_size must be a positive multiple of 64");
  if (!(rope_theta > 0.0)) return fail(SEGKV_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (pool_pages <= 0 || pool_pages > INT32_MAX / kPage)
    return fail(SEGKV_ERR_INVALID_ARG, "pool_pages must be in 1 .. 2^31 / page_size");
  int64_t T = 0;
  for (int r = 0; r < R; ++r) T += meta_host->seg_len[meta_host->seg_indptr[r + 1] - 1];
  if (T > INT32_MAX / 2) return fail(SEGKV_ERR_UNSUPPORTED, "too many query rows");
  if (workspace_bytes < qkv_ws_bytes(T, Hkv, D))
    return fail(SEGKV_ERR_WORKSPACE, "workspace smaller than segkv_qkv_workspace_size");
  if (!aligned16(hidden) || !aligned16(w_qkv) || !aligned16(q_out) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(workspace))
    return fail(SEGKV_ERR_ALIGNMENT, "tensors must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  QkvRowArgs ra;
  ra.cu_q = cu_q_dev;
  ra.seg_indptr = meta_dev->seg_indptr;
  ra.seg_start = meta_dev->seg_start;
  ra.seg_page_indptr = seg_page_indptr_dev;
  ra.seg_pages = seg_pages_dev;
  ra.rope_cs = static_cast<float2*>(workspace);
  ra.row_slot = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                           (((size_t)T * (D / 2) * sizeof(float2) + 255) & ~(size_t)255));
  ra.R = R;
  ra.T = (int)T;
  ra.Hkv = Hkv;
  ra.D = D;
  ra.pool_pages = pool_pages;
  ra.log2_theta = std::log2(rope_theta);
  qkv_rows_kernel<<<(unsigned)T, kRowThreads, 0, s>>>(ra);
  SEGKV_LAUNCH_CHECK();
  QkvArgs a;
  a.w = static_cast<const uint16_t*>(w_qkv);
  a.x = static_cast<const uint16_t*>(hidden);
  a.rope_cs = ra.rope_cs;
  a.row_slot = ra.row_slot;
  a.q_out = static_cast<uint16_t*>(q_out);
  a.k_pool = static_cast<uint16_t*>(k_pool);
  a.v_pool = static_cast<uint16_t*>(v_pool);
  a.T = (int)T;
  a.K = hidden_size;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  const int nx = cdiv((Hq + 2 * Hkv) * D, kRowsA);
  const size_t w_bytes = (size_t)(Hq + 2 * Hkv) * D * hidden_size * 2, x_bytes = (size_t)T * hidden_size * 2;
  constexpr int kQkvWB = 2, kQkvLds = BigTile<2, kQkvWB, 2, 2>::kLds;
  if (hidden_size % kBigBK == 0 && w_bytes < (size_t)INT_MAX && x_bytes < (size_t)INT_MAX &&
      big_lds_attr<qkv_big_kernel<kQkvWB, 2>>(kQkvLds))
    qkv_big_kernel<kQkvWB, 2><<<dim3(nx, cdiv((int)T, 64 * kQkvWB)), kFfnThreads, kQkvLds, s>>>(
        a, (uint32_t)w_bytes, (uint32_t)x_bytes);
  else if (small_grid(nx, (int)T))
    qkv_rope_append_kernel<1><<<dim3(nx, cdiv((int)T, 64)), kFfnThreads, 0, s>>>(a);
  else
    qkv_rope_append_kernel<2><<<dim3(nx, cdiv((int)T, kRowsB)), kFfnThreads, 0, s>>>(a);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}

extern "C" int32_t segkv_out_proj_residual(const void* attn, int32_t n_rows, int32_t in_features, const void* w_o,
                                           void* hidden, int32_t hidden_size, void* stream) {
  clear_error();
  if (n_rows < 0 || in_features <= 0 || hidden_size <= 0)
    return fail(SEGKV_ERR_INVALID_ARG, "need n_rows >= 0, in_features > 0 and hidden_size > 0");
  if (in_features % kBK != 0 || hidden_size % kRowsA != 0)
    return fail(SEGKV_ERR_UNSUPPORTED, "in_features must be a multiple of 64 and hidden_size of 128");
  if (n_rows == 0) return SEGKV_OK;
  if (!attn || !w_o || !hidden) return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(attn) || !aligned16(w_o) || !aligned16(hidden))
    return fail(SEGKV_ERR_ALIGNMENT, "tensors must be 16-byte aligned");
  FfnArgs g;
  g.a0 = static_cast<const uint16_t*>(w_o);
  g.a1 = nullptr;
  g.x = static_cast<const uint16_t*>(attn);
  g.out = static_cast<uint16_t*>(hidden);
  g.idx = nullptr;
  g.k_tokens = n_rows;
  g.K = in_features;
  g.out_ld = hidden_size;
  g.n_rows = n_rows;
  const int nx = hidden_size / kRowsA;
  // large-tile main loop, 128 x 64 tiles, two work-groups per CU (the same
  // tile as the 64-row-token form of ffn_gemm_kernel, which stays for
  // operands beyond 32-bit buffer offsets)
  const size_t w_bytes = (size_t)hidden_size * in_features * 2, x_bytes = (size_t)n_rows * in_features * 2;
  constexpr int kOpLds = BigTile<2, 1, 2, 2>::kLds;
  if (w_bytes < (size_t)INT_MAX && x_bytes < (size_t)INT_MAX &&
      big_lds_attr<ffn_big_kernel<kModeResidual, 2, 1, 2, 2, 2>>(kOpLds))
    ffn_big_kernel<kModeResidual, 2, 1, 2, 2, 2><<<dim3(nx, cdiv(n_rows, 64)), kFfnThreads, kOpLds,
                                                   hipStream_t(stream)>>>(g, (uint32_t)w_bytes, (uint32_t)x_bytes);
  else if (small_grid(nx, n_rows))
    ffn_gemm_kernel<kModeResidual, 1><<<dim3(nx, cdiv(n_rows, 64)), kFfnThreads, 0, hipStream_t(stream)>>>(g);
  else
    ffn_gemm_kernel<kModeResidual, 2><<<dim3(nx, cdiv(n_rows, kRowsB)), kFfnThreads, 0, hipStream_t(stream)>>>(g);
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}
