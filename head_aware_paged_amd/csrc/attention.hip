// EXECUTE attention: SegPagedAttention prefill for the recomputed segment.
//
// paooo.com "RedKnot的技术原理": KV lives in per-head pages and a fused varlen
// kernel reads it without ever building an attention mask; "如何使用RedKnot":
// global heads attend over the full range, local heads over reused paged KV;
// RedKnot README "About": every head class has its own visible window over a
// per-head page table.
//
// Work decomposition. A work-group (4 waves) owns one m-tile: the G query heads
// of one kv head times 128/G consecutive query positions (128 rows), so every
// K/V page staged in LDS serves all G heads of the group. The m-tile's visible
// table entries are walked in tiles of 4 pages (64 keys); long ranges are split
// into chunks whose partial (m, l, O) are merged by a second kernel. Items run
// in an XCD-aware order: the m-tiles that read the same key chunk are launched
// on one XCD, so the chunk's pages come from HBM once into that XCD's L2.
//
// Per wave (32 rows) and tile, with the gfx950 32x32x16 bf16 MFMA:
//   S^T[key][row] = K[key][:] . Q[row][:]     (A = K from LDS, B = Q in VGPRs)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row] (A = V^T from LDS, B = P in VGPRs)
// The S^T layout puts one query row in each lane (two lanes per row), so row
// max / sum stay in-lane, and the P fragment produced by the first MFMA is the
// B operand of the second with no shuffle: K rows are fed to the first MFMA in
// a permuted order chosen so each lane ends up holding 8 consecutive keys.
// Visibility is a per-element predicate evaluated only on tiles that straddle
// a window edge; other tiles take no mask work at all.
#include <type_traits>

#include "common.h"

namespace segkv {
namespace {

constexpr int kAttnThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // lazy rescale: p <= 2^8 between rescales
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]):
// wait for vector memory down to 0 / 1 outstanding, leave the other counters alone
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm1 = 0x0F71;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int64_t pool_pages;
  const int32_t* page_ids;
  const int32_t* page_pos;
  const char* plan;
  PlanLayout L;
  uint16_t* out;
  float* lse;
  char* partials;      // split-KV workspace, partial_slot_bytes(D) per chunk
  float scale_log2;  // softmax_scale * log2(e)
  int Hq, G;
};

// Key (within a 32-key block) whose K row the lane feeding MFMA row `slot`
// loads, so that output register i of lane group g holds key 8g+i (i < 8) or
// 16+8g+(i-8) (i >= 8).
__device__ __forceinline__ int slot_key(int slot) {
  const int a = slot >> 3, g = (slot >> 2) & 1, b = slot & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

constexpr int kMaxItemEntries = kTilePages * kMaxChunkTiles;  // table entries of one item

// LDS of one work-group: two stages of K and V tiles in natural [key][d]
// layout, whose 16-byte chunks are XOR-swizzled per row so that both operand
// reads below are free of bank conflicts, plus the item's page table. Every
// stage is its own __shared__ object and the loop is unrolled by the stage
// index, so the compiler can tell that reads of one stage do not alias the
// asynchronous copies into the other and does not wait on those copies.
template <int D>
struct StageBufs {
  uint16_t* k;
  uint16_t* v;
};

// (host+device so the device lambdas below may call them)
template <int D>
SEGKV_HD int k_swz(int row) { return row % (D / 8); }        // S^T reads: 16 rows, one chunk
template <int D>
SEGKV_HD int v_swz(int row) { return (2 * row) % (D / 8); }  // transpose reads: 4 rows, 2 chunks

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16 (the builtin exists only in the device compilation pass)
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
#else
  (void)p;
  return bf16x4{};
#endif
}

SEGKV_HD int sel4(int i, int a, int b, int c, int d) {
  return i == 0 ? a : i == 1 ? b : i == 2 ? c : d;
}

// Per item, key tiles t of [t_lo, t_hi) with double-buffered LDS and one
// barrier per tile: iteration t computes S(t) = K(t) Q^T, the softmax, and
// O += V(t)^T P(t) from buffer t%2 while K(t+1) and V(t+1) stream straight
// into the other buffer (global_load_lds, 1 KiB per wave instruction). Two
// work-groups share a CU, so one wave's softmax overlaps the other's matrix
// instructions on each SIMD. V^T operands come from LDS transpose reads
// (ds_read_b64_tr_b16): a 16-lane group whose lanes point at 8-byte runs of 4
// rows x 16 columns receives the 4-row column slices, so with V kept as
// [key][d] each lane gets 4 consecutive keys of its own d.
template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_main_kernel(AttnArgs a) {
  constexpr int KS = D / 16;            // MFMA k-steps over the head dim
  constexpr int DB = D / 32;            // 32-wide d blocks of O^T
  constexpr int KCH = D / 8;            // 16-byte chunks per row
  constexpr int RPK = 1024 / (2 * D);   // rows per 1 KiB wave transfer
  constexpr int KLOADS = kTileKeys * KCH / kAttnThreads;  // 1 KiB transfers per wave per tensor
  __shared__ __attribute__((aligned(1024))) uint16_t sk0[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sk1[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv0[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv1[kTileKeys * D];
  __shared__ int spid[kMaxItemEntries];
  __shared__ int spos[kMaxItemEntries];
  __shared__ uint32_t swarm[kAttnThreads];  // sink of the L2 warm-up loads

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const MTile* mts = reinterpret_cast<const MTile*>(a.plan + a.L.mtiles_off);
  const Item* items = reinterpret_cast<const Item*>(a.plan + a.L.items_off);
  if ((int)blockIdx.x >= hdr->n_items) return;
  const Item it = items[blockIdx.x];
  if (it.mtile < 0) return;  // empty slot of the XCD-aware order
  const MTile mt = mts[it.mtile];
  const int t_lo = chunk_tile_lo(mt.n_tiles, mt.n_chunks, it.chunk);
  const int t_hi = chunk_tile_lo(mt.n_tiles, mt.n_chunks, it.chunk + 1);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int MP = kMRows / a.G;
  const int rm = wave * 32 + lrow;               // row within the m-tile
  const int hg = rm / MP, p = rm % MP;
  const bool row_valid = p < mt.n_pos;
  const int pc = row_valid ? p : mt.n_pos - 1;    // padding rows mirror the last valid row
  const int qhead = mt.h * a.G + hg;
  const int qrow = mt.q_row0 + pc;
  const int pos = mt.pos0 + pc;
  const bool is_local = mt.cls == kClassLocal;
  const int lo_row = is_local ? local_lo(pos, mt.bq, mt.W) : 0;
  const int pos_min = mt.pos0, pos_max = mt.pos0 + mt.n_pos - 1;
  const int lo_max = is_local ? local_lo(pos_max, mt.bq, mt.W) : 0;

  // the item's page table -> LDS (entries past the m-tile's end, or with an
  // invalid page id, become pid -1 / pos INT_MAX)
  const int e_lo = mt.e_begin + kTilePages * t_lo;
  const int n_ent = kTilePages * (t_hi - t_lo);
  for (int x = tid; x < n_ent; x += kAttnThreads) {
    const int e = e_lo + x;
    int pid = -1, ps = INT_MAX;
    if (e < mt.e_end) {
      pid = a.page_ids[e];
      ps = a.page_pos[e];
      if (pid < 0 || pid >= a.pool_pages) {
        pid = -1;
        ps = INT_MAX;
      }
    }
    spid[x] = pid;
    spos[x] = ps;
  }

  // Q fragments (B operand): Q[row][16 ks + 8 lg + 0..7]
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + ((size_t)qrow * a.Hq + qhead) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
  }
  __syncthreads();

  // DMA of tile t into a stage: wave w moves rows [16 w, 16 w + 16) = page w
  // of the tile, so the page id is wave-uniform. A missing page reads page 0:
  // its keys are masked by position and its V rows are zeroed before use.
  // (per-lane element offsets inside the page are fixed: computed once)
  int koff[KLOADS], voff[KLOADS];
#pragma unroll
  for (int u = 0; u < KLOADS; ++u) {
    const int row = (wave * KLOADS + u) * RPK + lane / KCH;
    const int ph = lane % KCH;
    koff[u] = (row & 15) * D + 8 * (ph ^ k_swz<D>(row));
    voff[u] = (row & 15) * D + 8 * (ph ^ v_swz<D>(row));
  }
  // The copy of a tile is issued in KLOADS parts spread over the previous
  // tile's body, so no wave stalls on a burst of vector memory instructions.
  auto dma_part = [&](uint16_t* kdst, uint16_t* vdst, const uint16_t* kpage, const uint16_t* vpage, int u) {
    const int blk = wave * KLOADS + u;
    const uint16_t* ksrc = kpage + koff[u];
    const uint16_t* vsrc = vpage + voff[u];
    __builtin_amdgcn_global_load_lds(ksrc, (__attribute__((address_space(3))) void*)&kdst[blk * 512], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vsrc, (__attribute__((address_space(3))) void*)&vdst[blk * 512], 16, 0, 0);
  };
  auto page_of = [&](int t) {  // this wave's page of tile t (wave-uniform), in elements
    const int pid = __builtin_amdgcn_readfirstlane(spid[kTilePages * (t - t_lo) + wave]);
    return (size_t)(pid < 0 ? 0 : pid) * kPage * D;
  };
  auto dma = [&](uint16_t* kdst, uint16_t* vdst, int t) {
    const size_t page = page_of(t);
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) dma_part(kdst, vdst, a.k_pool + page, a.v_pool + page, u);
  };

  // L2 warm-up of tile t: one 4-byte load per 128-byte line of its K and V
  // pages (256 lines = 256 threads), so that its copy two tiles later hits the
  // cache. The words land in a scratch LDS area that is never read, so nothing
  // waits for them until the barrier two tiles on.
  auto touch = [&](int t) {
    const int x = kTilePages * (t - t_lo) + ((tid >> 5) & 3);
    const int pid = spid[x];
    const uint16_t* base = (tid >> 7) ? a.v_pool : a.k_pool;
    const uint16_t* src = base + (size_t)(pid < 0 ? 0 : pid) * kPage * D + (size_t)(tid & 31) * (kPage * D / 32);
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&swarm[wave * 64], 4, 0, 0);
  };

  // S^T operand: K row this lane feeds for key block 0 (slot permutation; block 1: +32)
  const int krow0 = slot_key(lrow);
  // V^T operand: this lane's 8-byte run for the transpose reads
  const int q16 = lane >> 4, bsrc = lane & 15;
  const int tr_row = 8 * (q16 >> 1) + (bsrc >> 2);         // + 16 kk + 4 half
  const int tr_chunk = 2 * (q16 & 1) + ((bsrc & 3) >> 1);   // + 4 b
  const int tr_sub = 4 * (bsrc & 1);                        // element offset inside the chunk

  f32x16 o_acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o_acc[b][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  dma(sk0, sv0, t_lo);
  if (t_lo + 1 < t_hi) touch(t_lo + 1);
  if (t_lo + 2 < t_hi) touch(t_lo + 2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // one tile; stage B holds tile t, stage B^1 receives tile t+1
  auto body = [&](auto stage, int t) {
    constexpr int B = decltype(stage)::value;
    uint16_t* kcur = B ? sk1 : sk0;
    uint16_t* vcur = B ? sv1 : sv0;
    // copy of tile t+1 (the last tile copies itself again into the idle stage)
    uint16_t* kn = B ? sk0 : sk1;
    uint16_t* vn = B ? sv0 : sv1;
    const size_t npage = page_of(imin(t + 1, t_hi - 1));
    const uint16_t* knp = a.k_pool + npage;
    const uint16_t* vnp = a.v_pool + npage;
    dma_part(kn, vn, knp, vnp, 0);
    const int x0 = kTilePages * (t - t_lo);
    const int p0 = spos[x0], p1 = spos[x0 + 1], p2 = spos[x0 + 2], p3 = spos[x0 + 3];
    const bool all_valid = p0 != INT_MAX && p1 != INT_MAX && p2 != INT_MAX && p3 != INT_MAX;
    if (!all_valid) {  // zero V rows of missing pages (0 * NaN would poison O); rare, block-uniform
      const int pg = tid >> 6;  // 4 pages x 64 threads, 16 rows x D per page
      if (sel4(pg, p0, p1, p2, p3) == INT_MAX)
        for (int e = (tid & 63) * 8; e < kPage * D; e += 64 * 8)
          *reinterpret_cast<u32x4*>(&vcur[pg * kPage * D + e]) = u32x4{0, 0, 0, 0};
      __syncthreads();
    }

    // ---- S^T = K Q^T ----
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + krow0;
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&kcur[row * D + 8 * ((2 * ks + lg) ^ k_swz<D>(row))]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc[kb], 0, 0, 0);
      }
      if (ks == KS / 2 - 1 && KLOADS > 1) dma_part(kn, vn, knp, vnp, 1);
    }
    if (KLOADS > 2) dma_part(kn, vn, knp, vnp, 2);

    // ---- visibility, only on tiles that straddle a window edge ----
    const int kmin = imin(imin(p0, p1), imin(p2, p3));
    const int kmax = imax(imax(p0 == INT_MAX ? 0 : p0, p1 == INT_MAX ? 0 : p1),
                          imax(p2 == INT_MAX ? 0 : p2, p3 == INT_MAX ? 0 : p3)) + kPage - 1;
    const bool full = all_valid && kmax <= pos_min && (!is_local || kmin >= lo_max);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int pp = 2 * kb + (i >> 3);
          const int ps = pp == 0 ? p0 : pp == 1 ? p1 : pp == 2 ? p2 : p3;
          const int j = ps + 8 * lg + (i & 7);
          const bool vis = ps != INT_MAX && j <= pos && j >= lo_row;
          sc[kb][i] = vis ? sc[kb][i] : -INFINITY;
        }
    }

    // ---- online softmax (lazy rescale: only when the max grows by > 2^8) ----
    // row max as a 4-way tree of 3-input maxima (short dependency chains)
    float tm[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = sc[c >> 1];
      const int o = 8 * (c & 1);
      tm[c] = fmaxf(fmaxf(fmaxf(v[o], v[o + 1]), fmaxf(v[o + 2], v[o + 3])),
                    fmaxf(fmaxf(v[o + 4], v[o + 5]), fmaxf(v[o + 6], v[o + 7])));
    }
    float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_tile = tmax * a.scale_log2;
    const bool rescale = m_tile > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
      const float alpha = rescale ? exp2f(m_run - m_tile) : 1.f;  // m_run = -inf -> 0
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[b][i] *= alpha;
      m_run = rescale ? m_tile : m_run;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 pf[4];
    float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums (short dependency chains)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * hh + j], a.scale_log2, -m_use));
          pf[2 * kb + hh][j] = (__bf16)pv;
          ls[j & 3] += pv;
        }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

    if (KLOADS > 3) dma_part(kn, vn, knp, vnp, 3);
    static_assert(KLOADS <= 4, "the tile copy is issued in at most four parts");
    if (t + 3 < t_hi) touch(t + 3);  // issued last: the wait below may leave it in flight

    // ---- O^T += V^T P^T (V^T fragments from transpose reads) ----
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        bf16x4 v4[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int row = 16 * kk + tr_row + 4 * half;
          const int ch = 4 * b + tr_chunk;
          const uint16_t* src = &vcur[row * D + 8 * (ch ^ v_swz<D>(row)) + tr_sub];
          v4[half] = lds_read_tr16(src);
        }
        const bf16x8 vf = {v4[0][0], v4[0][1], v4[0][2], v4[0][3], v4[1][0], v4[1][1], v4[1][2], v4[1][3]};
        o_acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], o_acc[b], 0, 0, 0);
      }

    // this wave's copy of tile t+1 has landed (only the warm-up load issued
    // after it may still be in flight; vector memory completes in order), then
    // a bare barrier: the workgroup fence of __syncthreads would also wait for
    // the warm-up. The empty asm statements keep the compiler from moving LDS
    // accesses across it.
    if (t + 3 < t_hi)
      __builtin_amdgcn_s_waitcnt(kWaitVm1);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  for (int t = t_lo; t < t_hi; t += 2) {
    body(std::integral_constant<int, 0>{}, t);
    if (t + 1 < t_hi) body(std::integral_constant<int, 1>{}, t + 1);
  }

  const float l_row = l_run + __shfl_xor(l_run, 32);
  if (mt.partial_base < 0) {
    if (!row_valid) return;
    const float inv = 1.f / l_row;
    uint16_t* op = a.out + ((size_t)qrow * a.Hq + qhead) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * b + 8 * g4 + 4 * lg;
        *reinterpret_cast<bf16x4*>(op + d) =
            bf16x4{(__bf16)(o_acc[b][4 * g4 + 0] * inv), (__bf16)(o_acc[b][4 * g4 + 1] * inv),
                   (__bf16)(o_acc[b][4 * g4 + 2] * inv), (__bf16)(o_acc[b][4 * g4 + 3] * inv)};
      }
    if (a.lse != nullptr && lg == 0) a.lse[(size_t)qrow * a.Hq + qhead] = (m_run + log2f(l_row)) * kLn2;
  } else {
    char* slot = a.partials + (size_t)(mt.partial_base + it.chunk) * partial_slot_bytes(D);
    uint16_t* po = reinterpret_cast<uint16_t*>(slot) + (size_t)rm * D;
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;  // a row may see no key of this chunk: O_c = 0, l_c = 0
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * b + 8 * g4 + 4 * lg;
        *reinterpret_cast<bf16x4*>(po + d) =
            bf16x4{(__bf16)(o_acc[b][4 * g4 + 0] * inv), (__bf16)(o_acc[b][4 * g4 + 1] * inv),
                   (__bf16)(o_acc[b][4 * g4 + 2] * inv), (__bf16)(o_acc[b][4 * g4 + 3] * inv)};
      }
    if (lg == 0) {
      float* ml = reinterpret_cast<float*>(slot + partial_o_bytes(D)) + 2 * rm;
      *reinterpret_cast<f32x2*>(ml) = f32x2{m_run, l_row};
    }
  }
}

// Grid (split m-tile, row group): each thread merges one row's 4-wide d group
// over the m-tile's chunks, in chunk order:
//   O = sum_c 2^(m_c - m*) l_c (O_c / l_c) / sum_c 2^(m_c - m*) l_c,
//   LSE = (m* + log2 sum_c 2^(m_c - m*) l_c) ln 2.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int DG = D / 4;                       // 4-element groups per row
  constexpr int kRowsPerBlock = kAttnThreads / DG;
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  if ((int)blockIdx.x >= hdr->n_split) return;
  const MTile* mts = reinterpret_cast<const MTile*>(a.plan + a.L.mtiles_off);
  const int32_t* split = reinterpret_cast<const int32_t*>(a.plan + a.L.split_off);
  const MTile mt = mts[split[blockIdx.x]];
  const int MP = kMRows / a.G;
  const int rm = blockIdx.y * kRowsPerBlock + threadIdx.x / DG, dg = threadIdx.x % DG;
  const int hg = rm / MP, p = rm % MP;
  if (p >= mt.n_pos) return;
  const size_t slot = partial_slot_bytes(D);
  const char* base = a.partials + (size_t)mt.partial_base * slot;
  const char* ml0 = base + partial_o_bytes(D) + (size_t)rm * 2 * sizeof(float);
  const char* o0 = base + ((size_t)rm * D + 4 * dg) * 2;
  const int nc = mt.n_chunks;
  // chunks in batches of 16 whose loads are all in flight together; the
  // running max and sums are rescaled between batches
  constexpr int CB = 16;
  float mstar = -INFINITY, lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += CB) {
    f32x2 ml[CB];
    bf16x4 o[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = imin(c0 + u, nc - 1);
      ml[u] = *reinterpret_cast<const f32x2*>(ml0 + c * slot);
      o[u] = *reinterpret_cast<const bf16x4*>(o0 + c * slot);
    }
    float mb = mstar;
#pragma unroll
    for (int u = 0; u < CB; ++u) mb = c0 + u < nc ? fmaxf(mb, ml[u][0]) : mb;
    const float sc = mb == -INFINITY ? 1.f : exp2f(mstar - mb);  // nothing seen yet: nothing to rescale
    lsum *= sc;
    acc[0] *= sc;
    acc[1] *= sc;
    acc[2] *= sc;
    acc[3] *= sc;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      // a chunk where the row sees no key has l = 0, m = -inf: weight 0
      const float wl = c0 + u < nc && ml[u][1] > 0.f ? exp2f(ml[u][0] - mb) * ml[u][1] : 0.f;
      lsum += wl;
      acc[0] += wl * (float)o[u][0];
      acc[1] += wl * (float)o[u][1];
      acc[2] += wl * (float)o[u][2];
      acc[3] += wl * (float)o[u][3];
    }
    mstar = mb;
  }
  const float inv = 1.f / lsum;
  const int qhead = mt.h * a.G + hg, qrow = mt.q_row0 + p;
  uint16_t* op = a.out + ((size_t)qrow * a.Hq + qhead) * D + 4 * dg;
  *reinterpret_cast<bf16x4*>(op) = bf16x4{(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv),
                                          (__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)};
  if (dg == 0 && a.lse != nullptr) a.lse[(size_t)qrow * a.Hq + qhead] = (mstar + log2f(lsum)) * kLn2;
}

}  // namespace
}  // namespace segkv

using namespace segkv;

extern "C" int32_t segpaged_attn_prefill(const segkv_dims* dims, const segkv_meta* meta_host, const void* q,
                                         const void* k_pool, const void* v_pool, int64_t pool_pages,
                                         const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                         const void* plan_dev, size_t plan_bytes, float softmax_scale, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  HostPlan hp;
  int32_t st = compute_host_plan(dims, meta_host, &hp);
  if (st != SEGKV_OK) return st;
  if (!q || !k_pool || !v_pool || !page_ids_dev || !page_pos_dev || !plan_dev || !out)
    return fail(SEGKV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (pool_pages <= 0) return fail(SEGKV_ERR_INVALID_ARG, "pool_pages must be > 0");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(SEGKV_ERR_INVALID_ARG, "softmax_scale must be a positive finite number");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) || !aligned16(plan_dev))
    return fail(SEGKV_ERR_ALIGNMENT, "q, pools, out and plan must be 16-byte aligned");
  if (plan_bytes < hp.plan_bytes) return fail(SEGKV_ERR_WORKSPACE, "plan buffer too small");
  if (workspace_bytes < hp.workspace_bytes)
    return fail(SEGKV_ERR_WORKSPACE, "attention workspace " + std::to_string(workspace_bytes) + " < " +
                                         std::to_string(hp.workspace_bytes));
  if (hp.workspace_bytes > 0 && (!workspace || !aligned16(workspace)))
    return fail(SEGKV_ERR_ALIGNMENT, "workspace must be a 16-byte aligned device buffer");
  if (hp.n_items == 0) return SEGKV_OK;

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.pool_pages = pool_pages;
  a.page_ids = page_ids_dev;
  a.page_pos = page_pos_dev;
  a.plan = static_cast<const char*>(plan_dev);
  a.L = host_plan_layout(*dims, hp);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.partials = static_cast<char*>(workspace);
  a.scale_log2 = softmax_scale * kLog2e;
  a.Hq = dims->num_q_heads;
  a.G = dims->num_q_heads / dims->num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dims->head_dim == 128) {
    attn_main_kernel<128><<<hp.n_items, kAttnThreads, 0, s>>>(a);
    SEGKV_LAUNCH_CHECK();
    if (hp.n_split > 0) attn_combine_kernel<128><<<dim3(hp.n_split, kMRows * 32 / kAttnThreads), kAttnThreads, 0, s>>>(a);
  } else {
    attn_main_kernel<64><<<hp.n_items, kAttnThreads, 0, s>>>(a);
    SEGKV_LAUNCH_CHECK();
    if (hp.n_split > 0) attn_combine_kernel<64><<<dim3(hp.n_split, kMRows * 16 / kAttnThreads), kAttnThreads, 0, s>>>(a);
  }
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}
