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
#include <mutex>
#include <type_traits>

#include "common.h"

namespace segkv {
namespace {

constexpr int kAttnWaves = 8;                   // waves per attention work-group
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kCombineThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // lazy rescale: p <= 2^8 between rescales
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]):
// wait for vector memory down to 0 outstanding, leave the other counters alone
constexpr int kWaitVm0 = 0x0F70;
// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format)
constexpr int kBufferRsrcWord3 = 0x00020000;

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
  const uint16_t* zero_page;  // device address of g_zero_page
  float scale_log2;  // softmax_scale * log2(e)
  int Hq, G;
  const uint8_t* mask;  // explicit mask [Hkv][mask_rows][mask_L] (mask mode only)
  int64_t mask_rows, mask_L;
};

// Key (within a 32-key block) whose K row the lane feeding MFMA row `slot`
// loads, so that output register i of lane group g holds key 8g+i (i < 8) or
// 16+8g+(i-8) (i >= 8).
__device__ __forceinline__ int slot_key(int slot) {
  const int a = slot >> 3, g = (slot >> 2) & 1, b = slot & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

constexpr int kMaxItemEntries = kTilePages * kMaxChunkTiles;  // table entries of one item

// Source of the copies of a missing page: zero K rows (masked by position
// anyway) and zero V rows, so nothing has to be cleared in LDS. Kernels get its
// device address through AttnArgs::zero_page.
__device__ __attribute__((aligned(1024))) uint16_t g_zero_page[kPage * 128] = {};

// Raw buffer resource over `bytes` bytes at p, and an LDS copy through it:
// each lane moves 16 (4) bytes from byte voff of the buffer to LDS dst + 16 (4) lane
// (the builtins exist only in the device compilation pass).
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kBufferRsrcWord3);
}
__device__ __forceinline__ void buffer_to_lds16(buf_rsrc rs, void* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds4(buf_rsrc rs, void* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 4, voff, 0, 0, 0);
}
#else
struct buf_rsrc {};
__device__ inline buf_rsrc make_rsrc(const void*, int) { return {}; }
__device__ inline void buffer_to_lds16(buf_rsrc, void*, int) {}
__device__ inline void buffer_to_lds4(buf_rsrc, void*, int) {}
#endif

// max of x over the two lanes l and l ^ 32 (v_permlane32_swap exchanges the
// upper half of one register with the lower half of another)
// (the builtin exists only in the device compilation pass)
__device__ __forceinline__ float max_halves(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
  return x;
#endif
}

// LDS of one work-group: two stages of K and V tiles, plus the item's page
// table. K pages are token-major ([key][d]) with their 16-byte chunks
// XOR-swizzled per row; V pages are d-major ([d][16 keys], as stored in the
// pool) with the two 16-byte halves of a row swapped on every other group of
// 8 rows. Both operand reads below are then free of bank conflicts and full
// 16-byte reads. Every stage is its own __shared__ object and the loop is
// unrolled by the stage index, so the compiler can tell that reads of one
// stage do not alias the asynchronous copies into the other and does not wait
// on those copies.

// (host+device so the device lambdas below may call them)
template <int D>
SEGKV_HD int k_swz(int row) { return row & (D / 8 - 1); }  // S^T reads: 16 rows, one chunk


// Per item, key tiles i = 0 .. T-1 (T = t_hi - t_lo, T >= 1) in two LDS
// stages: K(i) and V(i) live in stage i & 1. The work-group's 8 waves (32 rows
// each) form two sets with one wave of each on every SIMD (the SIMD id comes
// from the hardware), which run the same steps one slot apart:
//   MFMA step of tile i:    S(i) = K(i) Q^T, then O += V(i-1)^T P(i-1)
//   softmax step of tile i: mask, row max, P(i) = exp2(S(i) - m), l
// Between two barriers (a slot), set 0 runs the MFMA step of tile s/2 while
// set 1 runs the softmax step of tile s/2 - 1 (s even), or the softmax step of
// tile (s-1)/2 while set 1 runs its MFMA step (s odd). Each SIMD's matrix core
// then works for one of its two waves while the other does vector work. At the
// start of slot 2i every wave issues its share of the copies of K(i+1) and
// V(i) into the stages nobody reads any more; they land before the barrier
// that ends slot 2i+1, ahead of the MFMA step of tile i+1. The V^T operand of
// a 16-key page is one 16-byte read per lane: 8 consecutive keys of one d.
// kMask: every tile takes its visibility from the explicit mask (one byte per
// kv head, query row and key) instead of the head-class rule.
template <int D, bool kMask>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_main_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int KS = D / 16;                 // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                 // 32-wide d blocks of O^T
  constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  constexpr int RPK = 1024 / (2 * D);        // K rows per 1 KiB transfer
  constexpr int PLOADS = kPage * KCH / 64;   // 1 KiB transfers per page
  constexpr int WLOADS = kTilePages * PLOADS / kAttnWaves;  // transfers per wave, tensor and tile
  static_assert(WLOADS >= 1 && PLOADS % WLOADS == 0, "a wave's copies stay inside one page");
  __shared__ __attribute__((aligned(1024))) uint16_t sk0[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sk1[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sk2[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv0[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv1[kTileKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv2[kTileKeys * D];
  __shared__ int spid[kMaxItemEntries];
  __shared__ __attribute__((aligned(16))) int spos[kMaxItemEntries];
  __shared__ uint32_t swarm[kAttnThreads];  // sink of the L2 warm-up loads
  __shared__ int s_simd[kAttnWaves];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const MTile* mts = reinterpret_cast<const MTile*>(a.plan + a.L.mtiles_off);
  const Item* items = reinterpret_cast<const Item*>(a.plan + a.L.items_off);
  if ((int)blockIdx.x >= hdr->n_items) return;
  const Item it = items[blockIdx.x];
  if (it.mtile < 0) return;  // empty slot of the XCD-aware order
  const MTile mt = mts[it.mtile];
  const int t_lo = chunk_tile_lo(mt.n_tiles, mt.n_chunks, it.chunk);
  const int T = chunk_tile_lo(mt.n_tiles, mt.n_chunks, it.chunk + 1) - t_lo;
  if (T <= 0) return;  // every m-tile chunk holds a tile (each row sees its own key)

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
  const uint8_t* mrow = kMask ? a.mask + ((size_t)mt.h * a.mask_rows + qrow) * a.mask_L + 8 * lg : nullptr;

  // the item's page table -> LDS (entries past the m-tile's end, or with an
  // invalid page id, become pid -1 / pos INT_MAX)
  const int e_lo = mt.e_begin + kTilePages * t_lo;
  for (int x = tid; x < kTilePages * T; x += kAttnThreads) {
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
  // the two waves of each SIMD: the first joins set 0, the second set 1
  // (hardware register HW_ID, bits 5:4 = SIMD id)
  const int simd = __builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));
  if (lane == 0) s_simd[wave] = simd;

  // Q fragments (B operand): Q[row][16 ks + 8 lg + 0..7]
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + ((size_t)qrow * a.Hq + qhead) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
  }
  __syncthreads();
  int rank = 0;
  for (int w = 0; w < wave; ++w) rank += s_simd[w] == simd;
  const int set = __builtin_amdgcn_readfirstlane(rank & 1);

  // Copies. Transfer g = WLOADS wave + u of a tile moves 1 KiB of page
  // g / PLOADS, so each wave copies inside one page (wave-uniform page id). A
  // missing page (id -1) is copied from an all-zero page: its keys are masked
  // by position and its zero V rows add nothing.
  int koff[WLOADS], voff[WLOADS];
#pragma unroll
  for (int u = 0; u < WLOADS; ++u) {
    const int part = (wave * WLOADS + u) % PLOADS;
    const int row = part * RPK + lane / KCH;  // K row inside the page
    koff[u] = row * D + 8 * ((lane % KCH) ^ k_swz<D>(row));
    // V pages are d-major ([d][16 tokens], 32 bytes per d): 16-byte half hs of
    // row d lands at hs ^ ((d >> 3) & 1), so the operand reads below (32 rows d,
    // both halves) hit distinct banks
    const int c = part * 64 + lane, vd = c >> 1;
    voff[u] = vd * kPage + 8 * ((c & 1) ^ ((vd >> 3) & 1));
  }
  const int cpage = wave * WLOADS / PLOADS;  // this wave's page of every tile
  // buffer resource of one page (raw, 4 KiB at D = 128)
  auto page_rsrc = [&](const uint16_t* page) __attribute__((always_inline)) {
    return make_rsrc(page, kPage * D * 2);
  };
  auto kpage_of = [&](int pid) __attribute__((always_inline)) { return pid < 0 ? a.zero_page : a.k_pool + (size_t)pid * kPage * D; };
  auto vpage_of = [&](int pid) __attribute__((always_inline)) { return pid < 0 ? a.zero_page : a.v_pool + (size_t)pid * kPage * D; };
  auto pid_of = [&](int i) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(spid[kTilePages * imin(i, T - 1) + cpage]); };
  // Copies go through buffer loads (a page-sized buffer resource per source
  // page): unlike global_load_lds they leave the compiler's LDS-read waits
  // exact while a copy is in flight.
  auto copy_k = [&](uint16_t* dst, const uint16_t* page) __attribute__((always_inline)) {
    const buf_rsrc rs = page_rsrc(page);
#pragma unroll
    for (int u = 0; u < WLOADS; ++u) buffer_to_lds16(rs, &dst[(wave * WLOADS + u) * 512], 2 * koff[u]);
  };
  auto copy_v = [&](uint16_t* dst, const uint16_t* page) __attribute__((always_inline)) {
    const buf_rsrc rs = page_rsrc(page);
#pragma unroll
    for (int u = 0; u < WLOADS; ++u) buffer_to_lds16(rs, &dst[(wave * WLOADS + u) * 512], 2 * voff[u]);
  };
  // L2 warm-up of a tile: wave w loads one 4-byte word per 1/64 of the K (w
  // even) or V (w odd) copy of its page, so that the copy two tiles later hits
  // the cache. The words land in an LDS area that is never read.
  const int warm_off = lane * (kPage * D / 32);  // bytes
  const bool warm_v = (wave & 1) != 0;
  auto touch = [&](int pid) __attribute__((always_inline)) {
    buffer_to_lds4(page_rsrc(warm_v ? vpage_of(pid) : kpage_of(pid)), &swarm[wave * 64], warm_off);
  };

  // S^T operand: K row this lane feeds for key block 0 (slot permutation; block 1: +32)
  const int krow0 = slot_key(lrow);
  // V^T operand: d-major page rows, this lane's row lrow of each 32-row d
  // block and its 8 keys lg of the page (swizzled half, as written by the copy)
  const int v_lane = lrow * kPage + 8 * (lg ^ ((lrow >> 3) & 1));

  f32x16 o_acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o_acc[b][i] = 0.f;
  // The running max m_run is an integer (or -inf), so a rescale factor is an
  // exact power of two.
  float m_run = -INFINITY, l_run = 0.f;
  // P of the previous tile in bf16, the B operand of its PV product. The first
  // MFMA step multiplies these zeros with the zeroed V stage 1.
  bf16x8 pprev[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) pprev[kk][j] = (__bf16)0.f;
  f32x16 sc[2];   // S(i) from the MFMA step to the softmax step
  int4 tpos_v;    // key positions of tile i's pages (read in its MFMA step)
  // a rescale of O found due by a softmax step, applied before the next PV product
  float o_scale = 1.f;
  bool o_scale_due = false;

  // stage buffers of tile i (stage i % 3, a compile-time index)
  auto kst = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value % 3;
    return S == 0 ? sk0 : S == 1 ? sk1 : sk2;
  };
  auto vst = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value % 3;
    return S == 0 ? sv0 : S == 1 ? sv1 : sv2;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  // K(0), K(1), V(0) before the loop; V(-1) (stage 2) is zero; page ids of
  // this wave's page in tiles i+1 .. i+4 (wave-uniform, clamped to T-1)
  int pid1 = pid_of(1), pid2 = pid_of(2), pid3 = pid_of(3), pid4 = pid_of(4);
  {
    const int pid0 = pid_of(0);
    copy_k(sk0, kpage_of(pid0));
    copy_k(sk1, kpage_of(pid1));
    copy_v(sv0, vpage_of(pid0));
  }
  for (int e = tid * 8; e < kTileKeys * D; e += kAttnThreads * 8) *reinterpret_cast<u32x4*>(&sv2[e]) = u32x4{0, 0, 0, 0};
  touch(pid2);
  touch(pid3);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto bar = [&]() __attribute__((always_inline)) {  // bare barrier; the empty asm statements keep LDS accesses on their side
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // at the end of slot 2i+1: this wave's copies of slot 2i-2 have landed (those
  // of slot 2i, kCopyOps vector memory operations, may stay in flight; vector
  // memory completes in order), then a barrier
  constexpr int kCopyOps = 2 * WLOADS + 1;
  static_assert(kCopyOps < 16, "vmcnt immediate");
  auto wait_copies_bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | kCopyOps);
    bar();
  };
  // copies of slot 2i: K(i+2) (near the end the last tile's K again, into an
  // idle stage) and V(i+1), then the warm-up of tile i+4; next page id lookup
  auto copies = [&](uint16_t* kdst, uint16_t* vdst, int i) __attribute__((always_inline)) {
    copy_k(kdst, kpage_of(pid2));
    copy_v(vdst, vpage_of(pid1));
    touch(pid4);
    pid1 = pid2;
    pid2 = pid3;
    pid3 = pid4;
    pid4 = pid_of(i + 5);
  };
  auto rescale_o = [&]() __attribute__((always_inline)) {
    if (o_scale_due) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[b][i] *= o_scale;
      o_scale_due = false;
    }
  };
  // PV piece of page kk: O^T[b] += V^T(page kk) P^T(page kk) for every d block
  auto pv_page = [&](const uint16_t* vbuf, const bf16x8& pk, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vbuf[(kk * D + 32 * b) * kPage + v_lane]);
      o_acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk, o_acc[b], 0, 0, 0);
    }
  };

  // MFMA step of tile i (stage P = i % 3): S(i) = K(i) Q^T, O += V(i-1)^T P(i-1)
  auto mfma_step = [&](auto par, int i) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    const uint16_t* kcur = kst(par);
    const uint16_t* vprev = vst(std::integral_constant<int, P + 2>{});
    tpos_v = *reinterpret_cast<const int4*>(&spos[kTilePages * i]);
    rescale_o();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + krow0;
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&kcur[row * D + 8 * ((2 * ks + lg) ^ k_swz<D>(row))]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc[kb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pv_page(vprev, pprev[kk], kk);
    // schedule: keep kAhead operand reads in flight ahead of the matrix
    // instructions (each read is one MFMA's A operand), so that LDS latency
    // hides behind the MFMA pipeline
    constexpr int kOps = 2 * KS + 4 * DB, kAhead = 10;
    if (kAhead > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // DS reads
#pragma unroll
    for (int m = 0; m < kOps - kAhead; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    }
  };

  // softmax step of tile i: visibility, row max (lazy rescale: the running max
  // moves only when a tile's max exceeds it by more than 2^8, and then to the
  // integer above), P(i) in bf16 and the row sums
  auto softmax_step = [&]() __attribute__((always_inline)) {
    const int p0 = __builtin_amdgcn_readfirstlane(tpos_v.x), p1 = __builtin_amdgcn_readfirstlane(tpos_v.y);
    const int p2 = __builtin_amdgcn_readfirstlane(tpos_v.z), p3 = __builtin_amdgcn_readfirstlane(tpos_v.w);
    const bool all_valid = p0 != INT_MAX && p1 != INT_MAX && p2 != INT_MAX && p3 != INT_MAX;
    const int kmin = imin(imin(p0, p1), imin(p2, p3));
    const int kmax = imax(imax(p0 == INT_MAX ? 0 : p0, p1 == INT_MAX ? 0 : p1),
                          imax(p2 == INT_MAX ? 0 : p2, p3 == INT_MAX ? 0 : p3)) + kPage - 1;
    const bool full = all_valid && kmax <= pos_min && (!is_local || kmin >= lo_max);
    if (kMask || !full) {  // the class rule masks only tiles that straddle a window edge
      uint64_t mb[4] = {0, 0, 0, 0};  // mask mode: bytes of keys ps + 8 lg .. + 7 of each page
      if (kMask) {
        if (p0 != INT_MAX) mb[0] = *reinterpret_cast<const uint64_t*>(mrow + p0);
        if (p1 != INT_MAX) mb[1] = *reinterpret_cast<const uint64_t*>(mrow + p1);
        if (p2 != INT_MAX) mb[2] = *reinterpret_cast<const uint64_t*>(mrow + p2);
        if (p3 != INT_MAX) mb[3] = *reinterpret_cast<const uint64_t*>(mrow + p3);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int pp = 2 * kb + (e >> 3);
          const int ps = pp == 0 ? p0 : pp == 1 ? p1 : pp == 2 ? p2 : p3;
          const int j = ps + 8 * lg + (e & 7);
          const bool vis = kMask ? ((mb[pp] >> (8 * (e & 7))) & 0xffu) != 0
                                 : ps != INT_MAX && j <= pos && j >= lo_row;
          sc[kb][e] = vis ? sc[kb][e] : -INFINITY;
        }
    }
    float tm[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& v = sc[c >> 1];
      const int o = 8 * (c & 1);
      tm[c] = fmaxf(fmaxf(fmaxf(v[o], v[o + 1]), fmaxf(v[o + 2], v[o + 3])),
                    fmaxf(fmaxf(v[o + 4], v[o + 5]), fmaxf(v[o + 6], v[o + 7])));
    }
    const float tmax = max_halves(fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3])));
    const float m_tile = tmax * a.scale_log2;
    const bool grow = m_tile > m_run + kRescaleThreshold;
    const float m_new = grow ? ceilf(m_tile) : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums (short dependency chains)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kk >> 1][8 * (kk & 1) + j], a.scale_log2, -m_use));
        pprev[kk][j] = (__bf16)pv;
        ls[j & 3] += pv;
      }
    // l moves to the new max now; O before the next PV product
    const float alpha = grow ? (m_run == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(m_run - ceilf(m_tile)))) : 1.f;
    l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
    m_run = m_new;
    o_scale = alpha;
    o_scale_due = __builtin_amdgcn_ballot_w64(grow) != 0;
  };

  if (set == 0) {
    // slot 2i: copies + MFMA step of tile i; slot 2i+1: softmax step of tile i
    auto tile = [&](auto par, int i) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      copies(kst(std::integral_constant<int, P + 2>{}), vst(std::integral_constant<int, P + 1>{}), i);
      mfma_step(par, i);
      bar();
      softmax_step();
      wait_copies_bar();
    };
    for (int i = 0; i < T; i += 3) {
      tile(S0{}, i);
      if (i + 1 < T) tile(S1{}, i + 1);
      if (i + 2 < T) tile(S2{}, i + 2);
    }
  } else {
    // slot 0: copies of tile 0; then slot 2i+1: MFMA step of tile i; slot
    // 2i+2: copies of tile i+1 + softmax step of tile i
    copies(sk2, sv1, 0);
    bar();
    auto tile = [&](auto par, int i) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      mfma_step(par, i);
      wait_copies_bar();
      if (i + 1 < T) {
        copies(kst(std::integral_constant<int, P + 3>{}), vst(std::integral_constant<int, P + 2>{}), i + 1);
        softmax_step();
        bar();
      } else {
        softmax_step();
      }
    };
    for (int i = 0; i < T; i += 3) {
      tile(S0{}, i);
      if (i + 1 < T) tile(S1{}, i + 1);
      if (i + 2 < T) tile(S2{}, i + 2);
    }
  }
  // the last copies and warm-up loads land before the work-group may end
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  {  // the last tile's PV product: V(T-1) sits in stage (T-1) % 3, landed before the last barrier
    rescale_o();
    const int last = (T - 1) % 3;
    const uint16_t* vlast = last == 0 ? sv0 : last == 1 ? sv1 : sv2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pv_page(vlast, pprev[kk], kk);
  }

  const float l_row = l_run + __shfl_xor(l_run, 32);
  // O leaves through LDS: the lane's O^T fragment (its row, 4-wide d groups)
  // goes to a per-wave [32 rows][D] block, 16-byte chunks XOR-swizzled by
  // row, and comes back whole rows per instruction, so every store writes
  // full rows (writing the fragments directly puts 32 rows in every store)
  const bool split = mt.partial_base >= 0;
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;  // a chunk may hold no key of a row: O_c = 0, l_c = 0
  __syncthreads();  // every wave's last PV product has read its V stage
  constexpr int OCH = D / 8;  // 16-byte chunks per row
  uint16_t* ostage = ((wave >> 1) == 0 ? sk0 : (wave >> 1) == 1 ? sk1 : (wave >> 1) == 2 ? sk2 : sv0) +
                     (wave & 1) * 32 * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c = 4 * b + g4;  // d = 32 b + 8 g4 + 4 lg .. + 4
      *reinterpret_cast<bf16x4*>(ostage + lrow * D + 8 * (c ^ (lrow & (OCH - 1))) + 4 * lg) =
          bf16x4{(__bf16)(o_acc[b][4 * g4 + 0] * inv), (__bf16)(o_acc[b][4 * g4 + 1] * inv),
                 (__bf16)(o_acc[b][4 * g4 + 2] * inv), (__bf16)(o_acc[b][4 * g4 + 3] * inv)};
    }
  char* slot = split ? a.partials + (size_t)(mt.partial_base + it.chunk) * partial_slot_bytes(D) : nullptr;
  constexpr int RPI = 64 / OCH;  // rows per read-back instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / OCH, c = lane % OCH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ostage + r * D + 8 * (c ^ (r & (OCH - 1))));
    const int rmr = wave * 32 + r, hgr = rmr / MP, pr = rmr % MP;
    if (split) {
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(slot) + (size_t)rmr * D + 8 * c) = v;
    } else if (pr < mt.n_pos) {
      *reinterpret_cast<u32x4*>(a.out + ((size_t)(mt.q_row0 + pr) * a.Hq + mt.h * a.G + hgr) * D + 8 * c) = v;
    }
  }
  if (lg == 0) {
    if (split) {
      float* ml = reinterpret_cast<float*>(slot + partial_o_bytes(D)) + 2 * rm;
      *reinterpret_cast<f32x2*>(ml) = f32x2{m_run, l_row};
    } else if (row_valid && a.lse != nullptr) {
      a.lse[(size_t)qrow * a.Hq + qhead] = (m_run + log2f(l_row)) * kLn2;
    }
  }
}

// Grid (split m-tile, row group): each thread merges one row's 4-wide d group
// over the m-tile's chunks, in chunk order:
//   O = sum_c 2^(m_c - m*) l_c (O_c / l_c) / sum_c 2^(m_c - m*) l_c,
//   LSE = (m* + log2 sum_c 2^(m_c - m*) l_c) ln 2.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int DG = D / 4;                       // 4-element groups per row
  constexpr int kRowsPerBlock = kCombineThreads / DG;
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

// Device address of g_zero_page on the current device, looked up once per
// device (the symbol's host-side name is not a device address).
constexpr int kMaxDevices = 64;

const uint16_t* zero_page_address() {
  static std::mutex mu;
  static const uint16_t* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_zero_page)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = static_cast<const uint16_t*>(p);
  }
  return addr[dev];
}

}  // namespace
}  // namespace segkv

using namespace segkv;

namespace {
int32_t attn_prefill(const segkv_dims* dims, const segkv_meta* meta_host, const void* q, const void* k_pool,
                     const void* v_pool, int64_t pool_pages, const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                     const void* plan_dev, size_t plan_bytes, float softmax_scale, const uint8_t* mask,
                     int64_t mask_L, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
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
  a.zero_page = zero_page_address();
  if (a.zero_page == nullptr) return fail(SEGKV_ERR_HIP, "hipGetSymbolAddress of the zero page failed");
  a.scale_log2 = softmax_scale * kLog2e;
  a.Hq = dims->num_q_heads;
  a.G = dims->num_q_heads / dims->num_kv_heads;
  a.mask = mask;
  a.mask_rows = hp.total_q_rows;
  a.mask_L = mask_L;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dims->head_dim == 128) {
    if (mask)
      attn_main_kernel<128, true><<<hp.n_items, kAttnThreads, 0, s>>>(a);
    else
      attn_main_kernel<128, false><<<hp.n_items, kAttnThreads, 0, s>>>(a);
    SEGKV_LAUNCH_CHECK();
    if (hp.n_split > 0) attn_combine_kernel<128><<<dim3(hp.n_split, kMRows * 32 / kCombineThreads), kCombineThreads, 0, s>>>(a);
  } else {
    if (mask)
      attn_main_kernel<64, true><<<hp.n_items, kAttnThreads, 0, s>>>(a);
    else
      attn_main_kernel<64, false><<<hp.n_items, kAttnThreads, 0, s>>>(a);
    SEGKV_LAUNCH_CHECK();
    if (hp.n_split > 0) attn_combine_kernel<64><<<dim3(hp.n_split, kMRows * 16 / kCombineThreads), kCombineThreads, 0, s>>>(a);
  }
  SEGKV_LAUNCH_CHECK();
  return SEGKV_OK;
}
}  // namespace

extern "C" int32_t segpaged_attn_prefill(const segkv_dims* dims, const segkv_meta* meta_host, const void* q,
                                         const void* k_pool, const void* v_pool, int64_t pool_pages,
                                         const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                         const void* plan_dev, size_t plan_bytes, float softmax_scale, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_prefill(dims, meta_host, q, k_pool, v_pool, pool_pages, page_ids_dev, page_pos_dev, plan_dev,
                      plan_bytes, softmax_scale, nullptr, 0, out, lse, workspace, workspace_bytes, stream);
}

extern "C" int32_t segpaged_attn_prefill_masked(const segkv_dims* dims, const segkv_meta* meta_host, const void* q,
                                                const void* k_pool, const void* v_pool, int64_t pool_pages,
                                                const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                                const void* plan_dev, size_t plan_bytes, float softmax_scale,
                                                const uint8_t* mask, int64_t mask_L, void* out, float* lse,
                                                void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const int32_t st = validate_layout(dims, meta_host);
  if (st != SEGKV_OK) return st;
  int64_t need = 0;
  for (int r = 0; r < dims->num_requests; ++r) {
    const int sq = meta_host->seg_indptr[r + 1] - 1;
    need = std::max<int64_t>(need, ((int64_t)meta_host->seg_start[sq] + meta_host->seg_len[sq] + kPage - 1) / kPage * kPage);
  }
  if (!mask) return fail(SEGKV_ERR_INVALID_ARG, "mask is NULL");
  if (!aligned16(mask)) return fail(SEGKV_ERR_ALIGNMENT, "mask must be 16-byte aligned");
  if (mask_L % kPage != 0 || mask_L < need)
    return fail(SEGKV_ERR_INVALID_ARG, "mask_L must be a multiple of 16 covering every request's last page");
  return attn_prefill(dims, meta_host, q, k_pool, v_pool, pool_pages, page_ids_dev, page_pos_dev, plan_dev,
                      plan_bytes, softmax_scale, mask, mask_L, out, lse, workspace, workspace_bytes, stream);
}
