// EXECUTE attention: SegPagedAttention prefill for the recomputed segment.
//
// paooo.com "RedKnot的技术原理": KV lives in per-head pages and a fused varlen
// kernel reads it without ever building an attention mask; "如何使用RedKnot":
// global heads attend over the full range, local heads over reused paged KV;
// RedKnot README "About": every head class has its own visible window over a
// per-head page table.
//
// Work decomposition. A work-group (8 waves, two per SIMD) owns one m-tile: the
// G query heads of one kv head times 256/G consecutive query positions (256
// rows), so every K/V page staged in LDS serves all G heads of the group. The m-tile's visible
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

#include "common.h"

namespace segkv {
namespace {

SEGKV_DEVICE_FLAG(g_attn_check);  // bit 1: table page id outside the pool; bit 2: page position not a page start

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

// An item's page table sits in LDS as a ring of kRingTiles tiles: tile t at
// entry kTilePages * (t % kRingTiles). Items longer than the ring refill the
// half they have finished with, 128 tiles at a time.
constexpr int kRingTiles = 256;
constexpr int kRingEntries = kTilePages * kRingTiles;

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

// LDS of one work-group: three stages of K and three of V tiles, plus the
// item's page table. K pages are token-major ([key][d]) with their 16-byte
// chunks XOR-swizzled per row; V pages are d-major ([d][16 keys], as stored in
// the pool) with the two 16-byte halves of a row swapped on every other group
// of 8 rows. Both operand reads below are then free of bank conflicts and full
// 16-byte reads.

// (host+device so the device lambdas below may call them)
template <int D>
SEGKV_HD int k_swz(int row) { return row & (D / 8 - 1); }  // S^T reads: 16 rows, one chunk


// Per item, key tiles i = 0 .. T-1 (T = t_hi - t_lo, T >= 1). Each of the 8
// waves owns 32 query rows. The two waves of every SIMD form two sets that
// alternate between a matrix step and a softmax step, one barrier per slot:
//   matrix step of tile i:   S(i) = K(i) Q^T, then O += V(i-1)^T P(i-1)
//   softmax step of tile i:  mask, row max, P(i) = exp2(S(i) - m) in bf16, row sums
// In slot 2i set 0 runs the matrix step of tile i while set 1 runs the
// softmax step of tile i-1; in slot 2i+1 the other way round. So each SIMD's
// matrix core works for one wave while the other issues vector work. K and V
// tiles are copied straight into LDS (buffer loads with the LDS destination),
// three stages each, tile j in stage j % 3; the copies of K(i+2) and V(i+1)
// are issued in slots 2i / 2i+1 and have landed by slot 2i+4. Stages are
// addressed at run time, so each set's loop body is a single copy of the code.
// The V^T operand of a 16-key page is one 16-byte LDS read per lane: 8
// consecutive keys of one d. A rescale of O found due by the softmax step of
// tile i is applied before the PV product of tile i.
// kMask: every tile takes its visibility from the explicit mask (one byte per
// kv head, query row and key) instead of the head-class rule.
template <int D, bool kMask>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_main_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int KS = D / 16;                 // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                 // 32-wide d blocks of O^T
  constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  constexpr int PCH = kPage * D * 2 / 1024;  // 1 KiB chunks per page
  constexpr int WCH = kTilePages * PCH / kAttnWaves;  // chunks per wave, tensor and tile
  static_assert(WCH >= 1 && PCH % WCH == 0, "a wave's chunks stay inside one page");
  constexpr int kStage = kTileKeys * D;      // elements of one K or V stage
  __shared__ __attribute__((aligned(1024))) uint16_t skv[6 * kStage];  // K stages 0-2, V stages 0-2
  __shared__ int spid[kRingEntries];
  __shared__ __attribute__((aligned(16))) int spos[kRingEntries];
  __shared__ int s_simd[kAttnWaves];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const Item* items = reinterpret_cast<const Item*>(a.plan + a.L.items_off);
  // The item record holds everything the work-group needs from the plan; it
  // is read together with the header's item count (the grid never exceeds
  // the items region the host sized for this layout), one round trip.
  const Item it = items[blockIdx.x];
  const int n_items = hdr->n_items;
  if ((int)blockIdx.x >= n_items || it.mtile < 0) return;  // empty slot of the XCD-aware order
  const int T = it.T;
  if (T <= 0) return;  // every m-tile chunk holds a tile (each row sees its own key)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 31, lg = lane >> 5;
  const int MP = kMRows / a.G;
  const int rm = wave * 32 + lrow;               // row within the m-tile
  const int hg = rm / MP, p = rm % MP;
  const bool row_valid = p < it.n_pos;
  const int pc = row_valid ? p : it.n_pos - 1;    // padding rows mirror the last valid row
  const int qhead = it.h * a.G + hg;
  const int qrow = it.q_row0 + pc;
  const int pos = it.pos0 + pc;
  const bool is_local = it.cls == kClassLocal;
  const int lo_row = is_local ? local_lo(pos, it.bq, it.W) : 0;
  const int pos_min = it.pos0, pos_max = it.pos0 + it.n_pos - 1;
  const int lo_max = is_local ? local_lo(pos_max, it.bq, it.W) : 0;

  // the item's page table -> LDS ring (entries past the m-tile's end, or with
  // an invalid page id, become pid -1 / pos INT_MAX); the first kRingTiles
  // tiles now, later ones by stage_table
  const int e_lo = it.e_lo;
  auto stage_entry = [&](int x) __attribute__((always_inline)) {  // entry x of the item
    const int e = e_lo + x;
    int pid = -1, ps = INT_MAX;
    if (e < it.e_end) {
      pid = a.page_ids[e];
      ps = a.page_pos[e];
      SEGKV_DCHECK(g_attn_check, pid >= 0 && pid < a.pool_pages, 1);
      SEGKV_DCHECK(g_attn_check, ps >= 0 && ps % kPage == 0, 2);
      if (pid < 0 || pid >= a.pool_pages) {
        pid = -1;
        ps = INT_MAX;
      }
    }
    spid[x % kRingEntries] = pid;
    spos[x % kRingEntries] = ps;
  };
  for (int x = tid; x < kTilePages * imin(T, kRingTiles); x += kAttnThreads) stage_entry(x);

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

  // Copies. Chunk g = WCH wave + u of a tile is 1 KiB of page g / PCH, so each
  // wave copies inside one page (wave-uniform page id). Lane l moves 16 bytes
  // to LDS byte 16 l of the chunk's kilobyte; which 16 bytes of the page it
  // fetches is chosen so that the LDS layout comes out swizzled: K rows are
  // token-major with their 16-byte chunks XOR-swizzled per row, V pages are
  // d-major ([d][16 tokens]) with the two 16-byte halves of a row swapped on
  // every other group of 8 d. Both operand reads below are then free of bank
  // conflicts and full 16-byte reads. A missing page (id -1) is read from an
  // all-zero page: its keys are masked by position and its zero V rows add
  // nothing.
  const int cpage = wave * WCH / PCH;  // this wave's page of every tile
  constexpr int RPK = 1024 / (2 * D);  // K rows per kilobyte
  int koff[WCH], voff[WCH];            // source byte offsets in the page
#pragma unroll
  for (int u = 0; u < WCH; ++u) {
    const int part = (wave * WCH + u) % PCH;
    const int row = part * RPK + lane / KCH;  // K row inside the page
    koff[u] = 2 * (row * D + 8 * ((lane % KCH) ^ k_swz<D>(row)));
    const int c = part * 64 + lane, vd = c >> 1;
    voff[u] = 2 * (vd * kPage + 8 * ((c & 1) ^ ((vd >> 3) & 1)));
  }
  auto pid_of = [&](int i) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(spid[kTilePages * (imin(i, T - 1) % kRingTiles) + cpage]);
  };
  // raw buffer resource over one page
  auto page_rsrc = [&](const uint16_t* pool, int pid) __attribute__((always_inline)) {
    const uint64_t addr = reinterpret_cast<uint64_t>(pid < 0 ? a.zero_page : pool + (size_t)pid * kPage * D);
    return u32x4{(uint32_t)addr, (uint32_t)(addr >> 32) & 0xffffu, (uint32_t)(kPage * D * 2), (uint32_t)kBufferRsrcWord3};
  };
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(skv);  // LDS byte address
  const uint32_t wave_dst = (uint32_t)(wave * WCH * 1024);
  // one 16-byte-per-lane copy into LDS. Written as one asm statement so the
  // compiler does not treat the LDS reads of other stages as waiting on it:
  // completion is managed here (s_waitcnt vmcnt + barrier). The instruction
  // has no register result.
  auto dma = [&](uint32_t lds_byte, const u32x4& rs, int off) __attribute__((always_inline)) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_byte), "v"(off), "s"(rs)
                 : "memory", "m0");
  };
  auto copy_k = [&](int pid, int stage) __attribute__((always_inline)) {  // K page `pid` into K stage `stage`
    const u32x4 rs = page_rsrc(a.k_pool, pid);
    const uint32_t dst = lds_base + (uint32_t)(stage * kStage * 2) + wave_dst;
#pragma unroll
    for (int u = 0; u < WCH; ++u) dma(dst + 1024 * u, rs, koff[u]);
  };
  auto copy_v = [&](int pid, int stage) __attribute__((always_inline)) {  // V page `pid` into V stage `stage`
    const u32x4 rs = page_rsrc(a.v_pool, pid);
    const uint32_t dst = lds_base + (uint32_t)((3 + stage) * kStage * 2) + wave_dst;
#pragma unroll
    for (int u = 0; u < WCH; ++u) dma(dst + 1024 * u, rs, voff[u]);
  };
  constexpr int kCopyOps = 2 * WCH;  // vector memory operations of one iteration's copies
  static_assert(3 * WCH < 16, "vmcnt immediate");
  const char* lds = reinterpret_cast<const char*>(skv);
  auto kstage = [&](int stage) __attribute__((always_inline)) { return lds + stage * (kStage * 2); };
  auto vstage = [&](int stage) __attribute__((always_inline)) { return lds + (3 + stage) * (kStage * 2); };

  // S^T operand: the K row this lane feeds for key block 0 (slot permutation;
  // block 1: +32). The read of k-step ks sits at chunk (2 ks + lg) ^ swz of the
  // row (one xor-add per read).
  const int krow0 = slot_key(lrow);
  const int k_row_bytes = 2 * krow0 * D;
  const int k_sw = 16 * (lg ^ k_swz<D>(krow0));  // same swizzle for rows krow0 and krow0 + 32
  // V^T operand: d-major page rows, this lane's row lrow of each 32-row d
  // block and its 8 keys lg of the page (swizzled half, as written by the copy)
  const int v_lane_bytes = 2 * (lrow * kPage + 8 * (lg ^ ((lrow >> 3) & 1)));

  f32x16 o_acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o_acc[b][i] = 0.f;
  // The running max m_run is an integer (or -inf), so a rescale factor is an
  // exact power of two.
  float m_run = -INFINITY, l_run = 0.f;
  // P of the previous tile in bf16, the B operand of its PV product (zero
  // before tile 0); the softmax of a tile overwrites each page's part after the
  // PV product of the previous tile has read it
  bf16x8 pk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) pk[kk][j] = (__bf16)0.f;
  f32x16 sc[2];  // S^T of the current tile (two 32-key blocks)
  // a rescale of O found due by a softmax, applied before the next PV product
  float o_scale = 1.f;
  bool o_scale_due = false;

  auto bar = [&]() __attribute__((always_inline)) {  // bare barrier; the empty asm statements keep LDS accesses on their side
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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
  // visibility of tile i (positions tp of its 4 pages): a tile that does not
  // straddle a window edge, the causal diagonal or a missing page takes no
  // mask work
  auto mask_if_needed = [&](int i) __attribute__((always_inline)) {
    const int4 tp = *reinterpret_cast<const int4*>(&spos[kTilePages * (i % kRingTiles)]);
    const int ps4[4] = {__builtin_amdgcn_readfirstlane(tp.x), __builtin_amdgcn_readfirstlane(tp.y),
                        __builtin_amdgcn_readfirstlane(tp.z), __builtin_amdgcn_readfirstlane(tp.w)};
    bool full = true;
    if (!kMask) {
      int kmin = INT_MAX, kmax = 0;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        full = full && ps4[pp] != INT_MAX;
        kmin = imin(kmin, ps4[pp]);
        kmax = imax(kmax, ps4[pp] == INT_MAX ? 0 : ps4[pp]);
      }
      full = full && kmax + kPage - 1 <= pos_min && (!is_local || kmin >= lo_max);
    }
    if (kMask || !full) {
      if (kMask) {
        // bytes of keys ps + 8 lg .. + 7 of each page, this row
        const uint8_t* mrow = a.mask + ((size_t)it.h * a.mask_rows + qrow) * a.mask_L + 8 * lg;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint64_t mb = ps4[pp] != INT_MAX ? *reinterpret_cast<const uint64_t*>(mrow + ps4[pp]) : 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = 8 * (pp & 1) + e;
            sc[pp >> 1][k] = ((mb >> (8 * e)) & 0xffu) != 0 ? sc[pp >> 1][k] : -INFINITY;
          }
        }
      } else {
        // key j is visible iff lo_row <= j <= pos; a missing page (position
        // INT_MAX) is placed far below every row's window
        const unsigned span = (unsigned)(pos - lo_row);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int ps = ps4[pp] == INT_MAX ? -(1 << 30) : ps4[pp];
          const int d0 = ps + 8 * lg - lo_row;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = 8 * (pp & 1) + e;
            sc[pp >> 1][k] = (unsigned)(d0 + e) <= span ? sc[pp >> 1][k] : -INFINITY;
          }
        }
      }
    }
  };
  // K and V operand reads from LDS: K rows for S^T (the read of k-step ks
  // sits at chunk (2 ks + lg) ^ swz of the row), V^T rows d-major
  auto rd_k = [&](const char* kbuf, int kb, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(kbuf + k_row_bytes + 64 * D * kb + ((32 * ks) ^ k_sw));
  };
  auto rd_v = [&](const char* vbuf, int kk, int b) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(vbuf + v_lane_bytes + 2 * (kk * D + 32 * b) * kPage);
  };
  // matrix step of tile i: S(i) = K(i) Q^T, then O += V(i-1)^T P(i-1). Operand
  // reads run kAhead ahead of the matrix instructions that use them.
  auto mfma_step = [&](const char* kbuf, const char* vbuf) __attribute__((always_inline)) {
    rescale_o();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_k(kbuf, kb, ks), qf[ks], ks == 0 ? f32x16{} : sc[kb], 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int b = 0; b < DB; ++b)
        o_acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_v(vbuf, kk, b), pk[kk], o_acc[b], 0, 0, 0);
    constexpr int kOps = 2 * KS + 4 * DB, kAhead = 12;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // DS reads
#pragma unroll
    for (int m = 0; m < kOps - kAhead; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  // softmax step of tile i: visibility, row max and the running max (lazy:
  // it moves only when a tile's max exceeds it by more than 2^8, and then to
  // the integer above, so a rescale factor is an exact power of two), P(i) in
  // bf16, row sums of the unrounded probabilities in fp32
  auto softmax_step = [&](int i) __attribute__((always_inline)) {
    // The other wave of this SIMD is in its matrix step meanwhile; its MFMAs
    // and LDS reads cost this wave issue slots, and this (vector-ALU bound)
    // step is the longer of the two, so it takes the higher issue priority
    // while it runs. (The reverse, priority for the matrix step, is slower.)
    __builtin_amdgcn_s_setprio(2);
    mask_if_needed(i);
    float mx[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // four chains of three-input maxima over 8 values
      const f32x16& v = sc[c >> 1];
      const int o = 8 * (c & 1);
      float t = fmaxf(fmaxf(v[o], v[o + 1]), v[o + 2]);
      t = fmaxf(fmaxf(t, v[o + 3]), v[o + 4]);
      t = fmaxf(fmaxf(t, v[o + 5]), v[o + 6]);
      mx[c] = fmaxf(t, v[o + 7]);
    }
    const float tmax = max_halves(fmaxf(fmaxf(fmaxf(mx[0], mx[1]), mx[2]), mx[3]));
    const float m_tile = tmax * a.scale_log2;
    const bool grow = m_tile > m_run + kRescaleThreshold;
    const float m_new = grow ? ceilf(m_tile) : m_run;
    // l and O move to the new max (O before the next PV product).
    // Branch-free: from m_run = -inf the factor is 2^-200 = 0.
    const float alpha = grow ? __builtin_amdgcn_ldexpf(1.f, (int)fmaxf(m_run - m_new, -200.f)) : 1.f;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 pv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = __builtin_amdgcn_exp2f(fmaf(sc[kk >> 1][8 * (kk & 1) + j], a.scale_log2, -m_use));
        pv[j] = (__bf16)x;
        ls[j & 3] += x;
      }
      pk[kk] = pv;
    }
    l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
    m_run = m_new;
    o_scale = alpha;
    o_scale_due = __builtin_amdgcn_ballot_w64(grow) != 0;
    __builtin_amdgcn_s_setprio(0);
  };
  auto last_pv = [&](const char* vbuf) __attribute__((always_inline)) {
    rescale_o();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int b = 0; b < DB; ++b)
        o_acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_v(vbuf, kk, b), pk[kk], o_acc[b], 0, 0, 0);
  };
  // at the end of an odd slot: this wave's copies issued two slots before the
  // last even slot have landed (those of the last even slot, kCopyOps vector
  // memory operations, may stay in flight), then a barrier
  auto wait_copies_bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | kCopyOps);
    bar();
  };

  // prologue: K(0), K(1), V(0) land before the first slot; V(-1) = 0 in V stage 2
  copy_k(pid_of(0), 0);
  copy_k(pid_of(1), 1);
  copy_v(pid_of(0), 0);
  for (int e = tid * 16; e < kStage * 2; e += kAttnThreads * 16)
    *reinterpret_cast<u32x4*>(skv + 5 * kStage + e / 2) = u32x4{0, 0, 0, 0};
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // Slots alternate between the two sets: in slot 2i set 0 runs the matrix
  // step of tile i while set 1 runs the softmax step of tile i-1; in slot 2i+1
  // set 0 runs the softmax step of tile i while set 1 runs the matrix step of
  // tile i. Each SIMD's matrix core then works for one of its waves while the
  // other does vector work. At the start of slot 2i every wave issues the
  // copies of K(i+2) and V(i+1) (stages of tile j: j % 3). The page id of the
  // next K copy is read from LDS one tile ahead (its V copy reuses it a tile
  // later), so no copy waits on an LDS read.
  int st_m = 2, st_0 = 0, st_p = 1;  // stages of tiles i-1, i, i+1
  auto rotate = [&]() __attribute__((always_inline)) {
    const int t = st_m;
    st_m = st_0;
    st_0 = st_p;
    st_p = t;
  };
  int pid_v = pid_of(1), pid_k = pid_of(2);  // pages of the next V and K copies
  auto issue_copies = [&](int i) __attribute__((always_inline)) {  // K(i+2), V(i+1) of slot 2i
    copy_k(pid_k, st_m);
    copy_v(pid_v, st_p);
    const int nxt = spid[kTilePages * (imin(i + 3, T - 1) % kRingTiles) + cpage];  // K(i+3), read into a VGPR now
    pid_v = pid_k;
    return nxt;
  };
  // Ring refill: the table reads of iteration i (either set) stay within
  // tiles i-2 .. i+5, so at i = 128 k + 64 (k >= 1) the half holding tiles
  // 128 (k-1) .. 128 k - 1 is finished with; every thread, in its set's
  // iteration i, writes its entries of tiles 128 (k+1) .. 128 (k+1) + 127 into
  // it, first read some 60 iterations (and barriers) later.
  auto stage_table = [&](int i) __attribute__((always_inline)) {
    if (i >= kRingTiles - 64 && (i & 127) == 64 && (i & ~127) + 128 < T) {
      const int t0 = (i & ~127) + 128;
      const int x_end = kTilePages * imin(t0 + 128, T);
      for (int x = kTilePages * t0 + tid; x < x_end; x += kAttnThreads) stage_entry(x);
    }
  };
  if (set == 0) {
    for (int i = 0; i < T; ++i) {
      mfma_step(kstage(st_0), vstage(st_m));
      bar();
      // (set 0 issues the copies of slot 2i in slot 2i+1, off its matrix step)
      const int nxt = issue_copies(i);
      stage_table(i);
      softmax_step(i);
      wait_copies_bar();
      pid_k = __builtin_amdgcn_readfirstlane(nxt);
      rotate();
    }
  } else {
    pid_k = __builtin_amdgcn_readfirstlane(issue_copies(0));
    bar();
    for (int i = 0; i < T; ++i) {
      mfma_step(kstage(st_0), vstage(st_m));
      wait_copies_bar();
      stage_table(i);
      if (i + 1 < T) {
        rotate();
        const int nxt = issue_copies(i + 1);
        softmax_step(i);
        bar();
        pid_k = __builtin_amdgcn_readfirstlane(nxt);
      } else {
        softmax_step(i);
        rotate();
      }
    }
  }
  // the PV product of tile T-1 (V(T-1) has landed; st_m is its stage)
  last_pv(vstage(st_m));
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the last (unused) copies land before the work-group may end

  const float l_row = l_run + __shfl_xor(l_run, 32);
  // O leaves through LDS: the lane's O^T fragment (its row, 4-wide d groups)
  // goes to a per-wave [32 rows][D] block, 16-byte chunks XOR-swizzled by
  // row, and comes back whole rows per instruction, so every store writes
  // full rows (writing the fragments directly puts 32 rows in every store)
  const bool split = it.partial_slot >= 0;
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;  // a chunk may hold no key of a row: O_c = 0, l_c = 0
  __syncthreads();  // every wave's last PV product has read its V stage
  constexpr int OCH = D / 8;  // 16-byte chunks per row
  uint16_t* ostage = skv + wave * 32 * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c = 4 * b + g4;  // d = 32 b + 8 g4 + 4 lg .. + 4
      *reinterpret_cast<bf16x4*>(ostage + lrow * D + 8 * (c ^ (lrow & (OCH - 1))) + 4 * lg) =
          bf16x4{(__bf16)(o_acc[b][4 * g4 + 0] * inv), (__bf16)(o_acc[b][4 * g4 + 1] * inv),
                 (__bf16)(o_acc[b][4 * g4 + 2] * inv), (__bf16)(o_acc[b][4 * g4 + 3] * inv)};
    }
  char* slot = split ? a.partials + (size_t)it.partial_slot * partial_slot_bytes(D) : nullptr;
  constexpr int RPI = 64 / OCH;  // rows per read-back instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / OCH, c = lane % OCH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ostage + r * D + 8 * (c ^ (r & (OCH - 1))));
    const int rmr = wave * 32 + r, hgr = rmr / MP, pr = rmr % MP;
    if (split) {
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(slot) + (size_t)rmr * D + 8 * c) = v;
    } else if (pr < it.n_pos) {
      *reinterpret_cast<u32x4*>(a.out + ((size_t)(it.q_row0 + pr) * a.Hq + it.h * a.G + hgr) * D + 8 * c) = v;
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
  // the split record and the header's count in one round trip (the grid
  // never exceeds the split region the host sized for this layout)
  const SplitTile mt = reinterpret_cast<const SplitTile*>(a.plan + a.L.split_off)[blockIdx.x];
  const int n_split = hdr->n_split;
  if ((int)blockIdx.x >= n_split) return;
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

// Split-KV partials buffer of segpaged_attn_prefill_noalloc: a fixed device
// array, so that entry point calls no allocator. Each device holds its own
// copy for the life of the process. Its size is the most any layout needs on
// a part with up to 256 compute units: at most kMaxItemRounds x 256 work items,
// each with one D = 128 partial (bf16 O rows + fp32 m, l of 256 rows).
constexpr size_t kNoAllocScratchBytes = (size_t)kMaxItemRounds * 256 * (kMRows * 128 * 2 + kMRows * 2 * 4);
static_assert(kNoAllocScratchBytes == 69206016, "66 MiB");
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per device
// with that device current (the host-side name is only a stand-in).
char* scratch_address() {
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    char* p = nullptr;
    if (hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = p;
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
                     int64_t mask_L, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                     bool fixed_scratch = false) {
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
  if (workspace_bytes < hp.workspace_bytes) {
    if (fixed_scratch)
      return fail(SEGKV_ERR_WORKSPACE, "layout needs " + std::to_string(hp.workspace_bytes) +
                                           " bytes of split-KV partials, above the fixed " +
                                           std::to_string(workspace_bytes) + "-byte scratch of the no-alloc entry");
    return fail(SEGKV_ERR_WORKSPACE, "attention workspace " + std::to_string(workspace_bytes) + " < " +
                                         std::to_string(hp.workspace_bytes));
  }
  if (fixed_scratch) {
    workspace = scratch_address();
    if (workspace == nullptr) return fail(SEGKV_ERR_HIP, "hipGetSymbolAddress of the attention scratch failed");
  }
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
  SEGKV_DEVICE_CHECK(g_attn_check, s, "segpaged_attn_prefill: a page-table entry is out of range");
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

extern "C" int32_t segpaged_attn_prefill_noalloc(const segkv_dims* dims, const segkv_meta* meta_host,
                                                 const void* q, const void* k_pool, const void* v_pool,
                                                 int64_t pool_pages, const int32_t* page_ids_dev,
                                                 const int32_t* page_pos_dev, const void* plan_dev,
                                                 size_t plan_bytes, float softmax_scale, void* out, float* lse,
                                                 void* stream) {
  clear_error();
  // the scratch address is looked up after the size checks; every split chunk
  // writes its whole partial slot before the combine reads it, so the scratch
  // needs no clearing between calls
  return attn_prefill(dims, meta_host, q, k_pool, v_pool, pool_pages, page_ids_dev, page_pos_dev, plan_dev,
                      plan_bytes, softmax_scale, nullptr, 0, out, lse, nullptr, kNoAllocScratchBytes, stream,
                      true);
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
