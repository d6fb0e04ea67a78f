// Internal helpers shared by the segkv translation units (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/segkv.h"
#include "plan.h"

namespace segkv {

// ---- error reporting (thread-local detail, never throws) ----
void set_error(const std::string& msg);
int32_t fail(int32_t code, const std::string& msg);
void clear_error();

#define SEGKV_HIP_CHECK(expr)                                                            \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return ::segkv::fail(SEGKV_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

#define SEGKV_LAUNCH_CHECK() SEGKV_HIP_CHECK(hipGetLastError())

// Debug builds (compiled with SEGKV_DEBUG): kernels check the page ids and page
// positions they read and OR a bit into a device flag of their source file
// when one is out of range (release builds treat such a page as missing, or
// skip such a move, and check nothing). After its launches the entry point
// waits for the stream, reads the flag back, clears it, and returns
// SEGKV_ERR_DEVICE_CHECK if any bit was set. The wait makes debug builds
// synchronous, so they are for testing, not for graph capture.
#ifdef SEGKV_DEBUG
#define SEGKV_DEVICE_FLAG(name) static __device__ int name = 0
#define SEGKV_DCHECK(flag, cond, bit)        \
  do {                                       \
    if (!(cond)) atomicOr(&(flag), (bit));   \
  } while (0)
#define SEGKV_DEVICE_CHECK(flag, stream, what)                                                          \
  do {                                                                                                \
    SEGKV_HIP_CHECK(hipStreamSynchronize(stream));                                                    \
    int v_ = 0;                                                                                       \
    SEGKV_HIP_CHECK(hipMemcpyFromSymbol(&v_, HIP_SYMBOL(flag), sizeof(int), 0, hipMemcpyDeviceToHost)); \
    if (v_ != 0) {                                                                                    \
      const int z_ = 0;                                                                               \
      SEGKV_HIP_CHECK(hipMemcpyToSymbol(HIP_SYMBOL(flag), &z_, sizeof(int), 0, hipMemcpyHostToDevice)); \
      return ::segkv::fail(SEGKV_ERR_DEVICE_CHECK, std::string(what) + " (check bits " + std::to_string(v_) + ")"); \
    }                                                                                                 \
  } while (0)
#else
#define SEGKV_DEVICE_FLAG(name) static_assert(true, "")
#define SEGKV_DCHECK(flag, cond, bit) \
  do {                                \
  } while (0)
#define SEGKV_DEVICE_CHECK(flag, stream, what) \
  do {                                         \
  } while (0)
#endif

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- host-side layout helpers ----
// Validates dims + host metadata (all rules documented in segkv.h). Returns
// SEGKV_OK or an error code with the detail message set.
int32_t validate_layout(const segkv_dims* dims, const segkv_meta* m);

HeadView head_view_host(const segkv_dims& d, const segkv_meta& m, int r, int h);

// Host mirror of the device attention plan (exact counts).
struct HostPlan {
  int n_mtiles = 0, n_items = 0, n_split = 0, n_partials = 0, chunk_tiles = 1, max_tiles = 0, n_imp_items = 0;
  int key_blocks = 0;  // 64-key blocks of the longest request
  int64_t table_entries = 0, move_entries = 0, total_q_rows = 0, total_keys = 0;
  size_t plan_bytes = 0, workspace_bytes = 0;
};
int32_t compute_host_plan(const segkv_dims* dims, const segkv_meta* m, HostPlan* out);

inline PlanLayout host_plan_layout(const segkv_dims& d, const HostPlan& p) {
  return plan_layout(d.num_requests * d.num_kv_heads, d.num_requests, p.n_mtiles, p.n_items, p.n_split,
                     p.n_imp_items, p.key_blocks);
}

// Workspace of token_importance_topk: one fp32 partial per (kv head, key).
inline size_t importance_workspace_bytes(const segkv_dims& d, int64_t total_keys) {
  return (size_t)d.num_kv_heads * (size_t)total_keys * sizeof(float);
}

// Attention work-group slots of the current device (CUs x resident WGs per CU).
int attention_slots();

// ---- device-side types ----
typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Reads the metadata of (r, h) from the device copy.
__device__ __forceinline__ HeadView head_view_dev(const segkv_meta& m, int Hkv, int r, int h) {
  HeadView v;
  const int s_end = m.seg_indptr[r + 1];
  const int sq = s_end - 1;
  v.bq = m.seg_start[sq];
  v.Lq = m.seg_len[sq];
  v.Lk = v.bq + v.Lq;
  const int k = r * Hkv + h;
  v.cls = m.head_class[k];
  v.W = m.window[k];
  v.rlo[0] = v.rhi[0] = v.rlo[1] = v.rhi[1] = 0;
  if (v.cls == kClassRetrieval) {
    for (int a = 0; a < 2; ++a) {
      const int s = m.retr_seg[2 * k + a];
      v.rlo[a] = m.seg_start[s];
      v.rhi[a] = m.seg_start[s] + m.seg_len[s];
    }
  }
  return v;
}

}  // namespace segkv
