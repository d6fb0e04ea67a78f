/*
 * segkv — SegPagedAttention prefill on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libsegkv.so. The operations follow the four adapter calls the
 * RedKnot pages describe (paooo.com, "如何使用RedKnot": BUILDSTATE,
 * SELECTVISIBLESTATE, EXECUTE) and the runtime of the RedKnot README
 * (topairepos.com, "About" and "Key Ideas": per-(layer, kv_head) head classes,
 * per-head page tables over a segmented paged KV store, RoPE relocation of
 * reused segment K, attention-importance token selection for a sparse FFN).
 *
 * Conventions shared by every entry point
 *  - Every call returns an int32 status (SEGKV_OK or a negative error code);
 *    segkv_status_string() names it and segkv_last_error() gives a
 *    thread-local detail message. Nothing aborts, nothing throws across the
 *    boundary.
 *  - Arguments are validated on the host before anything is launched; a call
 *    that returns an error has enqueued no GPU work.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and is asynchronous: no call synchronises the host. The one
 *    exception is the debug build (libsegkv_debug.so, compiled with
 *    SEGKV_DEBUG): there rope_relocate, segpaged_attn_prefill (all forms),
 *    segpaged_attn_decode and token_importance_topk check every page id they
 *    read against the pool (and attention every table position against page
 *    starts), wait for the stream after their launches, and return
 *    SEGKV_ERR_DEVICE_CHECK if a check failed; the release build treats such
 *    a page as missing (or skips such a move) without reporting it.
 *  - The caller owns and allocates every buffer. The library allocates no
 *    device memory and keeps no device state between calls; scratch space is
 *    passed in as `workspace`/`plan`.
 *  - Pointers marked (host) are read synchronously during the call; (device)
 *    pointers must be device memory, 16-byte aligned for bf16 tensors.
 *  - bf16 tensors are raw 16-bit bfloat16 values. Token positions are
 *    absolute positions within a request.
 *  - Identical inputs give bitwise-identical outputs (no float atomics).
 *  - Supported: head_dim 64 or 128, page_size 16, num_q_heads a multiple of
 *    num_kv_heads with group size G = Hq/Hkv dividing 256.
 */
#ifndef SEGKV_H_
#define SEGKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define SEGKV_OK 0
#define SEGKV_ERR_INVALID_ARG (-1)   /* malformed shape, metadata or pointer */
#define SEGKV_ERR_UNSUPPORTED (-2)   /* valid but not implemented (head_dim, page size, group size) */
#define SEGKV_ERR_CAPACITY (-3)      /* an output buffer is too small */
#define SEGKV_ERR_ALIGNMENT (-4)     /* a device pointer is not 16-byte aligned */
#define SEGKV_ERR_WORKSPACE (-5)     /* workspace/plan buffer too small */
#define SEGKV_ERR_HIP (-6)           /* a HIP runtime call failed (no device, launch failure) */
#define SEGKV_ERR_DEVICE_CHECK (-7)  /* debug builds only (SEGKV_DEBUG): a device-side bounds check failed */

/* ---- head classes (RedKnot README, "About": global / local / retrieval / dense) ----
 * GLOBAL, DENSE : a query row at position i sees every key j <= i.
 * LOCAL(W)      : its own (query) segment causally plus a causal sliding window
 *                 of W keys that includes the row: j in [max(0, min(b_q, i-W+1)), i].
 * RETRIEVAL(S)  : its own segment causally plus two chosen reused segments in full. */
enum { SEGKV_GLOBAL = 0, SEGKV_LOCAL = 1, SEGKV_RETRIEVAL = 2, SEGKV_DENSE = 3 };

typedef struct {
  int32_t num_requests;   /* R */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv; query head g reads kv head g / (Hq/Hkv) */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t page_size;      /* P: 16 */
  int32_t num_segments;   /* S: total segments over all requests */
} segkv_dims;

/* Segment layout and head-class map. The same struct describes the host copy
 * (validated, used for sizing) and the device copy (read by kernels); the two
 * must hold identical values.
 * Segment s of request r is listed in [seg_indptr[r], seg_indptr[r+1]); a
 * request's segments are contiguous from position 0 (seg_start[first] = 0,
 * seg_start[s+1] = seg_start[s] + seg_len[s]), every start is a multiple of
 * page_size, and the LAST segment is the recomputed query segment (its rows
 * are the request's query rows). Only the query segment may have a length
 * that is not a multiple of page_size. */
typedef struct {
  const int32_t* seg_indptr;  /* [R+1] */
  const int32_t* seg_start;   /* [S]  new (insertion) start b_s */
  const int32_t* seg_len;     /* [S]  n_s > 0 */
  const int8_t* head_class;   /* [R*Hkv] SEGKV_GLOBAL..SEGKV_DENSE, request-major */
  const int32_t* window;      /* [R*Hkv] W > 0 for LOCAL heads, ignored otherwise */
  const int32_t* retr_seg;    /* [R*Hkv*2] absolute segment ids for RETRIEVAL heads:
                                 two distinct reused (non-query) segments of the same
                                 request; ignored otherwise */
} segkv_meta;

/* Sizes implied by a layout, computed on the host (exact, not bounds). */
typedef struct {
  int64_t table_entries;   /* total page-table entries over all (request, kv head) */
  int64_t move_entries;    /* head-aware relocation moves (table entries in reused segments) */
  int64_t total_q_rows;    /* T_q = sum of query-segment lengths */
  int64_t total_keys;      /* sum of context lengths L_k (importance vector length) */
  size_t plan_bytes;       /* device plan buffer for segkv_build_pages / segpaged_attn_prefill */
  size_t attn_workspace_bytes;  /* device workspace for segpaged_attn_prefill */
  size_t importance_workspace_bytes;  /* device workspace for token_importance_topk (Hkv x total_keys fp32) */
} segkv_sizes;

/* Status name ("SEGKV_OK", "SEGKV_ERR_INVALID_ARG", ...); static storage. */
const char* segkv_status_string(int32_t status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* segkv_last_error(void);

/* Validate a layout and compute its sizes. dims/meta/sizes: host. */
int32_t segkv_plan_sizes(const segkv_dims* dims, const segkv_meta* meta_host, segkv_sizes* sizes);

/*
 * SELECTVISIBLESTATE — per-(request, kv head) page tables over the working store.
 * (paooo.com "如何使用RedKnot": choose the reused local-head KV and the
 * global-head ranges; README "About": per-head page table + segmented store.)
 *
 * For each (r, h), the table lists, in ascending position order, every page
 * that holds at least one key visible to some query row of (r, h) under h's
 * class. Entry e of (r, h) is at index page_indptr[r*Hkv+h] + e:
 *   page_ids[e] = physical page in the working pool, page_pos[e] = position of
 *   the page's first token.
 * Working store layout: page q of segment s for kv head h is physical page
 *   seg_pages[seg_page_indptr[s*Hkv+h] + q]        (device, int32)
 * Optionally (move_src != NULL) it also writes the head-aware relocation move
 * list: for each (r, h) in order and each table entry inside a reused segment,
 *   move_src = cache page  cache_pages[cache_page_indptr[s*Hkv+h] + q],
 *   move_dst = the working page, move_delta = b_s - seg_orig_start[s].
 * Always writes the attention plan into `plan` (plan_bytes from
 * segkv_plan_sizes), consumed by segpaged_attn_prefill.
 * Capacities must be >= the exact sizes from segkv_plan_sizes (else
 * SEGKV_ERR_CAPACITY). cu_q: [R+1] device prefix sums of query lengths.
 */
int32_t segkv_build_pages(const segkv_dims* dims, const segkv_meta* meta_host, const segkv_meta* meta_dev,
                          const int32_t* cu_q_dev,
                          const int32_t* seg_page_indptr_dev, const int32_t* seg_pages_dev,
                          int32_t* page_indptr_dev, int32_t* page_ids_dev, int32_t* page_pos_dev,
                          int64_t table_capacity,
                          const int32_t* cache_page_indptr_dev, const int32_t* cache_pages_dev,
                          const int32_t* seg_orig_start_dev,
                          int32_t* move_src_dev, int32_t* move_dst_dev, int32_t* move_delta_dev,
                          int64_t move_capacity,
                          void* plan_dev, size_t plan_bytes, void* stream);

/*
 * Visible-span export (testing aid): for every query row and kv head, the
 * row's visible key set as up to 3 maximal half-open intervals [lo, hi) of
 * positions, ascending, padded with (-1, -1). spans: device int32
 * [T_q][Hkv][3][2].
 */
int32_t segkv_visible_spans(const segkv_dims* dims, const segkv_meta* meta_host, const segkv_meta* meta_dev,
                            const int32_t* cu_q_dev, int32_t* spans_dev, void* stream);

/*
 * BUILDSTATE relocation + page gather (README "About"/"Key Ideas": offline
 * segment KV with RoPE relocation "for numerical alignment"; aitrends.kr
 * "주요 기능").
 * For each move m: K page dst_page[m] of k_dst = RoPE rotation by delta[m]
 * positions of K page src_page[m] of k_src, and (if v_src != NULL) V page
 * dst_page[m] of v_dst = copy of V page src_page[m] of v_src.
 * Rotation: rotate-half pairs (j, j + D/2), angle delta * theta^(-2j/D);
 * angle formed and reduced modulo 2 pi in fp64, cos/sin in fp32, products in
 * fp32, result rounded to bf16 (RNE).
 * Pools: K [pages][page_size][head_dim] bf16 (token-major), V [pages][head_dim]
 * [page_size] bf16 (d-major); k_src/v_src with src_pool_pages pages and
 * k_dst/v_dst with dst_pool_pages pages. V pages are copied verbatim. Moves with a page id out of
 * range are skipped. In place (src page == dst page, same pool) is allowed;
 * otherwise destinations must not overlap sources.
 */
int32_t rope_relocate(const void* k_src, void* k_dst, const void* v_src, void* v_dst,
                      int64_t src_pool_pages, int64_t dst_pool_pages,
                      const int32_t* src_page_dev, const int32_t* dst_page_dev, const int32_t* delta_dev,
                      int32_t n_moves, int32_t page_size, int32_t head_dim, double rope_theta, void* stream);

/*
 * EXECUTE attention (paooo.com "RedKnot的技术原理": per-head paged storage with
 * a fused varlen kernel and no attention mask; "如何使用RedKnot": global heads
 * attend over the full range, local heads over reused paged KV).
 * q:   [T_q][Hq][D] bf16, RoPE already applied; row cu_q[r] + t of request r
 *      is the query at position b_q(r) + t.
 * out: [T_q][Hq][D] bf16, softmax(scale * q k^T) v over the row's visible keys.
 * lse: [T_q][Hq] fp32 natural-log sum of exp(scale * q k) over visible keys
 *      (nullable).
 * Keys are read only through the page tables written by segkv_build_pages for
 * the same layout, whose plan must be passed in `plan`. k_pool: [pool_pages]
 * [P][D] bf16, token-major; v_pool: [pool_pages][D][P] bf16, d-major (element
 * (d, t) of a page at d * P + t), so that the V^T operand of the PV product
 * is 8 consecutive tokens of one d. workspace: attn_workspace_bytes from
 * segkv_plan_sizes (may be NULL when that is 0).
 */
int32_t segpaged_attn_prefill(const segkv_dims* dims, const segkv_meta* meta_host,
                              const void* q, const void* k_pool, const void* v_pool, int64_t pool_pages,
                              const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                              const void* plan_dev, size_t plan_bytes,
                              float softmax_scale, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * segpaged_attn_prefill without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Arguments, layouts and results are those
 * of segpaged_attn_prefill. The split-KV partials live in a fixed device
 * array of 69206016 bytes (66 MiB) inside the library (one per GPU, held
 * until the process ends). That is the most attn_workspace_bytes can be on a
 * GPU with up to 256 compute units (the MI355X has 256), so there every
 * layout fits; elsewhere a layout needing more is rejected with
 * SEGKV_ERR_WORKSPACE before any launch. Calls no allocator. All calls
 * on one GPU share that array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give wrong results; calls ordered on
 * one stream are safe.
 */
int32_t segpaged_attn_prefill_noalloc(const segkv_dims* dims, const segkv_meta* meta_host,
                                      const void* q, const void* k_pool, const void* v_pool, int64_t pool_pages,
                                      const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                      const void* plan_dev, size_t plan_bytes,
                                      float softmax_scale, void* out, float* lse, void* stream);

/*
 * The same attention with an explicit mask in place of the class rule: the
 * tuned form of the masked-dense comparator (paooo.com "RedKnot的技术原理":
 * the fused kernel replaces a dense layout plus mask). Every key tile of
 * every m-tile reads mask[h][t][j] (t = batch query row, j = key position in
 * the row's request; nonzero = visible) instead of applying the head class.
 * Built with every kv head GLOBAL, the page tables hold every page up to
 * each request's end, which is the dense layout; keys after an m-tile's last
 * row position are still not computed, so the mask can only remove keys.
 * Every row's mask must keep at least one key (else its output is undefined).
 * Arguments as segpaged_attn_prefill, plus mask: device bytes
 * [Hkv][T_q][mask_L], 16-byte aligned; mask_L a multiple of 16 covering the
 * last page of every request (else SEGKV_ERR_INVALID_ARG).
 */
int32_t segpaged_attn_prefill_masked(const segkv_dims* dims, const segkv_meta* meta_host,
                                     const void* q, const void* k_pool, const void* v_pool, int64_t pool_pages,
                                     const int32_t* page_ids_dev, const int32_t* page_pos_dev,
                                     const void* plan_dev, size_t plan_bytes, float softmax_scale,
                                     const uint8_t* mask, int64_t mask_L, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-phase attention: one new query row per request, the next step of the
 * same requests (arXiv abstract: long-context generation; paooo.com
 * "如何使用RedKnot": EXECUTE over the visible state chosen per head).
 * The new token of request r sits at position i = L_k(r), right after its
 * query segment. Query head g (kv head h = g / G) attends over the keys the
 * class rule of the prefill gives position i: GLOBAL and DENSE every key,
 * LOCAL(W) the query segment and positions i-W+1..i, RETRIEVAL the query
 * segment and the two reused segments; always including the new token itself.
 * Stored keys are read through the page tables that segkv_build_pages wrote
 * for this layout (page_indptr/page_ids/page_pos, unchanged).
 * q_new: [R][Hq][D] bf16 (RoPE at i); k_new, v_new: [R][Hkv][D] bf16, the new
 * token's key (RoPE at i) and value. Pools as in segpaged_attn_prefill.
 * out: [R][Hq][D] bf16; lse: [R][Hq] fp32 natural log (nullable).
 * workspace: segkv_decode_workspace_size bytes (may be NULL when that is 0).
 * Limits: D in {64, 128}, G <= 16, page size 16 (else SEGKV_ERR_UNSUPPORTED).
 */
int32_t segkv_decode_workspace_size(const segkv_dims* dims, const segkv_meta* meta_host, size_t* bytes);
int32_t segpaged_attn_decode(const segkv_dims* dims, const segkv_meta* meta_host, const segkv_meta* meta_dev,
                             const void* q_new, const void* k_new, const void* v_new,
                             const void* k_pool, const void* v_pool, int64_t pool_pages,
                             const int32_t* page_indptr_dev, const int32_t* page_ids_dev,
                             const int32_t* page_pos_dev, float softmax_scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * EXECUTE selection (README "About": Elastic Sparsity, token-selective FFN from
 * attention importance; paooo.com "RedKnot的主要功能": top-k tokens by attention
 * score take the dense FFN).
 * importance[off_r + j] = sum over query heads g and the last n_last query rows
 * i of request r of exp(scale * q_{g,i} . k_j - lse[i][g]) for visible j, else
 * 0; off_r = sum of L_k over earlier requests, j in [0, L_k(r)). Summation
 * order is fixed. lse: as written by segpaged_attn_prefill (device, required).
 * topk_idx[koff_r + c], c < k[r]: the k[r] positions with the largest
 * importance, ties to the lower position, in ascending order; koff_r = sum of
 * k over earlier requests. k: host int32 [R], 0 <= k[r] <= L_k(r).
 * Other arguments as in segpaged_attn_prefill. topk_idx may be NULL to skip
 * selection. plan: the plan written by segkv_build_pages for this layout (its
 * importance work list: every 64-key block of every table). workspace:
 * device, 16-byte aligned, at least importance_workspace_bytes from
 * segkv_plan_sizes (else SEGKV_ERR_WORKSPACE); it receives one partial score
 * per (kv head, key of a block the head's table touches), summed over heads in
 * head order into `importance`. Limits: Hkv <= 64, R <= 65535,
 * Hq * (n_last rounded up to 32) <= 4096 (else SEGKV_ERR_UNSUPPORTED).
 */
int32_t token_importance_topk(const segkv_dims* dims, const segkv_meta* meta_host, const segkv_meta* meta_dev,
                              const int32_t* cu_q_dev, const void* q, const void* k_pool, int64_t pool_pages,
                              const int32_t* page_indptr_dev, const int32_t* page_ids_dev,
                              const int32_t* page_pos_dev, const void* plan_dev, size_t plan_bytes,
                              const float* lse_dev, float softmax_scale,
                              int32_t n_last, const int32_t* k_host, float* importance_dev,
                              int32_t* topk_idx_dev, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k of one fp32 score vector (scores: device [n], n <= 2^30): the k
 * indices with the largest scores, ties to the lower index, ascending; -0 and
 * +0 are equal. Same selection rule as token_importance_topk. NaN scores are
 * not supported (the selection is then unspecified). One 1024-thread
 * work-group per vector; vectors of up to 61440 scores stay in registers,
 * longer ones are re-read from memory on each of the five passes.
 */
int32_t segkv_topk_select(const float* scores_dev, int32_t n, int32_t k, int32_t* idx_dev, void* stream);

/*
 * Sparse SwiGLU FFN (paooo.com "RedKnot的主要功能"/"RedKnot的技术原理": dense
 * FFN for the selected tokens, identity residual for the rest).
 * For every selected row i = idx[c], c < k:
 *   hidden[i] <- bf16( hidden[i] + W_down . bf16( silu(W_gate . hidden[i]) * (W_up . hidden[i]) ) )
 * with fp32 accumulation; all other rows are left untouched (in place).
 * hidden: [n_rows][hidden_size] bf16; w_gate, w_up: [inter][hidden_size];
 * w_down: [hidden_size][inter]; idx: device int32 [k], distinct, in range.
 * hidden_size and inter must be multiples of 128. workspace:
 * sparse_ffn_workspace_size(k, inter) bytes (the bf16 activation).
 */
size_t sparse_ffn_workspace_size(int32_t k, int32_t inter);
int32_t sparse_ffn_swiglu(void* hidden, int32_t n_rows, int32_t hidden_size, int32_t inter,
                          const int32_t* idx_dev, int32_t k, const void* w_gate, const void* w_up,
                          const void* w_down, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Layer glue before the attention: the query segment's fused QKV projection,
 * RoPE at the rows' positions and the online append of their K/V into the
 * query segment's working pages (paooo.com "如何使用RedKnot": EXECUTE
 * recomputes the query segment; RedKnot README "About": the query segment's
 * KV is produced online into the per-head paged store).
 * Row t of request r (rows cu_q[r] .. cu_q[r+1]-1, cu_q as for
 * segkv_build_pages) sits at position p = b_q(r) + t - cu_q[r]. With
 * y = W_qkv . hidden[t] (fp32 accumulation) split into Hq query heads, then Hkv
 * key heads, then Hkv value heads of D values each:
 *   q_out[t][g]           = bf16(rope(y_q[g], p))
 *   K of (t, h)           = bf16(rope(y_k[h], p)) at page seg_pages[seg_page_indptr[s_q*Hkv+h] + (t-cu_q[r])/16],
 *                           slot (t-cu_q[r]) % 16 (k_pool token-major [pages][P][D])
 *   V of (t, h)           = bf16(y_v[h]) at the same page and slot (v_pool d-major [pages][D][P])
 * rope: rotate-half pairs (j, j + D/2) turned by p * rope_theta^(-2j/D), the
 * angle's cos/sin taken in fp64 and rounded to fp32. Rows whose page index
 * falls outside the segment's page run or the pool are not written.
 * hidden: [T_q][hidden_size] bf16; w_qkv: [(Hq + 2 Hkv) * D][hidden_size] bf16
 * (row-major, out_features first); q_out: [T_q][Hq][D] bf16. Every other pool
 * page is left untouched. workspace: segkv_qkv_workspace_size bytes (a
 * per-row cos/sin table and page-slot list).
 * Limits: hidden_size a multiple of 64 (else SEGKV_ERR_UNSUPPORTED).
 */
int32_t segkv_qkv_workspace_size(const segkv_dims* dims, const segkv_meta* meta_host, size_t* bytes);
int32_t segkv_qkv_rope_append(const segkv_dims* dims, const segkv_meta* meta_host, const segkv_meta* meta_dev,
                              const int32_t* cu_q_dev, const int32_t* seg_page_indptr_dev,
                              const int32_t* seg_pages_dev, int64_t pool_pages, const void* hidden,
                              int32_t hidden_size, const void* w_qkv, double rope_theta, void* q_out,
                              void* k_pool, void* v_pool, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Layer glue after the attention: the output projection added onto the
 * residual stream, in place (the attention half of the layer that EXECUTE
 * runs, paooo.com "如何使用RedKnot"):
 *   hidden[t] <- bf16( hidden[t] + W_o . attn[t] ),  t < n_rows, fp32 accumulation.
 * attn: [n_rows][in_features] bf16 (the attention output [T_q][Hq][D] is
 * in_features = Hq * D); w_o: [hidden_size][in_features] bf16; hidden:
 * [n_rows][hidden_size] bf16. Limits: in_features a multiple of 64,
 * hidden_size a multiple of 128 (else SEGKV_ERR_UNSUPPORTED).
 */
int32_t segkv_out_proj_residual(const void* attn, int32_t n_rows, int32_t in_features, const void* w_o,
                                void* hidden, int32_t hidden_size, void* stream);

/*
 * Masked-dense attention, the comparator of the paged head-aware layout
 * (paooo.com "RedKnot的技术原理", "RedKnot的核心优势": the fused varlen kernel
 * replaces a dense layout plus an attention mask, quoted as several times
 * slower). One request: for query row t and query head g (kv head
 * h = g / (Hq/Hkv)),
 *   O[t][g] = sum_j softmax_j( scale * q[t][g] . k[h][j] | mask[h][t][j] != 0 ) v[h][j]
 * over every key j < L; every score is computed, the mask only removes keys
 * from the softmax. A row whose mask is all zero gets O = 0, LSE = -inf.
 * q: [T][Hq][D] bf16; k: [Hkv][L][D] bf16; v_t: [Hkv][D][L] bf16 (V stored
 * d-major, element (j, d) at d * L + j); mask: [Hkv][T][L] bytes;
 * out: [T][Hq][D] bf16; lse: [T][Hq] fp32 natural log (nullable).
 * workspace: segkv_masked_dense_workspace_size bytes (split-KV partials).
 * Limits: D in {64, 128}; L a multiple of 64 (pad with masked keys).
 */
int32_t segkv_masked_dense_workspace_size(int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t L, size_t* bytes);
int32_t masked_dense_attn(const void* q, const void* k, const void* v_t, const uint8_t* mask, int32_t T, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t L, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SEGKV_H_ */
