/*
 * entmaxkv.h - C ABI of a support-aware sparse alpha-entmax decode library
 * for a paged KV cache, written for AMD Instinct MI355X (gfx950).
 *
 * What it computes follows "Riepilogo Tecnico: EntmaxKV - Decodifica
 * Consapevole del Supporto per l'Attention Entmax" (gist.science, paper
 * 2605.21649), cited here as [EntmaxKV page]:
 *   section 2.A  per-page key bounding boxes (k_min, k_max) and the
 *                deterministic upper bound they give on a page's best score;
 *   section 2.B  policy 1, a fixed budget of the top-k pages by that bound;
 *                policy 2, pages kept by a tau estimated from per-page
 *                Gaussian statistics of the keys (mean and variance);
 *   section 2.C  only the selected pages' K/V are read and alpha-entmax is
 *                solved on that reduced set;
 *   section 4    (efficiency) full-cache entmax decode as the baseline.
 * The alpha-entmax definition is the standard Tsallis one (Peters, Niculae &
 * Martins 2019): p_i = [(alpha-1) z_i - tau]_+^(1/(alpha-1)) with tau such
 * that sum_i p_i = 1; z_i = q . k_i on the stored values (no scaling inside).
 *
 * Conventions shared by every entry point
 *  - Array arguments are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or keeps a pointer after returning.
 *  - `shape` is a HOST pointer, read during the call only.
 *  - Alignment: q, k_pool, v_pool and meta must be 16-byte aligned and the
 *    workspace 256-byte aligned (hipMalloc gives both); otherwise the call
 *    returns ENTMAXKV_ERR_INVALID.
 *  - Work is enqueued on `stream` (0 = the null stream); calls return without
 *    waiting for the GPU.
 *  - `events` (nullable) is a host array of 2*k hipEvent_t handles created by
 *    the caller; when given, events[2i] is recorded on `stream` right before
 *    the call's i-th kernel and events[2i+1] right after it. k is stated per
 *    entry point. Used for per-kernel timing.
 *  - Every argument is validated on the host before any HIP call; on error
 *    nothing is enqueued. Return codes are the ENTMAXKV_* values below.
 *  - Device-side preconditions (not checked on the host, since they live in
 *    device memory): 0 <= seq_lens[b] <= max_pages_per_seq * page_size;
 *    block_table[b, j] in [0, num_phys_pages) for j < ceil(seq_lens[b] /
 *    page_size). Kernels clamp seq_lens into that range and treat a block
 *    table entry outside it as an empty page, so bad values give wrong
 *    results, never out-of-bounds accesses.
 *  - The library keeps no state between calls (apart from each kernel's
 *    LDS limit, raised once on its first launch) and is safe to call from
 *    several host threads (each call uses only its own arguments).
 *
 * Layouts (row-major, all dense):
 *   q            float32 [batch, num_q_heads, head_dim]
 *   k_pool,
 *   v_pool       kv_dtype [num_phys_pages, num_kv_heads, page_size, head_dim]
 *                (one (page, KV head) is a contiguous page_size*head_dim block)
 *   block_table  int32 [batch, max_pages_per_seq]: logical page j of sequence
 *                b lives in physical page block_table[b, j]
 *   seq_lens     int32 [batch]: tokens of sequence b are t < seq_lens[b];
 *                token t is row t % page_size of logical page t / page_size
 *   meta         kv_dtype [num_phys_pages, num_kv_heads, 2, head_dim]:
 *                [..., 0, :] = k_min, [..., 1, :] = k_max of the page's
 *                valid keys
 *   sel          int32 [batch, num_q_heads, budget_pages]: selected logical
 *                pages, strictly ascending, then -1 padding
 *   out          float32 [batch, num_q_heads, head_dim]
 *   tau          float32 [batch, num_q_heads] (nullable)
 *   support      int32 [batch, num_q_heads] (nullable)
 * Query head h uses KV head h / (num_q_heads / num_kv_heads).
 *
 * Supported: head_dim in {64, 128}; page_size in {16, 32, 64};
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}; kv_dtype F32 or BF16;
 * max_pages_per_seq <= 262144; num_phys_pages * page_size < 2^31. Anything
 * else returns ENTMAXKV_ERR_UNSUPPORTED.
 */
#ifndef ENTMAXKV_H
#define ENTMAXKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ENTMAXKV_OK = 0,
  ENTMAXKV_ERR_INVALID = -1,     /* null or misaligned pointer, non-positive size,
                                    H % H_kv != 0, budget <= 0, alpha <= 1 or not
                                    finite */
  ENTMAXKV_ERR_UNSUPPORTED = -2, /* head_dim, page_size, group size, dtype or size
                                    outside the supported set */
  ENTMAXKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  ENTMAXKV_ERR_HIP = -4          /* a HIP launch or event record failed */
};

typedef enum { ENTMAXKV_F32 = 0, ENTMAXKV_BF16 = 1 } entmaxkv_dtype;

typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_phys_pages;
  int32_t kv_dtype; /* entmaxkv_dtype */
} entmaxkv_shape;

/* Which call a workspace is for (entmaxkv_workspace_bytes). */
enum {
  ENTMAXKV_WS_SELECT = 0,
  ENTMAXKV_WS_SPARSE = 1,
  ENTMAXKV_WS_FULL = 2,
  ENTMAXKV_WS_GAUSS = 3,
  ENTMAXKV_WS_TOPK = 4
};

/*
 * Page bounding boxes ([EntmaxKV page] section 2.A): for every logical page
 * j < ceil(seq_lens[b]/page_size) of every sequence, writes the coordinate-
 * wise min and max of its valid keys (rows t < seq_lens[b]) for each KV head
 * to meta[block_table[b, j]]. min/max is exact, so meta holds stored key
 * values (a zero may come out as -0 or +0). Pages not referenced are left
 * untouched. A physical page listed by several sequences (a shared prefix)
 * must hold the same valid rows in each; otherwise the box it ends up with
 * is one of theirs. Kernels launched: 1.
 */
int entmaxkv_build_page_meta(const entmaxkv_shape* shape, const void* k_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             void* meta, hipStream_t stream, hipEvent_t* events);

/*
 * Page boxes after an append ([EntmaxKV page] section 2.A: the boxes are
 * per-page state that a decode loop keeps current as tokens arrive). The
 * caller has written the keys of tokens old_lens[b] <= t < new_lens[b] of
 * each sequence into k_pool (their pages already in block_table). For every
 * page holding such a token, the box becomes the min/max of its valid keys
 * t < new_lens[b]: a page whose first row is new is rebuilt from its rows; a
 * page that already held tokens combines its current box (which must be the
 * box of its rows below old_lens[b]) with the new rows. The result equals
 * entmaxkv_build_page_meta with seq_lens = new_lens on those pages (bit for
 * bit up to the sign of a zero); no other page is touched.
 *   old_lens, new_lens  int32 [batch] device arrays
 *   max_new_tokens      host int >= 1, at least new_lens[b] - old_lens[b] for
 *                       every b; it sizes the grid (pages beyond
 *                       ceil(max_new_tokens / page_size) + 1 per sequence are
 *                       not updated)
 * A sequence with new_lens[b] <= old_lens[b] is left as it is. Returns
 * ENTMAXKV_ERR_INVALID for a null pointer or max_new_tokens < 1. Kernels
 * launched: 1.
 */
int entmaxkv_append_page_meta(const entmaxkv_shape* shape, const void* k_pool,
                              const int32_t* block_table, const int32_t* old_lens,
                              const int32_t* new_lens, int32_t max_new_tokens, void* meta,
                              hipStream_t stream, hipEvent_t* events);

/*
 * Page key moments ([EntmaxKV page] section 2.A, the Gaussian statistics):
 * for every logical page j < ceil(seq_lens[b]/page_size) of every sequence
 * and each KV head, the per-coordinate mean and population variance (divisor
 * n, the page's valid rows t < seq_lens[b]) of the page's keys, written to
 *     moments[block_table[b, j], g, 0, :]  (mean)
 *     moments[block_table[b, j], g, 1, :]  (variance)
 * moments: kv_dtype [num_phys_pages, num_kv_heads, 2, head_dim] (the layout
 * of meta). Sums in float64, rounded to float32 and then to the cache dtype
 * (each to nearest even). Pages not referenced are left untouched. Returns
 * ENTMAXKV_ERR_INVALID for a null or misaligned pointer. Kernels launched: 1.
 */
int entmaxkv_build_page_moments(const entmaxkv_shape* shape, const void* k_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                void* moments, hipStream_t stream, hipEvent_t* events);

/*
 * Page key moments after an append (the statistics of [EntmaxKV page]
 * section 2.A kept current by a decode loop, like the boxes). The caller has
 * written the keys of tokens old_lens[b] <= t < new_lens[b] into k_pool. Every
 * page holding such a token is recomputed from all its valid rows t <
 * new_lens[b] (stored moments are rounded, so they are not updated in
 * place): the result on those pages is bit for bit that of
 * entmaxkv_build_page_moments with seq_lens = new_lens, and no other page is
 * touched. Arguments as for entmaxkv_append_page_meta (max_new_tokens >= 1,
 * at least every new_lens[b] - old_lens[b]; pages beyond
 * ceil(max_new_tokens / page_size) + 1 per sequence are not updated; a
 * sequence with new_lens[b] <= old_lens[b] is left as it is). Returns
 * ENTMAXKV_ERR_INVALID for a null or misaligned pointer or max_new_tokens < 1.
 * Kernels launched: 1.
 */
int entmaxkv_append_page_moments(const entmaxkv_shape* shape, const void* k_pool,
                                 const int32_t* block_table, const int32_t* old_lens,
                                 const int32_t* new_lens, int32_t max_new_tokens, void* moments,
                                 hipStream_t stream, hipEvent_t* events);

/*
 * Gaussian-aware entmax page selection ([EntmaxKV page] section 2.B, policy
 * 2). The page states the policy, not its formulas; this is one reading. For
 * each (b, h), with m = 1/(alpha-1), pages j < P_b and n_j their valid rows:
 *   mu_j = (alpha-1) q . mean_j,   s_j = (alpha-1) sqrt(sum_d q_d^2 var_j,d)
 *   (a page's token scores, in the units of tau, taken as N(mu_j, s_j^2));
 *   tau_hat solves  sum_j n_j E[(A_j - t)_+^m] = 1,  A_j ~ N(mu_j, s_j^2)
 *   (closed forms from the normal's truncated moments; float64);
 *   est_j = mu_j + s_j sqrt(2 ln n_j)  (mu_j when n_j = 1);
 *   the pages with est_j > tau_hat - delta are kept; if more than cap_pages
 *   qualify, the cap_pages with the largest est_j rounded to float32, ties
 *   to the lower j. Written ascending to sel[b, h, 0:cap_pages], -1 after.
 * alpha must be 2, 3/2, 4/3 or 5/4 (1/(alpha-1) within 1e-4 of 1..4; else
 * ENTMAXKV_ERR_UNSUPPORTED); delta >= 0 and finite, in the units of tau
 * (else ENTMAXKV_ERR_INVALID); cap_pages > 0. moments is the output of
 * entmaxkv_build_page_moments. tau_hat (nullable, float32 [batch,
 * num_q_heads]) receives tau_hat (NaN for an empty sequence). The selection
 * feeds entmaxkv_decode_sparse with budget_pages = cap_pages.
 * Workspace: entmaxkv_workspace_bytes(..., ENTMAXKV_WS_GAUSS).
 * Kernels launched: 2 (page statistics; tau_hat, keys and the capped select).
 */
int entmaxkv_gauss_select(const entmaxkv_shape* shape, const float* q, const void* moments,
                          const int32_t* block_table, const int32_t* seq_lens, float alpha,
                          float delta, int32_t cap_pages, int32_t* sel, float* tau_hat,
                          void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * Page bounds and fixed-budget top-k ([EntmaxKV page] sections 2.A and 2.B
 * policy 1). For each (b, h) and logical page j < P_b = ceil(seq_lens[b] /
 * page_size):
 *     ub[j] = fp32( sum_d max(q_d * kmin_d, q_d * kmax_d) )   (then -0 -> +0)
 * the maximum of q.k over the page's box. Every product is exact; the sum is
 * taken in float64 and rounded once to float32 for F32 boxes, and
 * accumulated in float32 on the matrix cores for BF16 boxes (q split exactly
 * into three bf16 parts; the bound then differs from the exactly rounded
 * sum by float32 accumulation error, about 1e-7 relative). A page whose
 * block-table entry is outside [0, num_phys_pages) gets ub = -inf. Selects
 * the budget_pages pages with the largest ub, ties to the lower j, written
 * ascending to sel[b, h, :]; if P_b <= budget_pages every page is kept.
 * Unused slots are -1.
 * sel_ub (nullable, float32 [batch, num_q_heads, budget_pages]) receives the
 * ub of each kept page (-inf in unused slots).
 * Workspace: entmaxkv_workspace_bytes(..., ENTMAXKV_WS_SELECT).
 * Kernels launched: 2 (bounds, select).
 */
int entmaxkv_score_select(const entmaxkv_shape* shape, const float* q, const void* meta,
                          const int32_t* block_table, const int32_t* seq_lens,
                          int32_t budget_pages, int32_t* sel, float* sel_ub, void* ws,
                          size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * entmaxkv_score_select without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same kernels, arguments and
 * results as entmaxkv_score_select (bit for bit); the per-head bounds go to
 * a file-scope device array of 16 MiB that the library holds on every GPU
 * it runs on until the process ends. The call allocates and frees nothing.
 * Limit: batch * num_q_heads * (max_pages_per_seq rounded up to a multiple
 * of 4) * 4 bytes <= 16 MiB (e.g. 128 heads x 32768 pages); beyond it the
 * call returns ENTMAXKV_ERR_WORKSPACE before any HIP call. All calls on one
 * GPU share that array: calls that overlap in time on one GPU (several
 * streams or host threads) race and must be serialized by the caller.
 * Kernels launched: 2 (bounds, select).
 */
int entmaxkv_score_select_noalloc(const entmaxkv_shape* shape, const float* q, const void* meta,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t budget_pages, int32_t* sel, float* sel_ub,
                                  hipStream_t stream, hipEvent_t* events);

/*
 * Sparse alpha-entmax decode ([EntmaxKV page] section 2.C). For each (b, h),
 * gathers the valid tokens of the pages listed in sel[b, h, :] (entries < 0
 * or >= P_b are ignored), computes z = q . k in float32 (float64 for F32
 * caches), solves tau over those tokens only, and writes
 *     out[b, h, :] = sum_i p_i v_i / sum_i p_i,  p_i = [(alpha-1) z_i - tau]_+^m
 * (m = 1/(alpha-1); dividing by sum p, which is 1 up to rounding, keeps the
 * output a convex combination). Only V rows with p_i > 0 are read. tau is in
 * the (alpha-1) z units; support = #{p_i > 0}. A head with no tokens gets
 * out = 0, tau = NaN, support = 0. The pages of the num_q_heads/num_kv_heads
 * heads sharing a KV head are read once per call (their union).
 * Workspace: entmaxkv_workspace_bytes(..., ENTMAXKV_WS_SPARSE) for the same
 * budget_pages. Kernels launched: 2 (gather-score, threshold + P.V).
 */
int entmaxkv_decode_sparse(const entmaxkv_shape* shape, const float* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* sel, int32_t budget_pages,
                           float alpha, float* out, float* tau, int32_t* support, void* ws,
                           size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * Page bounds, top-k selection and sparse decode in one call ([EntmaxKV page]
 * sections 2.A, 2.B policy 1 and 2.C): the same results as
 * entmaxkv_score_select (sel, sel_ub) followed by entmaxkv_decode_sparse on
 * that selection (out, tau, support; every score and sum computed the same
 * way, so equal up to the order of the threshold solve's float64 sums).
 * sel is required; sel_ub, tau and support are nullable.
 * With bf16 caches, at least 128 query heads in the batch (batch *
 * num_q_heads), budget_pages <= 1024 and at most 2 MiB of selected keys per
 * head (512 KiB beyond 256 heads), it runs two kernels: the bounds, then one
 * workgroup per query head that selects the head's pages, gathers and
 * scores them, solves tau and writes the output (no candidate crosses a
 * workgroup). With bf16 caches, fewer than 128 heads and budget_pages <=
 * 1024, it runs three: the bounds, several workgroups per head that each
 * select the head's pages and gather and score a share of them, and the
 * threshold kernel. Otherwise the four kernels of the two calls run.
 * Workspace: entmaxkv_workspace_bytes(..., ENTMAXKV_WS_TOPK) for the same
 * budget_pages. events (nullable): 2*4 handles; pairs 0 and 1 enclose the
 * bounds and the select (or the per-head kernel), pairs 2 and 3 the sparse
 * decode's two kernels (on the per-head path pair 2 encloses the threshold
 * kernel of the split form, else nothing, and pair 3 nothing).
 */
int entmaxkv_decode_topk(const entmaxkv_shape* shape, const float* q, const void* meta,
                         const void* k_pool, const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t budget_pages, float alpha,
                         int32_t* sel, float* sel_ub, float* out, float* tau, int32_t* support,
                         void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * Number of kernels entmaxkv_decode_topk launches at this shape and budget:
 * 2 on the per-head path, 3 on its split form, 4 otherwise. Writes
 * *kernels; returns an error code for an invalid or unsupported shape or
 * budget.
 */
int entmaxkv_topk_kernels(const entmaxkv_shape* shape, int32_t budget_pages, int32_t* kernels);

/*
 * Full-cache alpha-entmax decode ([EntmaxKV page] section 4, the full-cache
 * entmax baseline): as entmaxkv_decode_sparse with every page of every
 * sequence selected. Workspace: entmaxkv_workspace_bytes(...,
 * ENTMAXKV_WS_FULL). Kernels launched: 2 (score, threshold + P.V).
 */
int entmaxkv_decode_full(const entmaxkv_shape* shape, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, float alpha, float* out, float* tau,
                         int32_t* support, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipEvent_t* events);

/*
 * Workspace size in bytes for `which` (ENTMAXKV_WS_*) at this shape and
 * budget (budget is ignored for ENTMAXKV_WS_FULL). Writes *bytes and returns
 * ENTMAXKV_OK, or an error code for an invalid or unsupported shape.
 */
int entmaxkv_workspace_bytes(const entmaxkv_shape* shape, int32_t budget_pages, int32_t which,
                             size_t* bytes);

/* Static description of a return code; never NULL. */
const char* entmaxkv_strerror(int code);

/* Library version as major*10000 + minor*100 + patch. */
int entmaxkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAXKV_H */
