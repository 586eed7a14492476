// C ABI of the EntmaxKV-style decode library: host-side validation,
// workspace planning and kernel dispatch. Every check runs before the first
// HIP call, so a rejected call enqueues nothing.
#include <math.h>

#include <mutex>

#include "entmaxkv.h"
#include "launch.hpp"

using namespace ekv;

namespace {

// Scratch memory of entmaxkv_score_select_noalloc: the per-head page bounds
// that entmaxkv_score_select keeps in the caller's workspace. A file-scope
// device array, so the call allocates nothing; every GPU the library runs on
// holds its own copy until the process ends. Host code uses the address
// hipGetSymbolAddress reports for the current device, never the array's
// name (a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ENTMAXKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ENTMAXKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ENTMAXKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ENTMAXKV_OK;
}

constexpr int kMaxPagesPerSeq = 262144;
constexpr size_t kMaxScoreLds = kMaxScoreLdsBytes;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Kernels use 16-byte vector loads of q, the pools and the box metadata, and
// carve the workspace into 256-byte aligned pieces.
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(const entmaxkv_shape* s, LaunchShape* out) {
  if (!s) return ENTMAXKV_ERR_INVALID;
  if (s->batch <= 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->head_dim <= 0 ||
      s->page_size <= 0 || s->max_pages_per_seq <= 0 || s->num_phys_pages <= 0)
    return ENTMAXKV_ERR_INVALID;
  if (s->num_q_heads % s->num_kv_heads != 0) return ENTMAXKV_ERR_INVALID;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ENTMAXKV_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return ENTMAXKV_ERR_UNSUPPORTED;
  if (s->page_size != 16 && s->page_size != 32 && s->page_size != 64)
    return ENTMAXKV_ERR_UNSUPPORTED;
  if (s->kv_dtype != ENTMAXKV_F32 && s->kv_dtype != ENTMAXKV_BF16)
    return ENTMAXKV_ERR_UNSUPPORTED;
  if (s->max_pages_per_seq > kMaxPagesPerSeq) return ENTMAXKV_ERR_UNSUPPORTED;
  // a candidate token is named by its V row, physical_page * page_size + row
  if ((long long)s->num_phys_pages * s->page_size > 0x7fffffffLL) return ENTMAXKV_ERR_UNSUPPORTED;
  // grid sizes stay far below 2^31 blocks and byte offsets fit 64 bits
  if ((long long)s->batch * s->num_q_heads > (1LL << 24)) return ENTMAXKV_ERR_UNSUPPORTED;
  if (out) {
    out->batch = s->batch;
    out->num_q_heads = s->num_q_heads;
    out->num_kv_heads = s->num_kv_heads;
    out->head_dim = s->head_dim;
    out->page_size = s->page_size;
    out->max_pages = s->max_pages_per_seq;
    out->num_phys = s->num_phys_pages;
    out->group = G;
    out->bf16 = s->kv_dtype == ENTMAXKV_BF16;
  }
  return ENTMAXKV_OK;
}

int check_alpha(float alpha) {
  if (!isfinite(alpha) || !(alpha > 1.0f)) return ENTMAXKV_ERR_INVALID;
  return ENTMAXKV_OK;
}

int check_budget(int32_t budget) {
  if (budget <= 0) return ENTMAXKV_ERR_INVALID;
  if (budget > (1 << 22)) return ENTMAXKV_ERR_UNSUPPORTED;
  return ENTMAXKV_OK;
}

// Width (in z units) of the window that holds every token of the support,
// 1/(alpha-1), widened slightly so float32 rounding of z never drops one.
float window_of(float alpha) {
  const double w = 1.0 / ((double)alpha - 1.0);
  return (float)(w * (1.0 + 1e-6) + 1e-3);
}

int score_lds_ok(const LaunchShape& s, const SplitPlan& p, bool sparse, int budget) {
  const size_t total = score_lds_layout(s.group, s.page_size, p.pages_per_split, sparse,
                                        s.max_pages, budget, score_bytes(s.bf16),
                                        score_kbuf_bytes(s.bf16, s.group, s.page_size, s.head_dim, sparse),
                                        s.head_dim)
                           .total;
  return total <= kMaxScoreLds ? ENTMAXKV_OK : ENTMAXKV_ERR_UNSUPPORTED;
}

struct Events {
  hipEvent_t* ev;
  hipStream_t st;
  bool before(int i) const { return !ev || hipEventRecord(ev[2 * i], st) == hipSuccess; }
  bool after(int i) const { return !ev || hipEventRecord(ev[2 * i + 1], st) == hipSuccess; }
};

}  // namespace

namespace ekv {

// Largest pages-per-workgroup, at most `pps`, whose score-kernel LDS (per-wave
// candidate lists sized for every token of the split) fits; wide heads with
// float32 caches and many heads per KV head need shorter splits.
static int fit_pps(const LaunchShape& s, int pps, bool sparse, int budget) {
  while (pps > 1 && score_lds_layout(s.group, s.page_size, pps, sparse, s.max_pages, budget,
                                     score_bytes(s.bf16),
                                     score_kbuf_bytes(s.bf16, s.group, s.page_size, s.head_dim, sparse),
                                     s.head_dim)
                            .total > kMaxScoreLds)
    pps /= 2;
  return pps;
}

// One candidate region per (head, workgroup); their count per head is capped
// by the threshold kernel's LDS.
static SplitPlan finish_plan(const LaunchShape& s, long long pages, int pps) {
  SplitPlan p;
  const long long need = (pages + kMaxSplits - 1) / kMaxSplits;
  if (pps < need) pps = (int)need;
  p.pages_per_split = pps;
  p.splits = (int)((pages + pps - 1) / pps);
  if (p.splits < 1) p.splits = 1;
  p.cap = pps * s.page_size;
  p.regions = p.splits;
  p.rcap = p.cap;
  return p;
}

SplitPlan plan_sparse(const LaunchShape& s, int budget) {
  const int keep = budget < s.max_pages ? budget : s.max_pages;
  long long umax = (long long)s.group * keep;
  if (umax > s.max_pages) umax = s.max_pages;
  const long long units = (long long)s.batch * s.num_kv_heads;
  const long long page_bytes = (long long)s.page_size * s.head_dim * (s.bf16 ? 2 : 4);
  const auto grid = [&](long long n) { return units * ((umax + n - 1) / n); };
  long long pps = kSparseSplitBytes / page_bytes;
  if (pps < 1) pps = 1;
  while (pps > 1 && grid(pps) < kSparseMinGrid) pps /= 2;
  while (2 * pps * s.page_size <= kSparseMaxTokensPerSplit && pps < umax &&
         grid(pps) >= kSparseMaxGrid)
    pps *= 2;
  pps = fit_pps(s, (int)pps, true, budget);
  SplitPlan p = finish_plan(s, umax, pps);
  p.list_cap = keep * s.page_size;
  return p;
}

SplitPlan plan_full(const LaunchShape& s) {
  int pps = kFullTokensPerSplit / s.page_size;
  if (pps < 1) pps = 1;
  // short caches: halve the split while the grid would be under kFullMinGrid
  const long long units = (long long)s.batch * s.num_kv_heads;
  while (pps > 1 && units * ((s.max_pages + pps - 1) / pps) < kFullMinGrid) pps /= 2;
  pps = fit_pps(s, pps, false, 0);
  SplitPlan p = finish_plan(s, s.max_pages, pps);
  p.list_cap = s.max_pages * s.page_size;
  return p;
}

DecodeWs decode_ws_layout(const LaunchShape& s, const SplitPlan& p) {
  DecodeWs w;
  const size_t bh = (size_t)s.batch * s.num_q_heads;
  size_t o = 0;
  const size_t zb = score_bytes(s.bf16);
  w.cand = o;
  o = align256(o + bh * p.regions * (size_t)p.rcap * cand_bytes(s.bf16));
  w.counts = o;
  o = align256(o + bh * p.regions * 4);
  w.maxima = o;
  o = align256(o + bh * p.regions * zb);
  w.list = o;
  o = align256(o + bh * (size_t)p.list_cap * (zb + 4));
  // score-kernel spill areas: one per (head, workgroup, wave), each holding
  // every token the wave streams
  const size_t wcap = (size_t)((p.pages_per_split + kNW - 1) / kNW) * s.page_size;
  w.spill = o;
  o = align256(o + bh * p.splits * (size_t)kNW * wcap * cand_bytes(s.bf16));
  // the score step's shared maxima, one order key per head, kMaxStride
  // words apart
  w.gmax = o;
  o = align256(o + bh * kMaxStride * 4);
  w.total = o;
  return w;
}

}  // namespace ekv

namespace {

// Sets the order keys m[i * kMaxStride] and m[i * kMaxStride + 1], i < n, to
// that of -inf: the start of the score step's shared maxima and shared lower
// bounds on tau.
__global__ void reset_maxima_kernel(uint32_t* m, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    m[(size_t)i * kMaxStride] = 0x007fffffu;
    m[(size_t)i * kMaxStride + 1] = 0x007fffffu;
  }
}

hipError_t launch_score(const LaunchShape& s, const SplitPlan& p, const float* q,
                        const void* k_pool, const int32_t* bt, const int32_t* lens,
                        const int32_t* sel, int budget, float alpha, float window, void* ws,
                        const DecodeWs& L, hipStream_t st) {
  return s.bf16
             ? launch_score_bf16(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st)
             : launch_score_f32(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
}

hipError_t launch_tau_pv(const LaunchShape& s, const SplitPlan& p, const void* v_pool,
                         const int32_t* bt, const int32_t* lens, const int32_t* sel, int budget,
                         float alpha, float window, float* out, float* tau, int32_t* support,
                         void* ws, const DecodeWs& L, hipStream_t st) {
  return s.bf16 ? launch_tau_pv_bf16(s, p, v_pool, bt, lens, sel, budget, alpha, window, out,
                                     tau, support, ws, L, st)
                : launch_tau_pv_f32(s, p, v_pool, bt, lens, sel, budget, alpha, window, out, tau,
                                    support, ws, L, st);
}

int decode_common(const entmaxkv_shape* shape, const float* q, const void* k_pool,
                  const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* sel, int32_t budget, float alpha, float* out, float* tau,
                  int32_t* support, void* ws, size_t ws_bytes, hipStream_t stream,
                  hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  const bool sparse = sel != nullptr;
  if (sparse && (rc = check_budget(budget))) return rc;
  if ((rc = check_alpha(alpha))) return rc;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out) return ENTMAXKV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return ENTMAXKV_ERR_INVALID;
  const SplitPlan p = sparse ? plan_sparse(s, budget) : plan_full(s);
  if ((rc = score_lds_ok(s, p, sparse, budget))) return rc;
  const DecodeWs L = decode_ws_layout(s, p);
  if (!ws || ws_bytes < L.total) return ENTMAXKV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return ENTMAXKV_ERR_INVALID;
  const float window = window_of(alpha);
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (score_mode(s, p, sparse, budget, window).share) {
    const int bh = s.batch * s.num_q_heads;
    hipLaunchKernelGGL(reset_maxima_kernel, dim3((unsigned)((bh + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.gmax), bh);
    if (hipGetLastError() != hipSuccess) return ENTMAXKV_ERR_HIP;
  }
  if (launch_score(s, p, q, k_pool, block_table, seq_lens, sel, budget, alpha, window, ws, L,
                   stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0) || !ev.before(1)) return ENTMAXKV_ERR_HIP;
  if (launch_tau_pv(s, p, v_pool, block_table, seq_lens, sel, budget, alpha, window, out, tau,
                    support, ws, L, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(1)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

// Workspace of entmaxkv_decode_topk: the per-head path (bounds, then the
// per-head kernel's spill areas and lists), or the select workspace followed
// by the sparse decode's.
struct TopkWs {
  HeadPlan head;
  SplitPlan split;
  DecodeWs dec;
  size_t dec_off = 0, total = 0;
};
int topk_ws(const LaunchShape& s, int budget, TopkWs* w) {
  const size_t sel_bytes = align256(select_ws_bytes(s, budget));
  w->head = plan_head(s, budget, sel_bytes);
  if (w->head.use) {
    w->total = w->head.total;
    return ENTMAXKV_OK;
  }
  w->split = plan_sparse(s, budget);
  if (int rc = score_lds_ok(s, w->split, true, budget)) return rc;
  w->dec = decode_ws_layout(s, w->split);
  w->dec_off = sel_bytes;
  w->total = sel_bytes + w->dec.total;
  return ENTMAXKV_OK;
}

}  // namespace

extern "C" {

int entmaxkv_version(void) { return 100; }

const char* entmaxkv_strerror(int code) {
  switch (code) {
    case ENTMAXKV_OK: return "ok";
    case ENTMAXKV_ERR_INVALID: return "invalid argument";
    case ENTMAXKV_ERR_UNSUPPORTED: return "unsupported shape, dtype or size";
    case ENTMAXKV_ERR_WORKSPACE: return "workspace missing or too small";
    case ENTMAXKV_ERR_HIP: return "HIP launch or event error";
    default: return "unknown error code";
  }
}

int entmaxkv_workspace_bytes(const entmaxkv_shape* shape, int32_t budget_pages, int32_t which,
                             size_t* bytes) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if (!bytes) return ENTMAXKV_ERR_INVALID;
  switch (which) {
    case ENTMAXKV_WS_SELECT:
      if ((rc = check_budget(budget_pages))) return rc;
      *bytes = align256(select_ws_bytes(s, budget_pages));
      return ENTMAXKV_OK;
    case ENTMAXKV_WS_SPARSE: {
      if ((rc = check_budget(budget_pages))) return rc;
      const SplitPlan p = plan_sparse(s, budget_pages);
      if ((rc = score_lds_ok(s, p, true, budget_pages))) return rc;
      *bytes = decode_ws_layout(s, p).total;
      return ENTMAXKV_OK;
    }
    case ENTMAXKV_WS_FULL: {
      const SplitPlan p = plan_full(s);
      if ((rc = score_lds_ok(s, p, false, 0))) return rc;
      *bytes = decode_ws_layout(s, p).total;
      return ENTMAXKV_OK;
    }
    case ENTMAXKV_WS_GAUSS:
      if ((rc = check_budget(budget_pages))) return rc;
      *bytes = align256(gauss_ws_bytes(s));
      return ENTMAXKV_OK;
    case ENTMAXKV_WS_TOPK: {
      if ((rc = check_budget(budget_pages))) return rc;
      TopkWs w;
      if ((rc = topk_ws(s, budget_pages, &w))) return rc;
      *bytes = w.total;
      return ENTMAXKV_OK;
    }
    default:
      return ENTMAXKV_ERR_INVALID;
  }
}

int entmaxkv_build_page_meta(const entmaxkv_shape* shape, const void* k_pool,
                             const int32_t* block_table, const int32_t* seq_lens, void* meta,
                             hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if (!k_pool || !block_table || !seq_lens || !meta) return ENTMAXKV_ERR_INVALID;
  if (!aligned(k_pool, 16) || !aligned(meta, 16)) return ENTMAXKV_ERR_INVALID;
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_meta(s, k_pool, block_table, seq_lens, meta, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_build_page_moments(const entmaxkv_shape* shape, const void* k_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                void* moments, hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if (!k_pool || !block_table || !seq_lens || !moments) return ENTMAXKV_ERR_INVALID;
  if (!aligned(k_pool, 16) || !aligned(moments, 16)) return ENTMAXKV_ERR_INVALID;
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_moments(s, k_pool, block_table, nullptr, seq_lens, 0, moments, stream) !=
      hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_append_page_moments(const entmaxkv_shape* shape, const void* k_pool,
                                 const int32_t* block_table, const int32_t* old_lens,
                                 const int32_t* new_lens, int32_t max_new_tokens, void* moments,
                                 hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if (!k_pool || !block_table || !old_lens || !new_lens || !moments) return ENTMAXKV_ERR_INVALID;
  if (max_new_tokens <= 0) return ENTMAXKV_ERR_INVALID;
  if (!aligned(k_pool, 16) || !aligned(moments, 16)) return ENTMAXKV_ERR_INVALID;
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_moments(s, k_pool, block_table, old_lens, new_lens, max_new_tokens, moments,
                     stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_gauss_select(const entmaxkv_shape* shape, const float* q, const void* moments,
                          const int32_t* block_table, const int32_t* seq_lens, float alpha,
                          float delta, int32_t cap_pages, int32_t* sel, float* tau_hat,
                          void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if ((rc = check_budget(cap_pages))) return rc;
  if ((rc = check_alpha(alpha))) return rc;
  if (!isfinite(delta) || !(delta >= 0.0f)) return ENTMAXKV_ERR_INVALID;
  // m = 1/(alpha-1) must be an integer 1..4 (alpha 2, 3/2, 4/3, 5/4)
  const double am1 = (double)alpha - 1.0;
  const double mr = 1.0 / am1;
  const int m = (int)lround(mr);
  if (m < 1 || m > 4 || fabs(mr - m) > 1e-4) return ENTMAXKV_ERR_UNSUPPORTED;
  if (!q || !moments || !block_table || !seq_lens || !sel) return ENTMAXKV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(moments, 16)) return ENTMAXKV_ERR_INVALID;
  if (!ws || ws_bytes < gauss_ws_bytes(s)) return ENTMAXKV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return ENTMAXKV_ERR_INVALID;
  const size_t rows = (size_t)s.batch * s.num_q_heads * ub_ld(s.max_pages);
  void* stats = ws;
  float* keys = reinterpret_cast<float*>(static_cast<char*>(ws) + ((rows * 16 + 255) & ~(size_t)255));
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_gauss_stats(s, q, moments, block_table, seq_lens, am1, stats, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0) || !ev.before(1)) return ENTMAXKV_ERR_HIP;
  if (launch_gauss_solve(s, stats, seq_lens, m, (double)delta, keys, tau_hat, cap_pages, sel,
                         stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(1)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_append_page_meta(const entmaxkv_shape* shape, const void* k_pool,
                              const int32_t* block_table, const int32_t* old_lens,
                              const int32_t* new_lens, int32_t max_new_tokens, void* meta,
                              hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if (!k_pool || !block_table || !old_lens || !new_lens || !meta) return ENTMAXKV_ERR_INVALID;
  if (max_new_tokens <= 0) return ENTMAXKV_ERR_INVALID;
  if (!aligned(k_pool, 16) || !aligned(meta, 16)) return ENTMAXKV_ERR_INVALID;
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_append_meta(s, k_pool, block_table, old_lens, new_lens, max_new_tokens, meta,
                         stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_score_select(const entmaxkv_shape* shape, const float* q, const void* meta,
                          const int32_t* block_table, const int32_t* seq_lens,
                          int32_t budget_pages, int32_t* sel, float* sel_ub, void* ws,
                          size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if ((rc = check_budget(budget_pages))) return rc;
  if (!q || !meta || !block_table || !seq_lens || !sel) return ENTMAXKV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(meta, 16)) return ENTMAXKV_ERR_INVALID;
  if (!ws || ws_bytes < select_ws_bytes(s, budget_pages)) return ENTMAXKV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return ENTMAXKV_ERR_INVALID;
  float* ub = static_cast<float*>(ws);
  const SelectPlan sp = plan_select(s, budget_pages);
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_bounds(s, sp, q, meta, block_table, seq_lens, ub, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0) || !ev.before(1)) return ENTMAXKV_ERR_HIP;
  if (launch_select(s, sp, ub, seq_lens, budget_pages, sel, sel_ub, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(1)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_score_select_noalloc(const entmaxkv_shape* shape, const float* q, const void* meta,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t budget_pages, int32_t* sel, float* sel_ub,
                                  hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if ((rc = check_budget(budget_pages))) return rc;
  if (!q || !meta || !block_table || !seq_lens || !sel) return ENTMAXKV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(meta, 16)) return ENTMAXKV_ERR_INVALID;
  if (select_ws_bytes(s, budget_pages) > kNoAllocScratchBytes) return ENTMAXKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  // the same kernels as entmaxkv_score_select, with the bounds in `scratch`
  // (every bound the select reads is written first: nothing to clear)
  float* ub = static_cast<float*>(ws);
  const SelectPlan sp = plan_select(s, budget_pages);
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_bounds(s, sp, q, meta, block_table, seq_lens, ub, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0) || !ev.before(1)) return ENTMAXKV_ERR_HIP;
  if (launch_select(s, sp, ub, seq_lens, budget_pages, sel, sel_ub, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(1)) return ENTMAXKV_ERR_HIP;
  return ENTMAXKV_OK;
}

int entmaxkv_decode_sparse(const entmaxkv_shape* shape, const float* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* sel, int32_t budget_pages,
                           float alpha, float* out, float* tau, int32_t* support, void* ws,
                           size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  if (!sel) return ENTMAXKV_ERR_INVALID;
  return decode_common(shape, q, k_pool, v_pool, block_table, seq_lens, sel, budget_pages, alpha,
                       out, tau, support, ws, ws_bytes, stream, events);
}

int entmaxkv_decode_topk(const entmaxkv_shape* shape, const float* q, const void* meta,
                         const void* k_pool, const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t budget_pages, float alpha,
                         int32_t* sel, float* sel_ub, float* out, float* tau, int32_t* support,
                         void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if ((rc = check_budget(budget_pages))) return rc;
  if ((rc = check_alpha(alpha))) return rc;
  if (!q || !meta || !k_pool || !v_pool || !block_table || !seq_lens || !sel || !out)
    return ENTMAXKV_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(meta, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return ENTMAXKV_ERR_INVALID;
  TopkWs w;
  if ((rc = topk_ws(s, budget_pages, &w))) return rc;
  if (!ws || ws_bytes < w.total) return ENTMAXKV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return ENTMAXKV_ERR_INVALID;
  float* ub = static_cast<float*>(ws);
  const SelectPlan sp = plan_select(s, budget_pages);
  const float window = window_of(alpha);
  const Events ev{events, stream};
  if (!ev.before(0)) return ENTMAXKV_ERR_HIP;
  if (launch_bounds(s, sp, q, meta, block_table, seq_lens, ub, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(0) || !ev.before(1)) return ENTMAXKV_ERR_HIP;
  if (w.head.use) {
    const bool bt_lds = s.max_pages % 4 == 0 && aligned(block_table, 16);
    if (launch_head_decode(s, sp, w.head, q, k_pool, v_pool, block_table, seq_lens, budget_pages,
                           alpha, window, sel, sel_ub, out, tau, support, ws, bt_lds,
                           stream) != hipSuccess)
      return ENTMAXKV_ERR_HIP;
    if (!ev.after(1) || !ev.before(2)) return ENTMAXKV_ERR_HIP;
    if (w.head.splits > 1 &&
        launch_tau_pv(s, w.head.tp, v_pool, block_table, seq_lens, sel, budget_pages, alpha,
                      window, out, tau, support, static_cast<char*>(ws) + w.head.dec, w.head.tws,
                      stream) != hipSuccess)
      return ENTMAXKV_ERR_HIP;
    // pair 3 (and pair 2 without splits) encloses nothing on this path
    if (!ev.after(2) || !ev.before(3) || !ev.after(3)) return ENTMAXKV_ERR_HIP;
    return ENTMAXKV_OK;
  }
  if (launch_select(s, sp, ub, seq_lens, budget_pages, sel, sel_ub, stream) != hipSuccess)
    return ENTMAXKV_ERR_HIP;
  if (!ev.after(1)) return ENTMAXKV_ERR_HIP;
  return decode_common(shape, q, k_pool, v_pool, block_table, seq_lens, sel, budget_pages, alpha,
                       out, tau, support, static_cast<char*>(ws) + w.dec_off,
                       ws_bytes - w.dec_off, stream, events ? events + 4 : nullptr);
}

int entmaxkv_topk_kernels(const entmaxkv_shape* shape, int32_t budget_pages, int32_t* kernels) {
  LaunchShape s;
  int rc = check_shape(shape, &s);
  if (rc) return rc;
  if ((rc = check_budget(budget_pages))) return rc;
  if (!kernels) return ENTMAXKV_ERR_INVALID;
  TopkWs w;
  if ((rc = topk_ws(s, budget_pages, &w))) return rc;
  *kernels = w.head.use ? (w.head.splits > 1 ? 3 : 2) : 4;
  return ENTMAXKV_OK;
}

int entmaxkv_decode_full(const entmaxkv_shape* shape, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, float alpha, float* out, float* tau,
                         int32_t* support, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipEvent_t* events) {
  return decode_common(shape, q, k_pool, v_pool, block_table, seq_lens, nullptr, 0, alpha, out,
                       tau, support, ws, ws_bytes, stream, events);
}

}  // extern "C"
