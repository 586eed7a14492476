// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace ekv {

constexpr int kNumCUs = 256;  // compute units of the MI355X

struct LaunchShape {
  int batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages, num_phys;
  int group;  // num_q_heads / num_kv_heads
  bool bf16;
};

// Work of one workgroup of the gather-score kernels. Full cache: 4096 tokens
// (measured against 1024, 2048 and 8192 on the 64K-1M workloads), halved
// while the grid would have fewer than kFullMinGrid workgroups. Sparse: about kSparseSplitBytes of K, halved while the grid
// would have fewer than kSparseMinGrid workgroups (short selections: more,
// smaller splits keep the chip busy) and doubled, up to
// kSparseMaxTokensPerSplit tokens, while it would have kSparseMaxGrid or
// more (long selections: each workgroup's fixed cost is spread over more
// pages).
constexpr int kFullTokensPerSplit = 4096;
constexpr long long kFullMinGrid = 512;  // full-cache splits halve below this many workgroups
constexpr int kSparseMaxTokensPerSplit = 2048;
constexpr long long kSparseSplitBytes = 256 * 1024;
constexpr long long kSparseMinGrid = 512;
constexpr long long kSparseMaxGrid = 2048;
constexpr int kMaxSplits = 4096;  // candidate regions per head (LDS-sized in the threshold kernel)

constexpr int kNT = 256;
constexpr int kScoreChunks = 2;  // 16-byte K chunks per lane and token row in the score kernel
constexpr bool kMfmaScores = true;  // bf16 caches: q.k on the matrix cores
constexpr int kNW = kNT / kWave;
constexpr int kListCap = 4096;  // threshold list entries held in LDS
constexpr int kSupCap = 4096;   // support entries held in LDS
constexpr int kRegList = 4;     // list entries per lane kept in registers by the threshold solve
constexpr int kRegListLong = 16;  // the same, for lists of up to 1024 entries (one wave, no
                                  // barriers; twice as many per lane up to 2048)
constexpr int kSelCopy = 8192;  // selection ints staged in LDS by the sparse score kernel


constexpr int kListSlots = 64;  // LDS candidate slots per (wave, head) in the score kernel
// Full cache with a window of at least kWideWindow score units (alpha of
// 4/3 or less): on flat scores about a tenth of a split's tokens survive a
// workgroup's own running maximum. The lists then get kListSlotsWide slots
// where that keeps as many workgroups on a CU, and where at least
// kShareMinWgs workgroups share a CU (enough to hide two more memory round
// trips per workgroup) and the grid takes two or more rounds of them (so
// that later workgroups start from earlier ones' maxima) each head's
// maximum is shared across the call's workgroups, one entry per kMaxStride
// words (its own 128-byte line).
constexpr int kListSlotsWide = 128;
constexpr float kWideWindow = 3.0f;
constexpr int kMaxStride = 32;
constexpr int kShareMinWgs = 3;
constexpr size_t kLdsPerCU = 160 * 1024;
constexpr int kPassRegs = 4;    // candidates per lane read at once by the score kernel's final pass
constexpr size_t kMaxScoreLdsBytes = 150 * 1024;  // most LDS a score-kernel plan may use

// LDS layout of the score kernel (bytes), shared by host sizing and device carving.
struct ScoreLds {
  int wcap;  // candidates one wave can produce per head: every token of its pages
  int slots;  // LDS candidate slots per (wave, head)
  size_t kbuf, qtab, rz, ri, wcnt, slice, slot, phys, tmp, bitmap, ssel, total;
};

// Row pitch (bf16 values) of the split-q table of the matrix-core kernels:
// one row per (head, part), padded by 16 bytes against LDS bank conflicts.
__host__ __device__ constexpr int qtab_pitch(int k) { return k + 8; }

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Pages of K staged per wave on the matrix-core path: two (double-buffered)
// for the long full-cache slices, one for the short sparse ones, and one
// where two would leave no room for the rest of the workgroup's LDS (the
// split-q table and the G heads' candidate lists, plus 4 KiB for the slice
// tables): 8 heads of 128-dim keys in 64-token pages.
__host__ __device__ constexpr int score_kbuf_pages(bool sparse, int G, int ps, int head_dim) {
  return (sparse || (size_t)kNW * 2 * ps * head_dim * 2 + (size_t)G * 3 * qtab_pitch(head_dim) * 2 +
                            (size_t)kNW * G * kListSlots * 8 + 4096 > kMaxScoreLdsBytes)
             ? 1
             : 2;
}
// Bytes of K staging per wave on the matrix-core path, else 0.
__host__ __device__ inline int score_kbuf_bytes(bool bf16, int G, int ps, int head_dim,
                                                bool sparse) {
  return (kMfmaScores && bf16) ? score_kbuf_pages(sparse, G, ps, head_dim) * ps * head_dim * 2
                               : 0;
}

// zbytes: bytes of one score (4 for bf16 caches, 8 for float32 caches);
// kbuf_wave: score_kbuf_bytes (the matrix-core path when > 0).
__host__ __device__ inline ScoreLds score_lds_layout(int G, int ps, int pps, bool sparse,
                                                     int max_pages, int budget, int zbytes,
                                                     int kbuf_wave, int head_dim,
                                                     int slots = kListSlots) {
  ScoreLds l;
  l.wcap = ((pps + kNW - 1) / kNW) * ps;
  l.slots = slots;
  size_t o = 0;
  l.kbuf = o; o = align16(o + (size_t)kNW * kbuf_wave);
  l.qtab = o;
  if (kbuf_wave > 0) o = align16(o + (size_t)G * 3 * qtab_pitch(head_dim) * 2);
  const size_t nreg = (size_t)kNW * G * slots;
  l.rz = o; o = align16(o + nreg * zbytes);
  l.ri = o; o = align16(o + nreg * 4);
  l.wcnt = o; o = align16(o + (size_t)kNW * G * 4);
  // the page slice and per-head slots exist on the sparse path only
  l.slice = o;
  if (sparse) o = align16(o + (size_t)pps * 4);
  l.slot = o;
  if (sparse) o = align16(o + (size_t)pps * G * 4);
  l.phys = o; o = align16(o + (size_t)pps * 4);
  l.tmp = o; o = align16(o + (kNW + 2) * 4);
  l.bitmap = o;
  if (sparse) o = align16(o + (size_t)((max_pages + 31) / 32) * 4);
  l.ssel = o;
  if (sparse && (size_t)G * budget <= (size_t)kSelCopy) o = align16(o + (size_t)G * budget * 4);
  l.total = o;
  return l;
}


// Partition of one (sequence, KV head) unit's pages into workgroups, and of
// each head's candidates into regions (one per head and workgroup).
struct SplitPlan {
  int pages_per_split;  // pages one workgroup streams
  int splits;           // workgroups per unit
  int cap;              // tokens one workgroup streams per head = pages_per_split * page_size
  int regions;          // candidate regions per head
  int rcap;             // candidate slots per region (every token it covers)
  int list_cap;         // threshold-list slots per head (worst case: every gathered token)
};

SplitPlan plan_sparse(const LaunchShape& s, int budget);
SplitPlan plan_full(const LaunchShape& s);

// Workspace carve-up of the decode calls (byte offsets, 256-aligned).
struct DecodeWs {
  size_t cand, counts, maxima, list, spill, gmax, total;
};
// Scores are kept in the accumulation precision: float for bf16 caches,
// double for float32 caches. A candidate is (score, token index).
__host__ __device__ inline int score_bytes(bool bf16) { return bf16 ? 4 : 8; }
__host__ __device__ inline int cand_bytes(bool bf16) { return bf16 ? 8 : 16; }
// Candidate-list slots per (wave, head) of a score launch, and whether it
// shares each head's maximum across its workgroups (the decode then resets
// the workspace's per-head maxima before the launch); see kWideWindow.
struct ScoreMode {
  int slots = kListSlots;
  bool share = false;
};
inline ScoreMode score_mode(const LaunchShape& s, const SplitPlan& p, bool sparse, int budget,
                            float window) {
  ScoreMode m;
  if (sparse || window < kWideWindow || !(s.bf16 && kMfmaScores)) return m;
  auto lds = [&](int slots) {
    return score_lds_layout(s.group, s.page_size, p.pages_per_split, sparse, s.max_pages, budget,
                            score_bytes(s.bf16),
                            score_kbuf_bytes(s.bf16, s.group, s.page_size, s.head_dim, sparse),
                            s.head_dim, slots)
        .total;
  };
  const size_t narrow = lds(kListSlots), wide = lds(kListSlotsWide);
  if (wide <= kMaxScoreLdsBytes && kLdsPerCU / wide == kLdsPerCU / narrow)
    m.slots = kListSlotsWide;
  const long long per_cu = (long long)(kLdsPerCU / lds(m.slots));
  const long long grid = (long long)s.batch * s.num_kv_heads * p.splits;
  m.share = per_cu >= kShareMinWgs && grid >= 2 * per_cu * kNumCUs;
  return m;
}
DecodeWs decode_ws_layout(const LaunchShape& s, const SplitPlan& p);
// Row stride (floats) of the per-head page bounds in the select workspace:
// padded to a multiple of 4 so every row starts 16-byte aligned.
inline int ub_ld(int max_pages) { return (max_pages + 3) & ~3; }
// Top-k plan: the bounds kernel's chunk of cp pages (nchunks per sequence)
// and, when chunked, each head's top keepc pages of a chunk as the select's
// candidates instead of every page's bound.
struct SelectPlan {
  bool chunked = false;
  int nt = 1, cp = 64, nchunks = 0, keepc = 0;
};
SelectPlan plan_select(const LaunchShape& s, int budget);
size_t select_ws_bytes(const LaunchShape& s, int budget);

hipError_t launch_append_meta(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                              const int32_t* old_lens, const int32_t* new_lens, int max_new,
                              void* meta, hipStream_t st);
hipError_t launch_meta(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                       const int32_t* lens, void* meta, hipStream_t st);

hipError_t launch_bounds(const LaunchShape& s, const SelectPlan& p, const float* q,
                         const void* meta, const int32_t* bt, const int32_t* lens, float* ub,
                         hipStream_t st);

hipError_t launch_select(const LaunchShape& s, const SelectPlan& p, const float* ub,
                         const int32_t* lens, int budget, int32_t* sel, float* sel_ub,
                         hipStream_t st);

// Page key moments of every page (old_lens == nullptr), or, after an append,
// of the pages the tokens [old_lens, lens) touch (at most max_new per sequence).
hipError_t launch_moments(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                          const int32_t* old_lens, const int32_t* lens, int max_new,
                          void* moments, hipStream_t st);

// Gaussian-aware selection, before the top-cap select: per-page score
// statistics (mu_a, s_a) into `stats` ([B*H, ub_ld] double2), then per head
// tau_hat and the keys (estimated maximum, or -inf when it fails the rule)
// into `keys` ([B*H, ub_ld] float).
hipError_t launch_gauss_stats(const LaunchShape& s, const float* q, const void* moments,
                              const int32_t* bt, const int32_t* lens, double am1, void* stats,
                              hipStream_t st);
hipError_t launch_gauss_solve(const LaunchShape& s, const void* stats, const int32_t* lens, int m,
                              double delta, float* keys, float* tau_hat, int cap, int32_t* sel,
                              hipStream_t st);
size_t gauss_ws_bytes(const LaunchShape& s);

// Per-head select-and-decode (bf16 caches): one workgroup per query head
// selects its pages from the bounds in the select workspace and decodes
// them. Used when there are at least kHeadMinHeads heads (enough workgroups
// to stream at full rate), the budget is at most kHeadMaxBudget pages, a
// head's selected K is at most kHeadMaxBytes (beyond it re-reading pages
// that the heads of a KV head share costs more than the launches it saves:
// measured 343 -> 415 us at 4 MiB per head), or kHeadMaxBytesRounds when
// the grid takes more than one round of workgroups (one per CU; measured
// with 512 heads: 256 KiB per head 111 -> 107 us, 1 MiB 178 -> 186 us), and
// the kernel's LDS fits. Workspace: the select's bounds, then per (head,
// wave) spill areas of wcap candidates, then per head list_cap window-list
// entries (scores, then V rows).
constexpr long long kHeadMinHeads = 128;
constexpr long long kHeadMaxBytes = 2 << 20;
constexpr long long kHeadMaxBytesRounds = 512 << 10;
constexpr size_t kHeadMaxLds = 150 * 1024;
// With fewer than kHeadMinHeads heads, each head's selection is split over
// `splits` workgroups (enough for about one per CU) that write candidate
// regions, and the threshold kernel finishes the step (its plan `tp`, its
// workspace `tws` at offset `dec`).
struct HeadPlan {
  bool use = false;
  int splits = 1, pps = 0;
  int wcap = 0, list_cap = 0;
  size_t spill = 0, list = 0, total = 0;
  SplitPlan tp;
  DecodeWs tws;
  size_t dec = 0;
};
HeadPlan plan_head(const LaunchShape& s, int budget, size_t select_bytes);
// bt_lds: block_table is 16-byte aligned and max_pages a multiple of 4 (the
// kernel may then stage a block-table row in LDS with 16-byte loads).
hipError_t launch_head_decode(const LaunchShape& s, const SelectPlan& sp, const HeadPlan& hp,
                              const float* q, const void* k_pool, const void* v_pool,
                              const int32_t* bt, const int32_t* lens, int budget, float alpha,
                              float window, int32_t* sel, float* sel_ub, float* out, float* tau,
                              int32_t* support, void* ws, bool bt_lds, hipStream_t st);
constexpr long long kHeadSplitTarget = kNumCUs;  // workgroups the split form aims at

// Per-dtype instantiations (decode_bf16.hip, decode_f32.hip).
hipError_t launch_score_bf16(const LaunchShape& s, const SplitPlan& p, const float* q,
                             const void* k_pool, const int32_t* bt, const int32_t* lens,
                             const int32_t* sel, int budget, float alpha, float window, void* ws,
                             const DecodeWs& L, hipStream_t st);
hipError_t launch_score_f32(const LaunchShape& s, const SplitPlan& p, const float* q,
                            const void* k_pool, const int32_t* bt, const int32_t* lens,
                            const int32_t* sel, int budget, float alpha, float window, void* ws,
                            const DecodeWs& L, hipStream_t st);
hipError_t launch_tau_pv_bf16(const LaunchShape& s, const SplitPlan& p, const void* v_pool,
                              const int32_t* bt, const int32_t* lens, const int32_t* sel,
                              int budget, float alpha, float window, float* out, float* tau,
                              int32_t* support, void* ws, const DecodeWs& L, hipStream_t st);
hipError_t launch_tau_pv_f32(const LaunchShape& s, const SplitPlan& p, const void* v_pool,
                             const int32_t* bt, const int32_t* lens, const int32_t* sel,
                             int budget, float alpha, float window, float* out, float* tau,
                             int32_t* support, void* ws, const DecodeWs& L, hipStream_t st);


}  // namespace ekv
