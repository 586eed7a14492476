// Fixed-budget top-k of one row of page keys by one workgroup, shared by the
// select kernel and the per-head select-and-decode kernel.
// EntmaxKV summary page (gist.science paper 2605.21649), section 2.B policy 1:
// keep the k pages with the highest bounds (ties to the lower page index).
//
// Radix select on the order-preserving 32-bit image of the float32 key,
// starting at the highest bit where the keys differ (so the first histogram
// is spread), 8 bits per pass, stopping as soon as the boundary digit is
// taken whole. The kept pages are emitted in ascending order: each thread
// owns a contiguous run of keys and one two-value block scan of the runs'
// (above, equal) counts places them.
#pragma once

#include "launch.hpp"

namespace ekv {

constexpr int kSelLds = 16384;        // keys staged in LDS when the row has at most this many
constexpr int kSelCand = kSelLds / 2;  // chunked candidates per row (keys, then their pages)

// LDS of select_row, provided by the caller: `sord` kSelLds words (the staged
// keys; with chunked candidates the second half holds their pages), and the
// small arrays below.
template <int NT>
struct SelectScratch {
  int hist[2][256];
  unsigned int ured[NT / kWave][2];
  int wcnt[NT / kWave][2];
  int vcnt[NT / kWave];
  int bc[3];
};

// Top `budget` of the row's keys, one workgroup of NT threads (every thread
// must call it). The row is `row` (float32 keys, P of them, padded to a
// multiple of 4) or, with kCand, the chunked candidates `crow` (order key |
// page << 32; keepc per chunk of cp pages; P is then the row's page count).
// kDrop: keys at or below the order value of -inf are not candidates; when no
// more than `budget` remain all are kept. Calls emit(pos, page, key) for
// every kept page (pos its rank in ascending page order; key its order key)
// and returns the number kept (at most budget; the caller pads the rest).
// `row_cap` (>= 1): keys of the row (candidates with kCand) that are
// readable memory, at least P; the first batch of loads is issued from it
// before anything depends on P, so a caller may pass a P whose load is still
// in flight.
template <int NT, bool kDrop, bool kCand, typename Emit>
__device__ __forceinline__ int select_row(const float* __restrict__ row,
                                          const uint64_t* __restrict__ crow, int P, int budget,
                                          int cp, int keepc, int row_cap, uint32_t* sord,
                                          SelectScratch<NT>& sh, Emit emit) {
  static_assert(!(kDrop && kCand), "the Gaussian keys are not chunked");
  constexpr uint32_t drop_below = 0x007fffffu;  // float_order(-inf)
  constexpr int NW = NT / kWave;
  constexpr int UNR = 4;  // 16-byte loads in flight per thread
  constexpr int CU = 8;   // 8-byte candidate loads in flight per thread
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float4* row4 = reinterpret_cast<const float4*>(row);

  // The first batch of keys, from the readable part of the row (slots past
  // it re-read its last entry); the staging loop below uses it for its first
  // pass.
  float4 f0[UNR];
  uint64_t c0[CU];
  if constexpr (kCand) {
#pragma unroll
    for (int r = 0; r < CU; ++r) c0[r] = crow[min(r * NT + tid, row_cap - 1)];
  } else {
#pragma unroll
    for (int r = 0; r < UNR; ++r) f0[r] = row4[min(r * NT + tid, (row_cap >> 2) - 1)];
  }

  // chunked candidates: nk of them (every chunk but the last holds keepc)
  const int nc = kCand ? (P + cp - 1) / cp : 0;
  const int nk = kCand ? (nc == 0 ? 0 : (nc - 1) * keepc + min(keepc, P - (nc - 1) * cp)) : P;
  int* sj = reinterpret_cast<int*>(sord + kSelCand);  // kCand: candidates' pages

  if (!kDrop && P <= budget) {
    // every page kept (kCand: then one chunk holds them all, in page order)
    for (int i = tid; i < P; i += NT)
      emit(i, i, kCand ? (uint32_t)crow[i] : float_order(row[i] + 0.0f));
    return P;
  }

  // Order-preserving 32-bit keys, handled four at a time (rows are padded to
  // a multiple of 4 floats; a quad's entries at or past P are masked). They
  // are staged in LDS when they fit, else re-read from the bounds row.
  // kCand: the candidates' keys (always staged) take the place of the pages'.
  if constexpr (kCand) P = nk;
  const bool staged = kCand || P <= kSelLds;
  const int n4 = (P + 3) >> 2;
  const int qpt = (n4 + NT - 1) / NT;
  const int q0 = min(n4, tid * qpt), q1 = min(n4, q0 + qpt);
  auto from_global = [&](int i4) -> uint4 {
    const float4 f = row4[i4];
    return make_uint4(float_order(f.x + 0.0f), float_order(f.y + 0.0f), float_order(f.z + 0.0f),
                      float_order(f.w + 0.0f));
  };
  auto quad = [&](int i4) -> uint4 {
    return staged ? *reinterpret_cast<const uint4*>(&sord[4 * i4]) : from_global(i4);
  };
  auto at = [](const uint4& v, int e) -> uint32_t {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
  };

  // A key counts when its page is below P (and, with kDrop, it is above -inf).
  auto valid = [&](int j, uint32_t o) { return j < P && (!kDrop || o > drop_below); };
  uint32_t mn = 0xffffffffu, mx = 0u;
  int nvalid = 0;
  if constexpr (kCand) {
    // stage the candidates' keys and pages, every load of a batch issued
    // before the first is used
    for (int base = 0; base < P; base += CU * NT) {
      // unconditional loads (slots past the row re-read its last entry), so
      // that all of them are issued before the first wait
      uint64_t v[CU];
#pragma unroll
      for (int r = 0; r < CU; ++r)
        v[r] = base == 0 ? c0[r] : crow[min(base + r * NT + tid, P - 1)];
#pragma unroll
      for (int r = 0; r < CU; ++r) {
        const int i = base + r * NT + tid;
        if (i < P) {
          const uint32_t o = (uint32_t)v[r];
          sord[i] = o;
          sj[i] = (int)(uint32_t)(v[r] >> 32);
          mn = min(mn, o);
          mx = max(mx, o);
        }
      }
    }
  }
  for (int base = 0; !kCand && base < n4; base += UNR * NT) {
    // unconditional loads (slots past the row re-read its last quad), all
    // issued before the first is converted
    float4 f[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r)
      f[r] = base == 0 ? f0[r] : row4[min(base + r * NT + tid, n4 - 1)];
    uint4 v[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r)
      v[r] = make_uint4(float_order(f[r].x + 0.0f), float_order(f[r].y + 0.0f),
                        float_order(f[r].z + 0.0f), float_order(f[r].w + 0.0f));
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int i4 = base + r * NT + tid;
      if (i4 < n4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (valid(4 * i4 + e, at(v[r], e))) {
            mn = min(mn, at(v[r], e));
            mx = max(mx, at(v[r], e));
            if constexpr (kDrop) ++nvalid;
          }
        }
        if (staged) *reinterpret_cast<uint4*>(&sord[4 * i4]) = v[r];
      }
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if constexpr (kDrop) nvalid = wave_sum(nvalid);
  if (lane == 0) {
    sh.ured[wave][0] = mn;
    sh.ured[wave][1] = mx;
    if constexpr (kDrop) sh.vcnt[wave] = nvalid;
  }
  if (tid < 256) sh.hist[0][tid] = 0;
  __syncthreads();
  nvalid = kDrop ? 0 : P;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, sh.ured[w][0]);
    mx = max(mx, sh.ured[w][1]);
    if constexpr (kDrop) nvalid += sh.vcnt[w];
  }

  // Radix select of the budget-th largest key, 8 bits per pass from the
  // highest bit where keys differ; stop once the boundary digit is taken
  // whole. Two histograms alternate so that a pass needs two barriers.
  uint32_t prefix, pmask;
  int k = budget;  // rank still to place among keys matching the prefix
  if (kDrop && nvalid <= budget) {
    // every counted key is kept: all of them "equal" an empty prefix
    prefix = 0u;
    pmask = 0u;
    k = nvalid;
  } else if (mn == mx) {
    prefix = mx;
    pmask = 0xffffffffu;
  } else {
    int hb = 31 - __clz(mn ^ mx);
    pmask = ~((2u << hb) - 1u);
    prefix = mx & pmask;
    int cur = 0;
    while (true) {
      const int lo = hb >= 7 ? hb - 7 : 0;
      const int width = hb - lo + 1;
      const uint32_t dmask = (1u << width) - 1u;
      if (tid < 256) sh.hist[cur ^ 1][tid] = 0;
      for (int base = 0; base < n4; base += UNR * NT) {
        uint4 v[UNR];
#pragma unroll
        for (int r = 0; r < UNR; ++r) v[r] = quad(min(base + r * NT + tid, n4 - 1));
#pragma unroll
        for (int r = 0; r < UNR; ++r) {
          const int i4 = base + r * NT + tid;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t o = at(v[r], e);
            if (i4 < n4 && valid(4 * i4 + e, o) && (o & pmask) == prefix)
              atomicAdd(&sh.hist[cur][(o >> lo) & dmask], 1);
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        int c4[4];
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c4[i] = sh.hist[cur][4 * lane + i];
          s += c4[i];
        }
        // keys in this lane's bins and above: the total less the keys in
        // lower lanes' bins
        const int incl = wave_incl_scan(s, lane);
        const int suf = lane_value(incl, kWave - 1) - incl + s;
        int above = suf - s;
        if (above < k && k <= suf) {
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if (above < k && k <= above + c4[i]) {
              sh.bc[0] = 4 * lane + i;
              sh.bc[1] = above;
              sh.bc[2] = c4[i];
            }
            above += c4[i];
          }
        }
      }
      __syncthreads();
      const int d = sh.bc[0];
      const int cnt_d = sh.bc[2];
      k -= sh.bc[1];
      prefix |= ((uint32_t)d) << lo;
      pmask |= dmask << lo;
      if (cnt_d == k || lo == 0) break;
      hb = lo - 1;
      cur ^= 1;
    }
  }

  // Keep keys above the prefix and the first k (by page index) equal to it,
  // written in ascending page order: thread t owns a contiguous run of quads,
  // one block scan of the runs' (above, equal) counts places each run, and
  // the thread emits its kept pages in order.
  int n_gt = 0, n_eq = 0;
  for (int i4 = q0; i4 < q1; ++i4) {
    const uint4 v = quad(i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = valid(4 * i4 + e, at(v, e));
      const uint32_t m = at(v, e) & pmask;
      n_eq += (ok && m == prefix) ? 1 : 0;
      n_gt += (ok && m > prefix) ? 1 : 0;
    }
  }
  int gt_base, eq_base;
  block_excl_scan2<NT>(n_gt, n_eq, &sh.wcnt[0][0], &gt_base, &eq_base);
  int pos = gt_base + min(eq_base, k);
  int eqc = eq_base;  // equal keys on lower pages
  for (int i4 = q0; i4 < q1 && pos < budget; ++i4) {
    const uint4 v = quad(i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = valid(4 * i4 + e, at(v, e));
      const uint32_t m = at(v, e) & pmask;
      const bool eq = ok && m == prefix;
      const bool take = (ok && m > prefix) || (eq && eqc < k);
      eqc += eq ? 1 : 0;
      if (take) {
        if (pos < budget) emit(pos, kCand ? sj[4 * i4 + e] : 4 * i4 + e, at(v, e));
        ++pos;
      }
    }
  }
  // kept: every key above the prefix plus k equal ones, at most budget
  // (kDrop with few candidates: all nvalid of them)
  return kDrop && nvalid <= budget ? nvalid : budget;
}

}  // namespace ekv
