// Gather-score and threshold/P.V kernels of the alpha-entmax decode.
// EntmaxKV summary page (gist.science paper 2605.21649), section 2.C: read
// only the selected pages' K/V and solve alpha-entmax on that reduced set;
// section 4 (efficiency): the full-cache entmax decode is the same with
// every page. alpha-entmax: p_i = [(alpha-1) z_i - tau]_+^(1/(alpha-1)),
// sum p = 1 (Peters, Niculae & Martins 2019).
//
// score_kernel (one workgroup per (page split, sequence, KV head)):
//   Streams the split's K pages once for the G query heads of the KV head:
//   bf16 caches on the matrix cores (q split exactly into three bf16 parts,
//   keys through direct-to-LDS loads), float32 caches on the vector ALU (a
//   token row spread over LT lanes, the G partial dot products finished in a
//   multi-value butterfly). Only tokens that can be in the support are kept:
//   every token with p > 0 has z > max(z) - 1/(alpha-1) (at
//   tau = (alpha-1) max z - 1 the top token alone has weight 1), and a
//   running maximum can only underestimate max(z), so filtering against it
//   keeps a superset (the four waves share their running maxima through
//   LDS, so each filters against the largest). Survivors go to per-wave LDS
//   lists, are filtered again against the workgroup maximum and written, in
//   a fixed order, as this split's candidate region (z, token index) with its
//   count and maximum.
//   Sparse: the split is a slice of the union of the G heads' selected pages
//   (each page read once), built from a bitmap in LDS.
// tau_pv_kernel (one workgroup per (sequence, query head); one kernel for the
// budgeted and the full-cache decode):
//   Takes the global maximum over the regions, gathers the candidates inside
//   the window into a list (tightened first by a lower bound on tau when
//   there are many), solves tau on f(tau) = sum [a_i - tau]_+^m = 1 -- by
//   the sort-based closed form for m = 1, 2 on short lists, else by a
//   safeguarded iteration from the left (Newton's method on f^(1/m) - 1,
//   then on f near the root) bracketed by [a_max - 1, a_max] with bisection
//   when a step leaves the bracket -- then reads V rows only for
//   the tokens with p > 0 (for short lists they are requested before the
//   solve) and writes o = sum p v / sum p. The rarely taken steps are
//   out-of-line functions, which keeps the common path's code compact.
#pragma once

#include <float.h>

#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"

namespace ekv {

template <typename KV>
struct KvTraits;
template <>
struct KvTraits<bf16_t> {
  using Acc = float;
  static constexpr int VPC = 8;
};
template <>
struct KvTraits<float> {
  using Acc = double;
  static constexpr int VPC = 4;
};

template <typename KV>
__device__ __forceinline__ void widen(const uint4& x, typename KvTraits<KV>::Acc (&f)[KvTraits<KV>::VPC]) {
  if constexpr (sizeof(KV) == 2) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    f[0] = (double)__uint_as_float(x.x);
    f[1] = (double)__uint_as_float(x.y);
    f[2] = (double)__uint_as_float(x.z);
    f[3] = (double)__uint_as_float(x.w);
  }
}

// One candidate: a score in the accumulation precision and its token index
// in the head's gathered list (slot * page_size + row).
template <typename ZT>
struct alignas(2 * sizeof(ZT)) Cand {
  ZT z;
  int idx;
};

// A candidate read through a pointer into global memory, addressed as such
// (a global load even where the compiler cannot see the pointer's origin).
template <typename ZT>
__device__ __forceinline__ Cand<ZT> ld_global_cand(const Cand<ZT>* p) {
  Cand<ZT> c;
  if constexpr (sizeof(ZT) == 4) {
    const uint64_t v = *(const __attribute__((address_space(1))) uint64_t*)p;
    c.z = __builtin_bit_cast(float, (uint32_t)v);
    c.idx = (int)(uint32_t)(v >> 32);
  } else {
    c.z = *(const __attribute__((address_space(1))) double*)&p->z;
    c.idx = *(const __attribute__((address_space(1))) int*)&p->idx;
  }
  return c;
}

template <typename T>
__device__ __forceinline__ T neg_inf() {
  return -__builtin_huge_val();
}
template <>
__device__ __forceinline__ float neg_inf<float>() {
  return -__builtin_inff();
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 stream_load16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// First index in row[0..n) whose value (negatives read as +inf) is >= key; -1 if
// row has no entry equal to key.
__device__ __forceinline__ int find_slot(const int32_t* row, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = row[mid];
    const uint32_t kv = v < 0 ? 0xffffffffu : (uint32_t)v;
    if (kv < (uint32_t)key) lo = mid + 1;
    else hi = mid;
  }
  return (lo < n && row[lo] == key) ? lo : -1;
}

// This split's pages, in LDS: `slice` (sparse: logical page indices, taken
// from the union of the G heads' selections in ascending order), `slots`
// (sparse: each head's position of the page in its selection, -1 if the head
// did not select it) and `sphys` (physical page ids, fetched with one
// coalesced load per page). Returns the number of pages; ends with a barrier
// (every thread of the block must call it).
template <int G, bool SPARSE>
__device__ int build_slice(const int32_t* __restrict__ sel, const int32_t* __restrict__ block_table,
                           int b, int bh0, int budget, int P, int max_pages, int split, int pps,
                           unsigned* bm, int32_t* ssel, int* slice, int* slots, int* sphys,
                           int* tmp) {
  const int tid = threadIdx.x;
  int n_slice;
  if constexpr (SPARSE) {
    const int32_t* selrow = sel + (size_t)bh0 * budget;
    const bool staged = (size_t)G * budget <= (size_t)kSelCopy;
    const int nwords = (P + 31) >> 5;
    for (int i = tid; i < nwords; i += kNT) bm[i] = 0u;
    if (staged)
      for (int i = tid; i < G * budget; i += kNT) ssel[i] = selrow[i];
    __syncthreads();
    const int32_t* srow = staged ? ssel : selrow;
    for (int i = tid; i < G * budget; i += kNT) {
      const int jj = srow[i];
      if (jj >= 0 && jj < P) atomicOr(&bm[jj >> 5], 1u << (jj & 31));
    }
    __syncthreads();
    const int wpt = (nwords + kNT - 1) / kNT;
    const int w0 = min(nwords, tid * wpt), w1 = min(nwords, w0 + wpt);
    int local = 0;
    for (int w = w0; w < w1; ++w) local += __popc(bm[w]);
    int utot;
    const int rbase = block_excl_scan<kNT>(local, tmp, &utot);
    const int lo = split * pps;
    const int hi = min(utot, lo + pps);
    n_slice = max(0, hi - lo);
    if (n_slice > 0) {
      int r = rbase;
      for (int w = w0; w < w1 && r < hi; ++w) {
        unsigned bits = bm[w];
        while (bits) {
          const int bit = __ffs(bits) - 1;
          bits &= bits - 1u;
          if (r >= lo && r < hi) slice[r - lo] = w * 32 + bit;
          ++r;
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < n_slice * G; i += kNT) {
      const int p = i / G, h = i % G;
      slots[i] = find_slot(srow + (size_t)h * budget, budget, slice[p]);
    }
  } else {
    const int lo = split * pps;
    n_slice = max(0, min(P, lo + pps) - lo);
  }
  for (int p = tid; p < n_slice; p += kNT) {
    const int j = SPARSE ? slice[p] : split * pps + p;
    sphys[p] = block_table[(size_t)b * max_pages + j];
  }
  __syncthreads();
  return n_slice;
}

// ---------------------------------------------------------------------------
// threshold and P.V

// d^e through exp2/log2 (d > 0); kept out of line so that its registers do
// not add to those of the loops that call it.
__device__ __attribute__((noinline)) double pow_general(double d, double e) {
  return exp2(e * log2(d));
}

// d^(m-1) for the common exponents, pow_general otherwise (d > 0).
__device__ __forceinline__ double pow_m1(double d, double m, int mcode) {
  switch (mcode) {
    case 1: return 1.0;
    case 2: return d;
    case 3: return d * d;
    case 4: return d * d * d;
    default: return pow_general(d, m - 1.0);
  }
}

// The next iterate of the threshold solve from t, where f = sum [a_i - t]_+^m
// and fp = m sum [a_i - t]_+^(m-1) > 0 (so f'(t) = -fp). Far from the root
// (|f - 1| >= 1e-3) and for m >= 1 it is Newton's step on phi(t) =
// f(t)^(1/m) - 1: t + m (f - f^(1 - 1/m)) / fp. phi is convex and
// decreasing in t (the m-norm of the convex functions [a_i - t]_+), so from
// a point left of the root the step stays left of it and the iterates rise
// to the root, as Newton's on f does; the step is exact whenever the active
// terms are equal and the active set does not change, where Newton's on f
// needs many steps from a_max - 1. Near the root, and for m < 1 (where
// f^(1/m) is not a norm), it is Newton's step on f, whose numerator f - 1 is
// exact there.
__device__ __forceinline__ double tau_step(double t, double f, double fp, double m, int mcode) {
  if (m < 1.0 || fabs(f - 1.0) < 1e-3) return t + (f - 1.0) / fp;
  double g;  // f^(1 - 1/m)
  switch (mcode) {
    case 1: g = 1.0; break;
    case 2: g = sqrt(f); break;
    case 3: {
      const double c = cbrt(f);
      g = c * c;
      break;
    }
    case 4: {
      const double r = sqrt(f);
      g = r * sqrt(r);
      break;
    }
    default: g = pow_general(f, 1.0 - 1.0 / m);
  }
  return t + m * (f - g) / fp;
}

template <int SNT>
__device__ __forceinline__ void scope_sum2(double& a, double& c, double* red) {
  a = wave_allsum(a);
  c = wave_allsum(c);
  if constexpr (SNT > kWave) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == 0) {
      red[2 * wid] = a;
      red[2 * wid + 1] = c;
    }
    __syncthreads();
    a = 0.0;
    c = 0.0;
#pragma unroll
    for (int w = 0; w < SNT / kWave; ++w) {
      a += red[2 * w];
      c += red[2 * w + 1];
    }
    __syncthreads();
  }
}

// Safeguarded iteration (tau_step) for sum_i [a_i - t]_+^m = 1 with
// a_i = am1 * z_i. The
// root lies in [a_max - 1, a_max): f(a_max - 1) >= 1 (top term is 1) and
// f(a_max) = 0. tlo, when given, is a known lower bound on the root (the
// threshold of a subset of the tokens, less a margin): the bracket and the
// first step start at max(a_max - 1, tlo). Called by the SNT threads
// t0 = 0..SNT-1 of the scope.
template <int SNT, typename ZT>
__device__ double solve_tau(const ZT* z, int n, double am1, double m, int mcode, double amax,
                            int t0, double* red, double tlo = -DBL_MAX) {
  double lo = fmax(amax - 1.0, tlo), hi = amax, t = lo;
  for (int it = 0; it < 200; ++it) {
    double f = 0.0, fp = 0.0;
    for (int i = t0; i < n; i += SNT) {
      const double d = am1 * (double)z[i] - t;
      if (d > 0.0) {
        const double pm1 = pow_m1(d, m, mcode);
        fp += pm1;
        f += pm1 * d;
      }
    }
    scope_sum2<SNT>(f, fp, red);
    fp *= m;
    if (f >= 1.0) lo = t;
    else hi = t;
    if (f == 1.0) break;
    const double scale = fmax(1.0, fabs(t));
    double tn = fp > 0.0 ? tau_step(t, f, fp, m, mcode) : 0.5 * (lo + hi);
    if (fp > 0.0 && fabs(tn - t) <= 2.0 * DBL_EPSILON * scale) {
      t = fmin(fmax(tn, lo), hi);
      break;
    }
    if (!(tn > lo && tn < hi)) tn = 0.5 * (lo + hi);
    if (hi - lo <= 4.0 * DBL_EPSILON * scale) {
      t = 0.5 * (lo + hi);
      break;
    }
    t = tn;
  }
  return t;
}

__device__ __forceinline__ double pow_m(double d, double m, int mcode) {
  return d * pow_m1(d, m, mcode);
}

// The exponent of the threshold equation as a compile-time value: MC = m for
// the integer m = 1..4 (alpha = 2, 3/2, 4/3, 5/4), MC = 0 for any other m
// (taken at run time through pow_m1). With MC > 0 the Newton sums below are
// branch-free: no call to pow_general (a caller holding many values in
// registers spills none around it) and no per-term branch on mcode or on
// the sign of d.
template <int MC>
__device__ __forceinline__ double pow_m1_t(double d, double m, int mcode) {
  if constexpr (MC == 0) {
    return pow_m1(d, m, mcode);
  } else {
    (void)m;
    (void)mcode;
    if constexpr (MC == 1) return 1.0;
    else if constexpr (MC == 2) return d;
    else if constexpr (MC == 3) return d * d;
    else return d * d * d;
  }
}

// Adds [d]_+^(m-1) to fp and [d]_+^m to f: the terms of f(t) = sum [a_i -
// t]_+^m and of f'(t) / -m, the same values (and so the same sums) whether
// a term is skipped or added as zero.
template <int MC>
__device__ __forceinline__ void add_terms(double d, double m, int mcode, double& f, double& fp) {
  if constexpr (MC == 0) {
    if (d > 0.0) {
      const double pm1 = pow_m1(d, m, mcode);
      fp += pm1;
      f += pm1 * d;
    }
  } else {
    const double dd = fmax(d, 0.0);
    const double pm1 = MC == 1 ? (d > 0.0 ? 1.0 : 0.0) : pow_m1_t<MC>(dd, m, mcode);
    fp += pm1;
    f += pm1 * dd;
  }
}

// Calls fn(std::integral_constant<int, MC>) with MC = mcode for mcode 1..4,
// else MC = 0 (INT_ONLY: the caller has checked that m is an integer 1..4,
// and only those four are instantiated).
template <bool INT_ONLY = false, typename Fn>
__device__ __forceinline__ auto with_mcode(int mcode, Fn fn) {
  switch (mcode) {
    case 1: return fn(std::integral_constant<int, 1>());
    case 2: return fn(std::integral_constant<int, 2>());
    case 3: return fn(std::integral_constant<int, 3>());
    default:
      if constexpr (INT_ONLY) return fn(std::integral_constant<int, 4>());
      else if (mcode == 4) return fn(std::integral_constant<int, 4>());
      else return fn(std::integral_constant<int, 0>());
  }
}

// The same safeguarded Newton iteration for the whole workgroup, each thread
// holding K of the a_i in registers (-DBL_MAX marks an empty slot), of
// which only the first `used` (uniform) can be occupied; every thread of the
// block must call it and gets the same result.
template <int K, int MC, int NT>
__device__ double solve_tau_block(const double (&a)[K], int used, double m, int mcode,
                                  double amax, double* red, double tlo = -DBL_MAX) {
  double lo = fmax(amax - 1.0, tlo), hi = amax, t = lo;
  for (int it = 0; it < 200; ++it) {
    double f = 0.0, fp = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k < used) add_terms<MC>(a[k] - t, m, mcode, f, fp);
    scope_sum2<NT>(f, fp, red);
    fp *= m;
    if (f >= 1.0) lo = t;
    else hi = t;
    if (f == 1.0) break;
    const double scale = fmax(1.0, fabs(t));
    double tn = fp > 0.0 ? tau_step(t, f, fp, m, mcode) : 0.5 * (lo + hi);
    if (fp > 0.0 && fabs(tn - t) <= 2.0 * DBL_EPSILON * scale) {
      t = fmin(fmax(tn, lo), hi);
      break;
    }
    if (!(tn > lo && tn < hi)) tn = 0.5 * (lo + hi);
    if (hi - lo <= 4.0 * DBL_EPSILON * scale) {
      t = 0.5 * (lo + hi);
      break;
    }
    t = tn;
  }
  return t;
}

// The safeguarded Newton iteration of solve_tau for one wave whose lanes
// hold the list's a_i = am1 * z_i in registers (K per lane, entry e in slot
// e / 64 of lane e % 64; -DBL_MAX marks an empty slot), so an iteration reads
// no memory; only the slots below n (uniform) entries are summed. Same steps
// and stopping rules.
template <int K, int MC>
__device__ double solve_tau_regs(const double (&a)[K], int n, double am1, double m, int mcode,
                                 double amax, double tlo = -DBL_MAX) {
  (void)am1;
  double lo = fmax(amax - 1.0, tlo), hi = amax, t = lo;
  for (int it = 0; it < 200; ++it) {
    double f = 0.0, fp = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k * kWave < n) add_terms<MC>(a[k] - t, m, mcode, f, fp);
    f = wave_allsum(f);
    fp = wave_allsum(fp) * m;
    if (f >= 1.0) lo = t;
    else hi = t;
    if (f == 1.0) break;
    const double scale = fmax(1.0, fabs(t));
    double tn = fp > 0.0 ? tau_step(t, f, fp, m, mcode) : 0.5 * (lo + hi);
    if (fp > 0.0 && fabs(tn - t) <= 2.0 * DBL_EPSILON * scale) {
      t = fmin(fmax(tn, lo), hi);
      break;
    }
    if (!(tn > lo && tn < hi)) tn = 0.5 * (lo + hi);
    if (hi - lo <= 4.0 * DBL_EPSILON * scale) {
      t = 0.5 * (lo + hi);
      break;
    }
    t = tn;
  }
  return t;
}

// Exact threshold for m = 1 (alpha = 2) and m = 2 (alpha = 1.5) by the
// sort-based rule, without sorting: one wave, lane i holding a_i (-DBL_MAX
// past the n <= 64 entries). Lane i finds its rank k_i in descending order
// (ties to the lower lane) and the sums S1, S2 of b = a - amax over the k_i
// largest entries; the support size k* is the largest rank with
// sum_{j <= k} (a_(j) - a_(k))^m < 1 (the sum grows with k), and tau = amax + t with t the root of
// sum_{j <= k*} (b_(j) - t)^m = 1: (S1 - 1) / k* for m = 1, the smaller root
// (S1 - sqrt(S1^2 - k* (S2 - 1))) / k* for m = 2. Every lane returns tau.
__device__ double solve_tau_ranked(double a, int n, int mcode, double amax) {
  const int lane = threadIdx.x & (kWave - 1);
  const double bi = a - amax;
  int k = 0;
  double s1 = 0.0, s2 = 0.0;
  for (int j = 0; j < n; ++j) {
    const uint64_t bits = __double_as_longlong(a);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)bits, j);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(bits >> 32), j);
    const double aj = __longlong_as_double(((uint64_t)hi << 32) | lo);
    if (aj > a || (aj == a && j <= lane)) {
      const double bj = aj - amax;
      ++k;
      s1 += bj;
      s2 = fma(bj, bj, s2);
    }
  }
  const bool live = lane < n;
  const double F = mcode == 1 ? s1 - k * bi : s2 - 2.0 * bi * s1 + k * bi * bi;
  const int kstar = wave_max((live && F < 1.0) ? k : 0);  // >= 1: F = 0 at rank 1
  const uint64_t at = __ballot(live && k == kstar);
  const int src = __ffsll((unsigned long long)at) - 1;
  const double S1 = lane_value(s1, src), S2 = lane_value(s2, src);
  double t;
  if (mcode == 1) {
    t = (S1 - 1.0) / kstar;
  } else {
    const double disc = fmax(0.0, S1 * S1 - kstar * (S2 - 1.0));
    t = (S1 - sqrt(disc)) / kstar;
  }
  return amax + t;
}

// One wave solves tau over a window list held K entries per lane in
// registers (a_i = am1 * z_i), then (when `compact`) compacts the support
// (V row, p) to the front of the list in list order; returns the support
// size, the wave's sum of p and tau (every lane). Lists of up to 64 entries
// at m = 1, 2 take the rank-based closed form. Without `compact` li and sp
// are left as they are: other waves may still be reading li.
template <int K, int MC, typename ZT>
__device__ __forceinline__ void wave_solve_list(const ZT* lz, int* li, float* sp, int n_list, double am1, double m,
                                int mcode, double amax, int lane, uint64_t ltm, bool compact,
                                int& n_sup, double& psum, double& tau, double tlo) {
  double a[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int e = k * kWave + lane;
    a[k] = e < n_list ? am1 * (double)lz[e] : -DBL_MAX;
  }
  const double t = (n_list <= kWave && (mcode == 1 || mcode == 2))
                       ? solve_tau_ranked(a[0], n_list, mcode, amax)
                       : solve_tau_regs<K, MC>(a, n_list, am1, m, mcode, amax, tlo);
  int o = 0;
  double ps = 0.0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int e = k * kWave + lane;
    const double d = a[k] - t;
    const bool f = e < n_list && d > 0.0;
    const int ix = (f && compact) ? li[e] : 0;
    const uint64_t bal = __ballot(f);
    if (f) {
      const double pv = d * pow_m1_t<MC>(d, m, mcode);
      ps += pv;
      if (compact) {
        li[o + __popcll(bal & ltm)] = ix;
        sp[o + __popcll(bal & ltm)] = (float)pv;
      }
    }
    o += __popcll(bal);
  }
  psum = wave_allsum(ps);
  n_sup = o;
  tau = t;
}

// Candidate lists of the score kernel: a wave appends the survivors of each
// head in page order; the first `slots` of them stay in LDS, the rest go
// to the wave's spill area in global memory (only when scores are nearly
// uniform, or the window is wide, does a wave keep more).
template <typename Acc>
struct CandLists {
  Acc* rz;              // LDS scores  [wave][head][slots]
  int* ri;              // LDS indices [wave][head][slots]
  Cand<Acc>* spill;     // this workgroup's spill areas [wave][head][wcap]
  int wcap;
  int slots;
  __device__ __forceinline__ void put_lds(int wave, int h, int G, int pos, Acc z, int idx) const {
    const int o = (wave * G + h) * slots + pos;
    rz[o] = z;
    ri[o] = idx;
  }
  __device__ __forceinline__ void put_spill(int wave, int h, int G, int pos, Acc z,
                                            int idx) const {
    Cand<Acc> cv;
    cv.z = z;
    cv.idx = idx;
    spill[(size_t)(wave * G + h) * wcap + (pos - slots)] = cv;
  }
  __device__ __forceinline__ void put(int wave, int h, int G, int pos, Acc z, int idx) const {
    if (pos < slots) {
      const int o = (wave * G + h) * slots + pos;
      rz[o] = z;
      ri[o] = idx;
    } else {
      Cand<Acc> cv;
      cv.z = z;
      cv.idx = idx;
      spill[(size_t)(wave * G + h) * wcap + (pos - slots)] = cv;
    }
  }
  __device__ __forceinline__ void get(int wave, int h, int G, int pos, Acc& z, int& idx) const {
    if (pos < slots) {
      const int o = (wave * G + h) * slots + pos;
      z = rz[o];
      idx = ri[o];
    } else {
      const Cand<Acc> cv = spill[(size_t)(wave * G + h) * wcap + (pos - slots)];
      z = cv.z;
      idx = cv.idx;
    }
  }
};

// Arguments of the score step (device pointers; regions are this call's
// candidate regions, spill the per-wave overflow areas).
template <typename KV>
struct ScoreArgs {
  const float* q;
  const KV* k_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel;
  int H, Hkv, U, max_pages, num_phys, budget, pps, splits, cap;
  double window_d;
  Cand<typename KvTraits<KV>::Acc>* cand;
  int* counts;
  typename KvTraits<KV>::Acc* maxima;
  Cand<typename KvTraits<KV>::Acc>* spill;
  // full cache on the matrix cores with a wide window: each head's maximum
  // shared by every workgroup of the call (order keys kMaxStride apart,
  // reset to that of -inf before the launch), else null
  uint32_t* gmax;
  int slots;  // LDS candidate slots per (wave, head)
  // wide windows on the matrix cores: each workgroup solves the threshold of
  // its own first candidates (a lower bound on tau) and keeps only those
  // above it; with shared maxima the bound is shared too (word 1 of each
  // head's gmax line)
  int local_bound;
  float alpha;
};

// One split of one (sequence, KV head) unit, by the whole workgroup.
template <typename KV, int D, int G, int PS, bool SPARSE>
__device__ __forceinline__ void score_split(const ScoreArgs<KV>& args, int split, int u, unsigned char* smem) {
  using Tr = KvTraits<KV>;
  using Acc = typename Tr::Acc;  // also the score type
  constexpr bool MFMA = kMfmaScores && sizeof(KV) == 2;
  const float* __restrict__ q = args.q;
  const KV* __restrict__ k_pool = args.k_pool;
  const int32_t* __restrict__ block_table = args.block_table;
  const int32_t* __restrict__ seq_lens = args.seq_lens;
  const int32_t* __restrict__ sel = args.sel;
  const int H = args.H, Hkv = args.Hkv, max_pages = args.max_pages, num_phys = args.num_phys;
  const int budget = args.budget, pps = args.pps, splits = args.splits, cap = args.cap;
  Cand<Acc>* __restrict__ cand = args.cand;
  int* __restrict__ counts = args.counts;
  Acc* __restrict__ maxima = args.maxima;
  Cand<Acc>* __restrict__ spill = args.spill;
  const Acc window = (Acc)args.window_d;
  auto put_count = [&](size_t r, int n, Acc mval) {
    counts[r] = n;
    maxima[r] = mval;
  };

  const ScoreLds lay = score_lds_layout(G, PS, pps, SPARSE, max_pages, budget, sizeof(Acc),
                                        score_kbuf_bytes(sizeof(KV) == 2, G, PS, D, SPARSE), D, args.slots);
  // The waves' running maxima per head: a static LDS array, so the compiler
  // can tell it apart from the page buffers that direct-to-LDS loads fill
  // (reads of it then need not wait for those loads).
  __shared__ Acc wmax[kNW * G];
  __shared__ Acc wfloor[G];
  __shared__ Acc wlb[G];
  int* wcnt = reinterpret_cast<int*>(smem + lay.wcnt);
  int* slice = reinterpret_cast<int*>(smem + lay.slice);
  int* slots = reinterpret_cast<int*>(smem + lay.slot);
  int* sphys = reinterpret_cast<int*>(smem + lay.phys);
  int* tmp = reinterpret_cast<int*>(smem + lay.tmp);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int b = u / Hkv, g = u % Hkv;
  const int L = clamp_len(seq_lens[b], max_pages * PS);
  const int P = (L + PS - 1) / PS;
  const int bh0 = b * H + g * G;
  const CandLists<Acc> lists{reinterpret_cast<Acc*>(smem + lay.rz),
                             reinterpret_cast<int*>(smem + lay.ri),
                             spill + (size_t)(b * Hkv + g) * splits * kNW * G * lay.wcap +
                                 (size_t)split * kNW * G * lay.wcap,
                             lay.wcap, lay.slots};

  // Matrix-core path: this thread's q values of the group, read now so that
  // their latency overlaps the slice set-up.
  constexpr int QPT = (G * D + kNT - 1) / kNT;
  float qx[QPT];
  // and, full cache, the call's shared maxima of the group's heads (thread
  // t < kNW * G: head t % G), the waves' starting maxima
  uint32_t gstart = 0x007fffffu;    // the order key of -inf
  uint32_t gstartlb = 0x007fffffu;  // and the shared lower bound on tau (z units)
  if constexpr (MFMA) {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = k * kNT + tid;
      qx[k] = i < G * D ? q[(size_t)bh0 * D + i] : 0.0f;
    }
    if (!SPARSE && args.gmax && tid < kNW * G) {
      gstart = __hip_atomic_load(args.gmax + (size_t)(bh0 + tid % G) * kMaxStride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      gstartlb = __hip_atomic_load(args.gmax + (size_t)(bh0 + tid % G) * kMaxStride + 1,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  const int n_slice = build_slice<G, SPARSE>(
      sel, block_table, b, bh0, budget, P, max_pages, split, pps,
      reinterpret_cast<unsigned*>(smem + lay.bitmap), reinterpret_cast<int32_t*>(smem + lay.ssel),
      slice, slots, sphys, tmp);
  if (n_slice == 0) {
    if (tid < G) put_count((size_t)(bh0 + tid) * splits + split, 0, neg_inf<Acc>());
    return;
  }

  const uint64_t ltm = lanemask_below(lane);
  uint32_t gkey = 0u;  // full cache on the matrix cores: a shared maximum (see below)
  uint32_t gkeylb = 0x007fffffu;  // and the shared lower bound on tau (order key of -inf)
  if constexpr (MFMA) {
    // Matrix-core scores. Each wave streams its pages into its own two LDS
    // page buffers with direct-to-LDS 16-byte loads: every load instruction
    // reads 1 KiB of the page contiguously, and lane i of it writes LDS bytes
    // [16i, 16i + 16); the lanes' source chunks are permuted within each row
    // (chunk c of row r sits in slot c ^ swz(r)) so that the operand reads
    // below hit distinct LDS banks. z for 16 tokens x 4 heads is a chain of
    // v_mfma_f32_16x16x32_bf16 over head_dim: A rows are (head, part) =
    // 4 * head + part with q split exactly into three bf16 parts, B columns
    // are the 16 token rows of a page tile. Lane l ends with head l/16's three
    // part sums for token l%16 and adds them.
    constexpr int KS = D / 32;        // k-steps of 32 dims
    constexpr int NMB = (G + 3) / 4;  // blocks of 4 heads
    // Full cache: each head's maximum shared by every workgroup of the call
    // (raised by each workgroup to its split's maximum when it ends, read
    // when one starts and again before its final pass). Every value there
    // is the score of one of the head's tokens, so at most the head's
    // maximum: filtering against it still keeps every token within the
    // window of that maximum, and far fewer others once earlier workgroups
    // have seen large scores.
    uint32_t* const gm = SPARSE ? nullptr : args.gmax;
    constexpr int TILES = PS / 16;    // 16-token tiles per page
    constexpr int RB = D * 2;         // bytes per K row
    constexpr int PB = PS * RB;       // bytes per page
    constexpr int NI = PB / 1024;     // 1 KiB load instructions per page
    constexpr int RPI = 1024 / RB;    // rows per load instruction
    constexpr int CPR = RB / 16;      // 16-byte chunks per row
    static_assert(NI >= 1 && NI * 1024 == PB && CPR * 16 == RB, "page tiling");
    auto swz = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & (CPR - 1)); };
    const int kgrp = lane >> 4, tok = lane & 15;
    constexpr int NBUF = score_kbuf_pages(SPARSE, G, PS, D);
    unsigned char* kbuf = smem + lay.kbuf + (size_t)wave * NBUF * PB;

    // q split exactly into three bf16 parts, staged in LDS as rows
    // (head, part): each thread splits its q values, then lane l reads its A
    // fragments (row l%16 = (head, part), dims ks*32 + (l/16)*8 .. +8) with
    // 16-byte loads; rows past the group are zero.
    constexpr int QP = qtab_pitch(D);
    uint16_t* qtab = reinterpret_cast<uint16_t*>(smem + lay.qtab);
    if (tid < kNW * G) wmax[tid] = neg_inf<Acc>();  // the waves' shared running maxima
    // the call's shared maxima at the start, a floor under the filter level
    // (never a split maximum: those stay the maxima of the split's own
    // tokens, which the threshold step takes as distinct token scores)
    if (tid < G) {
      wfloor[tid] = gm ? order_float(gstart) : neg_inf<Acc>();
      wlb[tid] = gm ? order_float(gstartlb) : neg_inf<Acc>();
    }
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = k * kNT + tid;
      if (i >= G * D) break;
      const float x = qx[k];
      const uint32_t p0 = bf16_rne_bits(x);
      const float r1 = x - __uint_as_float(p0 << 16);
      const uint32_t p1 = bf16_rne_bits(r1);
      const uint32_t p2 = bf16_rne_bits(r1 - __uint_as_float(p1 << 16));
      uint16_t* row = qtab + (size_t)(i / D) * 3 * QP + (i % D);
      row[0] = (uint16_t)p0;
      row[QP] = (uint16_t)p1;
      row[2 * QP] = (uint16_t)p2;
    }
    __syncthreads();
    bf16x8 qa[NMB][KS];
#pragma unroll
    for (int blk = 0; blk < NMB; ++blk) {
      const int h = blk * 4 + ((lane & 15) >> 2), part = lane & 3;
      const bool live = h < G && part < 3;
      const uint16_t* row = qtab + (size_t)((live ? h : 0) * 3 + (live ? part : 0)) * QP + kgrp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + ks * 32);
        qa[blk][ks] = __builtin_bit_cast(bf16x8, live ? v : make_uint4(0u, 0u, 0u, 0u));
      }
    }
    // Source byte offset, within a page, of the chunk this lane stores in
    // load instruction i.
    int src_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = i * RPI + lane / CPR;
      src_off[i] = r * RB + (((lane % CPR) ^ swz(r)) * 16);
    }
    const uint64_t gmask = 0xffffull << (16 * kgrp);
    Acc M[NMB];
    int mycnt[NMB];
    // The filter level starts from the call's shared maxima (gfl, read
    // into wfloor before the barrier above) and never drops below the
    // call's shared lower bound on tau (glb, from wlb).
    Acc gfl[NMB], glb[NMB];
#pragma unroll
    for (int blk = 0; blk < NMB; ++blk) {
      const int h = blk * 4 + kgrp;
      M[blk] = neg_inf<Acc>();
      mycnt[blk] = 0;
      gfl[blk] = h < G ? wfloor[h] : neg_inf<Acc>();
      glb[blk] = h < G ? wlb[h] : neg_inf<Acc>();
    }
    // Page pp into buffer `bsel` (an invalid physical page, or a page past
    // the slice, reads page 0 of the pool; its scores are dropped). The loads
    // are issued on every path, so the waits below count them exactly.
    auto issue = [&](int pp, int bsel) {
      const int ph = pp < n_slice ? sphys[pp] : 0;
      const bool okp = ph >= 0 && ph < num_phys;
      const unsigned char* base = reinterpret_cast<const unsigned char*>(
          k_pool + ((size_t)(okp ? ph : 0) * Hkv + g) * (size_t)PS * D);
      unsigned char* dst = kbuf + bsel * PB;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        lds_load16(base + src_off[i], dst + i * 1024);
    };
    // Scores one page; returns the number of store instructions it issued
    // (spilled candidates), which the waits below must allow in flight:
    // vmcnt counts stores as well as loads.
    auto score_page = [&](int p, int bsel) -> int {
      int nst = 0;
      const int j = SPARSE ? slice[p] : split * pps + p;
      const int phys = sphys[p];
      const int nvalid = (phys >= 0 && phys < num_phys) ? min(PS, L - j * PS) : 0;
      int myslot[NMB];
#pragma unroll
      for (int blk = 0; blk < NMB; ++blk) {
        const int h = blk * 4 + kgrp;
        if constexpr (SPARSE) {
          int v = -1;
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            if (hh == h) v = slots[p * G + hh];
          myslot[blk] = v;
        } else {
          myslot[blk] = h < G ? j : -1;
        }
      }
      // The waves' running maxima of these heads (wmax[w][h], updated after
      // every page without a barrier; a read sees some earlier value, each
      // the maximum of some of this split's tokens): filtering against the
      // largest still keeps every token within the window of the split's
      // maximum, and far fewer others than a wave's own maximum would.
      // Plain 32/64-bit LDS accesses (single-copy atomic on the hardware);
      // atomic forms would lose the alias information that lets the
      // compiler skip waiting for the page loads in flight.
      Acc om[NMB];
#pragma unroll
      for (int blk = 0; blk < NMB; ++blk) {
        const int h = blk * 4 + kgrp;
        Acc v = neg_inf<Acc>();
#pragma unroll
        for (int w = 0; w < kNW; ++w)
          if (h < G) v = max(v, wmax[w * G + h]);
        om[blk] = max(v, gfl[blk]);
      }
      const unsigned char* src = kbuf + bsel * PB;
      Acc zz[TILES][NMB];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int row = t * 16 + tok;
        bf16x8 kv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kv[ks] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(
                          src + row * RB + (((ks * 4 + kgrp) ^ swz(row)) * 16)));
#pragma unroll
        for (int blk = 0; blk < NMB; ++blk) {
          f32x4 cacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[blk][ks], kv[ks], cacc, 0, 0, 0);
          const bool ok = row < nvalid && myslot[blk] >= 0;
          zz[t][blk] = ok ? (cacc[0] + cacc[1]) + cacc[2] : neg_inf<Acc>();
        }
      }
#pragma unroll
      for (int blk = 0; blk < NMB; ++blk) {
        Acc pm = zz[0][blk];
#pragma unroll
        for (int t = 1; t < TILES; ++t) pm = max(pm, zz[t][blk]);
        pm = max(pm, partner<1>(pm));
        pm = max(pm, partner<2>(pm));
        pm = max(pm, partner<4>(pm));
        pm = max(pm, partner<8>(pm));
        M[blk] = max(M[blk], pm);
        const Acc thr = max(max(M[blk], om[blk]) - window, glb[blk]);
        const int h = blk * 4 + kgrp;
        if (tok == 0 && h < G) wmax[wave * G + h] = M[blk];
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
          const Acc z = zz[t][blk];
          const bool f = z > neg_inf<Acc>() && z >= thr;
          const uint64_t bal = __ballot(f);
          const int pos = mycnt[blk] + __popcll(bal & gmask & ltm);
          const int ix = phys * PS + t * 16 + tok;
          if (f && pos < lists.slots) lists.put_lds(wave, h, G, pos, z, ix);
          // spilled entries: one store instruction for the wave, counted
          if (__ballot(f && pos >= lists.slots) != 0ull) {
            ++nst;
            if (f && pos >= lists.slots) lists.put_spill(wave, h, G, pos, z, ix);
          }
          mycnt[blk] += __popcll(bal & gmask);
        }
      }
      return nst;
    };
    if constexpr (NBUF == 2) {
      // Two page buffers alternate, each refilled as soon as its page has
      // been read, so two pages are in flight while one is scored. Before a
      // buffer is read, only the other buffer's NI loads and the stores of
      // the page scored in between may be outstanding (vmcnt completes in
      // issue order).
      issue(wave, 0);
      issue(wave + kNW, 1);
      int nst = 0;
      for (int p = wave; p < n_slice; p += 2 * kNW) {
        wait_vmcnt_plus<NI>(nst);
        nst = score_page(p, 0);
        issue(p + 2 * kNW, 0);
        if (p + kNW >= n_slice) break;
        wait_vmcnt_plus<NI>(nst);
        nst = score_page(p + kNW, 1);
        issue(p + 3 * kNW, 1);
      }
      // the shared maxima once more, for the workgroup pass below (lane h
      // of every wave holds head h's), waited for with the page loads
      if (gm && lane < G) {
        gkey = __hip_atomic_load(gm + (size_t)(bh0 + lane) * kMaxStride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        gkeylb = __hip_atomic_load(gm + (size_t)(bh0 + lane) * kMaxStride + 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_vmcnt<0>();  // no load into LDS is left in flight
    } else {
      // One buffer: short slices (the sparse path) keep more workgroups
      // resident instead.
      for (int p = wave; p < n_slice; p += kNW) {
        issue(p, 0);
        wait_vmcnt<0>();
        score_page(p, 0);
      }
    }
#pragma unroll
    for (int blk = 0; blk < NMB; ++blk) {
      const int h = blk * 4 + kgrp;
      if (tok == 0 && h < G) {
        wmax[wave * G + h] = M[blk];
        wcnt[wave * G + h] = mycnt[blk];
      }
    }
  } else {
    // Vector-ALU scores: a token row is spread over LT lanes, each holding
    // NCH 16-byte chunks; the G partial dot products finish in a multi-value
    // butterfly.
    constexpr int VPC = Tr::VPC;
    constexpr int NCH = kScoreChunks;
    constexpr int LT = D / (NCH * VPC);  // lanes per token row
    constexpr int RW = kWave / LT;       // rows per wave step
    static_assert(PS % RW == 0, "page must hold whole wave steps");
    constexpr int STEPS = PS / RW;
    using BF = Butterfly<G, LT>;
    constexpr int CNT = BF::CNT;
    const int c = lane % LT;
    const int rsub = lane / LT;
    Acc qv[G][NCH][VPC];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* qh = q + (size_t)(bh0 + h) * D;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int e = 0; e < VPC; ++e) qv[h][ch][e] = (Acc)qh[ch * (D / NCH) + c * VPC + e];
    }
    const int first = BF::first_index(lane);
    const bool owner = BF::owner(lane);
    uint64_t mymask[CNT];
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      mymask[i] = 0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint64_t m = __ballot(owner && (first + i) == h);
        if (first + i == h) mymask[i] = m;
      }
    }
    Acc M[CNT];
    int mycnt[CNT];
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      M[i] = neg_inf<Acc>();
      mycnt[i] = 0;
    }
    for (int p = wave; p < n_slice; p += kNW) {
      const int j = SPARSE ? slice[p] : split * pps + p;
      const int phys = sphys[p];
      if (phys < 0 || phys >= num_phys) continue;
      const int nvalid = min(PS, L - j * PS);
      int myslot[CNT];
#pragma unroll
      for (int i = 0; i < CNT; ++i) {
        if constexpr (SPARSE) {
          int v = -1;
#pragma unroll
          for (int h = 0; h < G; ++h)
            if (first + i == h) v = slots[p * G + h];
          myslot[i] = v;
        } else {
          myslot[i] = j;
        }
      }
      const KV* base = k_pool + ((size_t)phys * Hkv + g) * (size_t)PS * D;
      uint4 x[STEPS][NCH];
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const KV* rp = base + (size_t)(s * RW + rsub) * D;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) x[s][ch] = stream_load16(rp + ch * (D / NCH) + c * VPC);
      }
      Acc zz[STEPS][CNT];
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        Acc acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          Acc f[VPC];
          widen<KV>(x[s][ch], f);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            Acc a = 0;
#pragma unroll
            for (int e = 0; e < VPC; ++e) a = fma(qv[h][ch][e], f[e], a);
            acc[h] += a;
          }
        }
        BF::reduce(acc, lane);
#pragma unroll
        for (int i = 0; i < CNT; ++i) zz[s][i] = acc[i];
      }
      // mask invalid rows and heads that did not select this page
      Acc pm[CNT];
#pragma unroll
      for (int i = 0; i < CNT; ++i) {
        pm[i] = neg_inf<Acc>();
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          const bool ok = owner && (s * RW + rsub) < nvalid && myslot[i] >= 0;
          if (!ok) zz[s][i] = neg_inf<Acc>();
          pm[i] = max(pm[i], zz[s][i]);
        }
#pragma unroll
        for (int w = LT; w < kWave; w <<= 1) pm[i] = max(pm[i], shfl_xor(pm[i], w));
#pragma unroll
        for (int w = 1; w < BF::DUP; w <<= 1) pm[i] = max(pm[i], shfl_xor(pm[i], w));
        M[i] = max(M[i], pm[i]);
      }
#pragma unroll
      for (int i = 0; i < CNT; ++i) {
        const Acc thr = M[i] - window;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          const Acc z = zz[s][i];
          const bool f = z > neg_inf<Acc>() && z >= thr;
          const uint64_t bal = __ballot(f);
          if (f)
            lists.put(wave, first + i, G, mycnt[i] + __popcll(bal & mymask[i] & ltm), z,
                      phys * PS + s * RW + rsub);
          mycnt[i] += __popcll(bal & mymask[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      if (owner && rsub == 0) {
        wmax[wave * G + first + i] = M[i];
        wcnt[wave * G + first + i] = mycnt[i];
      }
    }
  }
  __syncthreads();

  // Workgroup pass: keep the candidates within the window of the workgroup
  // maximum, in (wave, page) order, as this split's region of each head.
  const bool shared = !SPARSE && MFMA && args.gmax != nullptr;
  for (int h = wave; h < G; h += kNW) {
    Acc mg = neg_inf<Acc>();
#pragma unroll
    for (int w = 0; w < kNW; ++w) mg = max(mg, wmax[w * G + h]);
    Acc mf = mg;  // filter level: this split's maximum or the call's, if larger
    if (shared) {
      const uint32_t key = lane_value(gkey, h);
      if (key > float_order((float)mg)) mf = (Acc)order_float(key);
    }
    Acc thr = mf - window;
    if (shared) thr = max(thr, (Acc)order_float(lane_value(gkeylb, h)));
    const size_t r = (size_t)(bh0 + h) * splits + split;
    Cand<Acc>* dst = cand + r * (size_t)cap;
    // The waves' lists, concatenated in wave order, are read kWave *
    // kPassRegs entries at a time with every read of a batch issued before
    // the first is used (spilled entries then cost one round trip per batch,
    // not one per 64 entries).
    int nb[kNW + 1];  // list starts in the concatenation
    nb[0] = 0;
    int nsp = 0;      // spilled entries of this head
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const int n = wcnt[w * G + h];
      nb[w + 1] = nb[w] + n;
      nsp += max(0, n - lists.slots);
    }
    const int ntot = nb[kNW];
    // entries base + k * 64 + lane of the concatenation (past the end: its
    // last entry) into zr / ir
    auto load_batch = [&](int base, Acc (&zr)[kPassRegs], int (&ir)[kPassRegs]) {
      int pr[kPassRegs];
      Cand<Acc> cs[kPassRegs];
#pragma unroll
      for (int k = 0; k < kPassRegs; ++k) {
        const int t = min(base + k * kWave + lane, ntot - 1);
        int w = 0;
#pragma unroll
        for (int v = 1; v < kNW; ++v) w += (t >= nb[v]) ? 1 : 0;
        const int pos = t - nb[w];
        pr[k] = pos;
        const int lo = (w * G + h) * lists.slots + min(pos, lists.slots - 1);
        zr[k] = lists.rz[lo];
        ir[k] = lists.ri[lo];
        if (nsp > 0)  // (uniform) the spill slot, or the area's first slot
          cs[k] = lists.spill[pos >= lists.slots
                                  ? (size_t)(w * G + h) * lists.wcap + (pos - lists.slots)
                                  : 0];
      }
#pragma unroll
      for (int k = 0; k < kPassRegs; ++k) {
        if (nsp > 0 && pr[k] >= lists.slots) {
          zr[k] = cs[k].z;
          ir[k] = cs[k].idx;
        }
      }
    };
    if constexpr (MFMA) {
      if (args.local_bound && ntot > 0) {
        // The threshold t_S of any set S of the head's tokens is at most tau
        // (the left side of the threshold equation only grows with more
        // tokens), so every support token has a = (alpha-1) z > t_S. S = the
        // first kWave * kPassRegs candidates above the filter level, solved
        // in this wave's registers; the filter level rises to t_S (less a
        // relative 1e-6 for rounding) and, with shared maxima, so does the
        // call's shared bound of the head.
        Acc zr[kPassRegs];
        int ir[kPassRegs];
        load_batch(0, zr, ir);
        const double am1 = (double)args.alpha - 1.0;
        const double m = 1.0 / am1;
        const int mcode = (m == 1.0) ? 1 : (m == 2.0) ? 2 : (m == 3.0) ? 3 : (m == 4.0) ? 4 : 0;
        double av[kPassRegs];
        double amx = -DBL_MAX;
#pragma unroll
        for (int k = 0; k < kPassRegs; ++k) {
          const bool ok = k * kWave + lane < ntot && zr[k] >= thr;
          av[k] = ok ? am1 * (double)zr[k] : -DBL_MAX;
          amx = fmax(amx, av[k]);
        }
        amx = wave_max(amx);
        if (amx > -DBL_MAX) {
          const double ts = with_mcode(mcode, [&](auto mc) {
            return solve_tau_regs<kPassRegs, decltype(mc)::value>(
                av, min(ntot, kWave * kPassRegs), am1, m, mcode, amx);
          });
          const Acc lbz = (Acc)((ts - 1e-6 * fmax(1.0, fabs(ts))) / am1);
          if (lbz > thr) {
            thr = lbz;
            if (shared && lane == 0)
              __hip_atomic_fetch_max(args.gmax + (size_t)(bh0 + h) * kMaxStride + 1,
                                     float_order((float)lbz), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    int o = 0;
    for (int base = 0; base < ntot; base += kWave * kPassRegs) {
      Acc zr[kPassRegs];
      int ir[kPassRegs];
      load_batch(base, zr, ir);
#pragma unroll
      for (int k = 0; k < kPassRegs; ++k) {
        const bool f = base + k * kWave + lane < ntot && zr[k] >= thr;
        const uint64_t bal = __ballot(f);
        if (f) {
          Cand<Acc> cv;
          cv.z = zr[k];
          cv.idx = ir[k];
          dst[o + __popcll(bal & ltm)] = cv;
        }
        o += __popcll(bal);
      }
    }
    if (lane == 0) put_count(r, o, mg);
    // raise the call's shared maximum of the head to this split's, last
    // (nothing waits for the atomic: later workgroups see it when it lands)
    if (shared && lane == 0 && mg > neg_inf<Acc>())
      __hip_atomic_fetch_max(args.gmax + (size_t)(bh0 + h) * kMaxStride, float_order((float)mg),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename KV, int D, int G, int PS, bool SPARSE>
__global__ void __launch_bounds__(kNT)
score_kernel(ScoreArgs<KV> args) {
  extern __shared__ __align__(16) unsigned char smem[];
  score_split<KV, D, G, PS, SPARSE>(args, blockIdx.x / args.U, blockIdx.x % args.U, smem);
}

// ---------------------------------------------------------------------------
// threshold and P.V kernel

// One batch of the threshold kernel's gather (see there): thread t takes
// entries [bbase + t*per, bbase + t*per + per) of the head's concatenated
// candidate regions, per <= R; returns the window members counted so far.
template <typename ZT>
struct GatherArgs {
  const int* roff;
  const Cand<ZT>* creg;
  int splits, cap;
  ZT thr;
  ZT* lz;
  int* li;
  ZT* gz;
  int* gi;
  int lcap;
  int* tmp;
};
template <int R, typename ZT>
__device__ __forceinline__ int gather_batch(const GatherArgs<ZT>& a, int bbase, int nb, int n_list) {
  const int tid = threadIdx.x;
  const int per = (nb + kNT - 1) / kNT;
  const int e0 = bbase + min(nb, tid * per), e1 = bbase + min(nb, tid * per + per);
  // Offsets first (LDS only), then every load unconditionally and
  // branch-free, so all of them are in flight before the first is used
  // (slots past the run reload its last entry, or entry 0 of region 0).
  int off[R];  // < regions * cap: the head's gathered tokens (< 2^31)
  {
    const int ef = e0 < e1 ? e0 : 0;
    int lo = 0, hi = a.splits;  // roff[lo] <= ef < roff[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.roff[mid] <= ef) lo = mid;
      else hi = mid;
    }
    int r = lo, rbeg = a.roff[lo], rend = a.roff[lo + 1];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int e = e0 + k < e1 ? e0 + k : (e0 < e1 ? e1 - 1 : 0);
      while (e >= rend && r + 1 < a.splits) {  // next non-empty region (LDS read on crossings)
        ++r;
        rbeg = rend;
        rend = a.roff[r + 1];
      }
      off[k] = r * a.cap + (e - rbeg);
    }
  }
  Cand<ZT> v[R];
#pragma unroll
  for (int k = 0; k < R; ++k) v[k] = ld_global_cand(a.creg + off[k]);
  int keep = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) keep += (e0 + k < e1 && v[k].z >= a.thr) ? 1 : 0;
  int kept;
  int pos = n_list + block_excl_scan<kNT>(keep, a.tmp, &kept);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (e0 + k < e1 && v[k].z >= a.thr) {
      if (pos < a.lcap) {
        a.lz[pos] = v[k].z;
        a.li[pos] = v[k].idx;
      } else {
        a.gz[pos] = v[k].z;
        a.gi[pos] = v[k].idx;
      }
      ++pos;
    }
  }
  return n_list + kept;
}

// LDS of the threshold kernel: region offsets, `lcap` window members
// (score, V row, weight), the P.V partial rows and the region maxima used for
// the lower bound. Longer lists take a global-memory path.
constexpr int kTauMaxList = 8192;  // most window members one workgroup holds in LDS
constexpr int kTauBoundFrom = 2048;  // candidates from which the window is tightened first
struct TauLds {
  size_t lz, li, sp, pv, rmax, total;
};
__host__ __device__ inline TauLds tau_lds_layout(int regions, int lcap, int zbytes, int ng,
                                                 int D) {
  TauLds l;
  size_t o = align16((size_t)(regions + 1) * 4);
  l.lz = o; o = align16(o + (size_t)lcap * zbytes);
  l.li = o; o = align16(o + (size_t)lcap * 4);
  l.sp = o; o = align16(o + (size_t)lcap * 4);
  l.pv = o; o = align16(o + (size_t)ng * D * 4);
  l.rmax = o; o = align16(o + (size_t)kNT * 8);
  l.total = o;
  return l;
}

// Arguments of the threshold + P.V step.
// The threshold kernel's rarely taken steps (many candidates, long window
// lists, lists beyond the LDS capacity) are out-of-line functions: the
// common step (a short list solved by one wave) then runs through a compact
// block of instructions, which matters when the kernel starts with a cold
// instruction cache.
struct TauSolution {
  double tau, psum;
  int n_sup;
};

// A generic pointer that points into LDS, re-qualified so that accesses
// through it compile to LDS instructions inside an out-of-line function
// (where the compiler cannot see where the pointer came from).
template <typename T>
__device__ __forceinline__ T* lds_view(T* p) {
#if __HIP_DEVICE_COMPILE__  // (the builtin exists in the device pass only)
  __builtin_assume(__builtin_amdgcn_is_shared((const void*)p));
#endif
  return p;
}

// Gather runs of more than 8 entries per thread (batches of over 2048
// candidates). The arguments come one by one (an aggregate argument would
// pass through scratch memory).
template <int R, typename ZT>
__device__ __attribute__((noinline)) int gather_batch_wide(const int* roff, const Cand<ZT>* creg,
                                                           int splits, int cap, ZT thr, ZT* lz,
                                                           int* li, ZT* gz, int* gi, int lcap,
                                                           int* tmp, int bbase, int nb,
                                                           int n_list) {
  const GatherArgs<ZT> a{lds_view(roff), creg, splits, cap, thr, lds_view(lz), lds_view(li),
                         gz, gi, lcap, lds_view(tmp)};
  return gather_batch<R>(a, bbase, nb, n_list);
}

// Lower bound on tau from a subset of the head's tokens. The threshold t_S of
// any subset S is at most tau (the left side of the threshold equation only
// grows when tokens are added, and it decreases in t); S = the per-thread
// maxima of the region maxima (up to 256 token scores), solved by wave 0 in
// registers. Every support token has a > t_S, so the window may start at
// t_S - 1e-6 max(1, |t_S|) (returned in score units, z = a / (alpha - 1)).
template <typename ZT>
__device__ __attribute__((noinline)) ZT tau_window_bound(ZT mloc, double* rmax, double* tau_b,
                                                         double am1, double m, int mcode,
                                                         double amax) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  rmax = lds_view(rmax);
  tau_b = lds_view(tau_b);
  rmax[tid] = mloc == neg_inf<ZT>() ? -DBL_MAX : am1 * (double)mloc;
  __syncthreads();
  if (tid < kWave) {
    double a[kRegList];
#pragma unroll
    for (int k = 0; k < kRegList; ++k) a[k] = rmax[k * kWave + lane];
    const double ts = with_mcode(mcode, [&](auto mc) {
      return solve_tau_regs<kRegList, decltype(mc)::value>(a, kRegList * kWave, am1, m, mcode,
                                                           amax);
    });
    if (lane == 0) *tau_b = ts;
  }
  __syncthreads();
  const double ts = *tau_b;
  return (ZT)((ts - 1e-6 * fmax(1.0, fabs(ts))) / am1);
}

// Window lists in LDS too long for one wave: thread t holds the contiguous
// entries [t*per, t*per + per) (per <= KB) in registers for the whole solve,
// and one block scan compacts the support's (V row, p) to the front of
// (li, sp) in list order. Every thread of the workgroup calls it.
template <typename ZT, int KB, int NT>
__device__ __attribute__((noinline)) TauSolution tau_long_list(const ZT* lz, int* li, float* sp,
                                                               int n_list, double am1, double m,
                                                               int mcode, double amax, double* red,
                                                               int* tmp, double tlo) {
  const int tid = threadIdx.x;
  lz = lds_view(lz);
  li = lds_view(li);
  sp = lds_view(sp);
  red = lds_view(red);
  tmp = lds_view(tmp);
  TauSolution r;
  const int per = (n_list + NT - 1) / NT;
  const int e0 = min(n_list, tid * per), e1 = min(n_list, e0 + per);
  double a[KB];
#pragma unroll
  for (int k = 0; k < KB; ++k) a[k] = (e0 + k < e1) ? am1 * (double)lz[e0 + k] : -DBL_MAX;
  const double tau = with_mcode(mcode, [&](auto mc) {
    return solve_tau_block<KB, decltype(mc)::value, NT>(a, per, m, mcode, amax, red, tlo);
  });
  int ns = 0;
#pragma unroll
  for (int k = 0; k < KB; ++k) ns += (a[k] - tau > 0.0) ? 1 : 0;
  int ix[KB];
#pragma unroll
  for (int k = 0; k < KB; ++k) ix[k] = (e0 + k < e1) ? li[e0 + k] : 0;
  int base = block_excl_scan<NT>(ns, tmp, &r.n_sup);  // (its barriers order the reads above)
  double psum = 0.0;
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const double d = a[k] - tau;
    if (d > 0.0) {
      const double pv = pow_m(d, m, mcode);
      psum += pv;
      li[base] = ix[k];
      sp[base] = (float)pv;
      ++base;
    }
  }
  double zero = 0.0;
  scope_sum2<NT>(psum, zero, red);
  r.tau = tau;
  r.psum = psum;
  return r;
}

// A window list in LDS longer than one wave's registers hold (integer m):
// a few block-wide Newton steps from the left raise the lower bound on tau
// (each iterate with f(t) >= 1 is at most tau), then the entries at or below
// it, which take no part in the threshold or the output, are dropped and the
// rest compacted to the front in list order. Repeated while the list is
// longer than kWave * kRegListLong and the steps make progress. Returns the
// new length; *tlo gets the bound. Every thread of the workgroup calls it.
template <typename ZT, int KB, int NT>
__device__ __attribute__((noinline)) int tau_prune_list(ZT* lz, int* li, int n_list, double am1,
                                                        double m, int mcode, double amax,
                                                        double* red, int* tmp, double* tlo) {
  const int tid = threadIdx.x;
  lz = lds_view(lz);
  li = lds_view(li);
  red = lds_view(red);
  tmp = lds_view(tmp);
  constexpr int kSteps = 3;
  double lo = fmax(amax - 1.0, *tlo);
  for (int round = 0; round < 4 && n_list > kWave * kRegListLong; ++round) {
    const int per = (n_list + NT - 1) / NT;
    const int e0 = min(n_list, tid * per), e1 = min(n_list, e0 + per);
    const double lo0 = lo;
    int ns = 0;
    {
      double a[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) a[k] = e0 + k < e1 ? am1 * (double)lz[e0 + k] : -DBL_MAX;
      double t = lo;
      for (int it = 0; it < kSteps; ++it) {
        double f = 0.0, fp = 0.0;
        with_mcode<true>(mcode, [&](auto mc) {
#pragma unroll
          for (int k = 0; k < KB; ++k)
            if (k < per) add_terms<decltype(mc)::value>(a[k] - t, m, mcode, f, fp);
        });
        scope_sum2<NT>(f, fp, red);
        fp *= m;
        if (!(f >= 1.0) || !(fp > 0.0)) break;  // (not left of the root)
        lo = t;
        if (f == 1.0) break;
        t = tau_step(t, f, fp, m, mcode);
        if (!(t < amax)) break;
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) ns += (a[k] > lo) ? 1 : 0;
    }
    int kept;
    int base = block_excl_scan<NT>(ns, tmp, &kept);
    // every thread reads its run before any is overwritten
    ZT zv[KB];
    int iv[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      zv[k] = e0 + k < e1 ? lz[e0 + k] : (ZT)0;
      iv[k] = e0 + k < e1 ? li[e0 + k] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      if (e0 + k < e1 && am1 * (double)zv[k] > lo) {
        lz[base] = zv[k];
        li[base] = iv[k];
        ++base;
      }
    }
    __syncthreads();
    const bool progress = kept < n_list && lo > lo0;
    n_list = kept;
    if (!progress) break;
  }
  *tlo = lo;
  return n_list;
}

// A window list in global memory (longer than the LDS capacity): the
// block-wide Newton solve over it, the support size and the sum of p.
template <typename ZT, int NT>
__device__ __attribute__((noinline)) TauSolution tau_global_list(const ZT* dz, int n_list,
                                                                 double am1, double m, int mcode,
                                                                 double amax, double* red,
                                                                 double tlo) {
  const int tid = threadIdx.x;
  red = lds_view(red);
  TauSolution r;
  r.tau = solve_tau<NT>(dz, n_list, am1, m, mcode, amax, tid, red, tlo);
  int ns = 0;
  double psum = 0.0;
  for (int i = tid; i < n_list; i += NT) {
    const double d = am1 * (double)dz[i] - r.tau;
    if (d > 0.0) {
      ++ns;
      psum += pow_m(d, m, mcode);
    }
  }
  double nsd = (double)ns;
  scope_sum2<NT>(psum, nsd, red);
  r.psum = psum;
  r.n_sup = (int)nsd;
  return r;
}

// P.V over a global-memory window list: thread (grp, c) accumulates the
// weighted 16-byte slice c of every grp-th support row and writes its partial
// sums to prow.
template <typename KV, int D, int NT>
__device__ __attribute__((noinline)) void pv_global_list(const KV* v_pool, int Hkv, int g, int PS,
                                                         const typename KvTraits<KV>::Acc* dz,
                                                         const int* di, int n_list, double am1,
                                                         double m, int mcode, double tau,
                                                         float* prow) {
  constexpr int VPC = 16 / sizeof(KV);
  constexpr int LR = D / VPC;
  constexpr int NG = NT / LR;
  const int grp = threadIdx.x / LR, c = threadIdx.x % LR;
  float acc[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) acc[e] = 0.0f;
  for (int i = grp; i < n_list; i += NG) {
    const double d = am1 * (double)dz[i] - tau;
    if (d > 0.0) {
      const int vrow = di[i];
      const int phys = vrow / PS, rr = vrow - phys * PS;
      const uint4 x = *reinterpret_cast<const uint4*>(
          v_pool + (((size_t)phys * Hkv + g) * PS + rr) * D + c * VPC);
      typename KvTraits<KV>::Acc f[VPC];
      widen<KV>(x, f);
      const float pk = (float)pow_m(d, m, mcode);
#pragma unroll
      for (int e = 0; e < VPC; ++e) acc[e] = fmaf(pk, (float)f[e], acc[e]);
    }
  }
  prow = lds_view(prow);
#pragma unroll
  for (int e = 0; e < VPC; ++e) prow[e] = acc[e];
}

// The window list's threshold, support and output for one head, by a
// workgroup of NT threads (every thread calls it, after a barrier that
// orders the list's writes): the list is (lz, li) in LDS, n_list entries
// (score, V row); when n_list > lcap the first lcap entries are in LDS and
// the rest already in (gz, gi) at the same positions, and the whole list
// moves there. Solves tau (one wave in registers for up to 256 entries, or
// 1024 at integer m; the workgroup beyond), then o = sum p v / sum p from
// the support's V rows, written to out_row[0, D); tau and the support size
// to *tau_p and *sup_p when not null. pvbase: NT / (D / VPC) rows of D
// floats of LDS.
template <int NT>
struct TauShared {
  double red[2 * (NT / kWave)];
  int tmp[NT / kWave + 2];
  double tau_b;
  int nb[2];
};
template <typename KV, int D, int NT>
__device__ __forceinline__ void tau_solve_pv(
    const KV* __restrict__ v_pool, int Hkv, int g, int PS, typename KvTraits<KV>::Acc* lz,
    int* li, float* sp, float* pvbase, int n_list, int lcap, typename KvTraits<KV>::Acc* gz,
    int* gi, double am1, double m, int mcode, double amax, TauShared<NT>& sh,
    float* __restrict__ out_row, float* tau_p, int32_t* sup_p, double tlo) {
  using ZT = typename KvTraits<KV>::Acc;
  constexpr int VPC = 16 / sizeof(KV);
  constexpr int LR = D / VPC;     // lanes per V row
  constexpr int NG = NT / LR;     // rows in flight per pass
  constexpr int KB = kTauMaxList / NT;  // most list entries per thread in block-wide steps
  float (*pvacc)[D] = reinterpret_cast<float (*)[D]>(pvbase);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint64_t ltm = lanemask_below(lane);
  ZT* dz = lz;
  int* di = li;
  if (n_list > lcap) {
    // the whole list goes to global memory
    for (int i = tid; i < lcap; i += NT) {
      gz[i] = lz[i];
      gi[i] = li[i];
    }
    __syncthreads();
    dz = gz;
    di = gi;
  }
  const bool list_lds = dz == lz;

  // A candidate's index is its V row, physical_page * page_size + row; thread
  // (grp, c) handles 16-byte slice c of rows grp, grp + NG, ...
  const int grp = tid / LR, c = tid % LR;
  auto row_ptr = [&](int vrow) -> const KV* {
    const int phys = vrow / PS, r = vrow - phys * PS;
    return v_pool + (((size_t)phys * Hkv + g) * PS + r) * D + c * VPC;
  };
  // Short lists (up to kVPre entries, the common case): the V rows of every
  // list entry are requested now, so that their latency overlaps the solve;
  // the P.V step then weights the rows it holds (p = 0 off the support).
  constexpr int kVPre = 32;
  constexpr int NPRE = (kVPre + NG - 1) / NG;
  const bool vpre = list_lds && n_list >= 1 && n_list <= NPRE * NG;
  uint4 vrow[NPRE];
  if (vpre) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int k = min(grp + i * NG, n_list - 1);
      vrow[i] = *reinterpret_cast<const uint4*>(row_ptr(li[k]));
    }
  }

  // Threshold, support (a_i > tau) with p_i = (a_i - tau)^m, sum p in float64.
  double tau;
  int n_sup;
  double psum = 0.0;
  if (list_lds && mcode != 0 && n_list > kWave * 2 * kRegListLong)
    n_list = tau_prune_list<ZT, KB, NT>(lz, li, n_list, am1, m, mcode, amax, sh.red, sh.tmp, &tlo);

  if (list_lds && n_list <= kWave * kRegList) {
    // Short lists (up to 256): wave 0 holds a_i = am1 * z_i in registers for
    // the whole solve (no barrier per iteration), then compacts (V row, p)
    // in list order.
    if (wave == 0) {
      int o;
      double t;
      // With the V rows requested up front the P.V step weights them from
      // lz, and the other waves' reads of li may still be in flight, so the
      // support is not compacted into li.
      with_mcode(mcode, [&](auto mc) {
        wave_solve_list<kRegList, decltype(mc)::value>(lz, li, sp, n_list, am1, m, mcode, amax,
                                                       lane, ltm, !vpre, o, psum, t, tlo);
      });
      if (lane == 0) {
        sh.nb[1] = o;
        sh.red[0] = psum;
        sh.tau_b = t;
      }
    }
    __syncthreads();
    tau = sh.tau_b;
    n_sup = sh.nb[1];
    psum = sh.red[0];
  } else if (list_lds && n_list <= kWave * 2 * kRegListLong && mcode != 0) {
    // Up to 2048 entries at integer m: the same by wave 0 with 16 entries
    // per lane, or 32 beyond 1024 (no barrier per iteration, no call to the
    // general power).
    if (wave == 0) {
      int o;
      double t;
      with_mcode<true>(mcode, [&](auto mc) {
        if (n_list <= kWave * kRegListLong)
          wave_solve_list<kRegListLong, decltype(mc)::value>(
              lz, li, sp, n_list, am1, m, mcode, amax, lane, ltm, true, o, psum, t, tlo);
        else
          wave_solve_list<2 * kRegListLong, decltype(mc)::value>(
              lz, li, sp, n_list, am1, m, mcode, amax, lane, ltm, true, o, psum, t, tlo);
      });
      if (lane == 0) {
        sh.nb[1] = o;
        sh.red[0] = psum;
        sh.tau_b = t;
      }
    }
    __syncthreads();
    tau = sh.tau_b;
    n_sup = sh.nb[1];
    psum = sh.red[0];
  } else {
    // Longer lists, out of line: up to the LDS capacity by the workgroup,
    // beyond it from global memory.
    const TauSolution r = list_lds ? tau_long_list<ZT, KB, NT>(lz, li, sp, n_list, am1, m, mcode, amax,
                                                          sh.red, sh.tmp, tlo)
                                   : tau_global_list<ZT, NT>(dz, n_list, am1, m, mcode, amax, sh.red,
                                                             tlo);
    tau = r.tau;
    n_sup = r.n_sup;
    psum = r.psum;
  }

  // o = sum p v / sum p.
  float acc[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) acc[e] = 0.0f;
  auto accumulate_x = [&](const uint4& x, float pk) {
    typename KvTraits<KV>::Acc f[VPC];
    widen<KV>(x, f);
#pragma unroll
    for (int e = 0; e < VPC; ++e) acc[e] = fmaf(pk, (float)f[e], acc[e]);
  };
  if (vpre) {
    // p from the list's scores (z is not moved by the support compaction),
    // by the same expression the solve summed
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int k = grp + i * NG;
      if (k < n_list) {
        const double d = am1 * (double)lz[k] - tau;
        if (d > 0.0) accumulate_x(vrow[i], (float)(d * pow_m1(d, m, mcode)));
      }
    }
#pragma unroll
    for (int e = 0; e < VPC; ++e) pvacc[grp][c * VPC + e] = acc[e];
  } else if (list_lds) {
    // the support's rows in batches of RPT per thread (rows grp, grp + NG,
    // ...), every load of a batch issued before the first is used (slots
    // past the support re-read its last row with weight 0; every use is
    // unconditional, so no load is moved into a branch), so a support of up
    // to RPT * NG rows costs one round trip
    constexpr int RPT = 4096 / NT;
    for (int k0 = grp; k0 < n_sup; k0 += RPT * NG) {
      uint4 x[RPT];
      float pk[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int k = min(k0 + i * NG, n_sup - 1);
        x[i] = *reinterpret_cast<const uint4*>(row_ptr(li[k]));
        pk[i] = k0 + i * NG < n_sup ? sp[k] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) accumulate_x(x[i], pk[i]);
    }
#pragma unroll
    for (int e = 0; e < VPC; ++e) pvacc[grp][c * VPC + e] = acc[e];
  } else {
    pv_global_list<KV, D, NT>(v_pool, Hkv, g, PS, dz, di, n_list, am1, m, mcode, tau,
                          &pvacc[grp][c * VPC]);
  }
  __syncthreads();
  const double inv = psum > 0.0 ? 1.0 / psum : 0.0;
  for (int d = tid; d < D; d += NT) {
    float sacc = 0.0f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) sacc += pvacc[gg][d];
    out_row[d] = (float)((double)sacc * inv);
  }
  if (tid == 0) {
    if (tau_p) *tau_p = (float)tau;
    if (sup_p) *sup_p = n_sup;
  }
}


template <typename KV>
struct TauArgs {
  const KV* v_pool;
  int H, Hkv, G, U, PS, splits, cap, list_cap, lcap;
  float alpha;
  double window_d;
  const Cand<typename KvTraits<KV>::Acc>* cand;
  const int* counts;
  const typename KvTraits<KV>::Acc* maxima;
  typename KvTraits<KV>::Acc* list_z;
  int* list_i;
  float* out;
  float* tau_out;
  int32_t* sup_out;
  // the score step's per-head lines of shared maxima (word 1: its shared
  // lower bound on tau), or null when it shares none
  const uint32_t* glb;
};

// One query head (unit u, head hh of its group), by the whole workgroup.
template <typename KV, int D>
__device__ __forceinline__ void tau_head(const TauArgs<KV>& args, int u, int hh, unsigned char* smem) {
  using ZT = typename KvTraits<KV>::Acc;
  const KV* __restrict__ v_pool = args.v_pool;
  const int H = args.H, Hkv = args.Hkv, G = args.G, PS = args.PS, splits = args.splits;
  const int cap = args.cap, list_cap = args.list_cap, lcap = args.lcap;
  const float alpha = args.alpha;
  const Cand<ZT>* __restrict__ cand = args.cand;
  const int* __restrict__ counts = args.counts;
  const ZT* __restrict__ maxima = args.maxima;
  ZT* __restrict__ list_z = args.list_z;
  int* __restrict__ list_i = args.list_i;
  float* __restrict__ out = args.out;
  float* __restrict__ tau_out = args.tau_out;
  int32_t* __restrict__ sup_out = args.sup_out;
  const ZT window = (ZT)args.window_d;
  constexpr int VPC = 16 / sizeof(KV);
  constexpr int LR = D / VPC;     // lanes per V row
  constexpr int NG = kNT / LR;    // rows in flight per pass
  constexpr int KB = kTauMaxList / kNT;  // most entries per thread in a gather batch
  const TauLds lay = tau_lds_layout(splits, lcap, sizeof(ZT), NG, D);
  int* roff = reinterpret_cast<int*>(smem);  // region offsets
  ZT* lz = reinterpret_cast<ZT*>(smem + lay.lz);
  int* li = reinterpret_cast<int*>(smem + lay.li);
  float* sp = reinterpret_cast<float*>(smem + lay.sp);
  float (*pvacc)[D] = reinterpret_cast<float (*)[D]>(smem + lay.pv);
  double* rmax = reinterpret_cast<double*>(smem + lay.rmax);  // kNT doubles
  __shared__ ZT fred[kNW];
  __shared__ TauShared<kNT> tsh;
  int* tmp = tsh.tmp;

  const int tid = threadIdx.x;
  const int b = u / Hkv, g = u % Hkv;
  const int h = g * G + hh;
  const int bh = b * H + h;
  const ZT* mx = maxima + (size_t)bh * splits;
  const int* cn = counts + (size_t)bh * splits;
  const Cand<ZT>* creg = cand + (size_t)bh * splits * cap;
  // the score step's shared lower bound on tau (order key; -inf without one)
  const uint32_t glb_key = args.glb ? args.glb[(size_t)bh * kMaxStride + 1] : 0x007fffffu;
  const double am1 = (double)alpha - 1.0;
  const double m = 1.0 / am1;
  const int mcode = (m == 1.0) ? 1 : (m == 2.0) ? 2 : (m == 3.0) ? 3 : (m == 4.0) ? 4 : 0;

  // Region counts and maxima: every thread loads its contiguous block of
  // regions at once; one block scan turns counts into offsets.
  const int cpt = (splits + kNT - 1) / kNT;
  const int r0 = min(splits, tid * cpt), r1 = min(splits, r0 + cpt);
  int s = 0;
  ZT mloc = neg_inf<ZT>();
  for (int r = r0; r < r1; ++r) {
    const int c = cn[r];
    roff[r] = c;
    s += c;
    mloc = max(mloc, mx[r]);
  }
  const ZT M = block_reduce<kNT>(mloc, fred, [](ZT a, ZT c) { return max(a, c); });
  int n_cand;
  {
    int base = block_excl_scan<kNT>(s, tmp, &n_cand);
    for (int r = r0; r < r1; ++r) {
      const int v = roff[r];
      roff[r] = base;
      base += v;
    }
    if (tid == 0) roff[splits] = n_cand;
  }
  __syncthreads();
  if (M == neg_inf<ZT>()) {
    for (int d = tid; d < D; d += kNT) out[(size_t)bh * D + d] = 0.0f;
    if (tid == 0) {
      if (tau_out) tau_out[bh] = __builtin_nanf("");
      if (sup_out) sup_out[bh] = 0;
    }
    return;
  }
  const double amax = am1 * (double)M;
  ZT thr = M - window;
  // the score step's shared lower bound on tau of this head (wide windows)
  if (glb_key != 0x007fffffu && (ZT)order_float(glb_key) > thr) thr = (ZT)order_float(glb_key);
  if (n_cand > kTauBoundFrom) {
    // Many candidates: tighten the window with a lower bound on tau.
    const ZT lb = tau_window_bound(mloc, rmax, &tsh.tau_b, am1, m, mcode, amax);
    if (lb > thr) thr = lb;
  }

  // Gather and window filter, in batches of up to kNT * KB entries: thread t
  // takes a contiguous run of the batch (all of its loads in flight
  // together), keeps those with z >= thr, and one block scan places them in
  // order; members beyond the LDS capacity go to the head's global list. The
  // run length is a compile-time 2, 8, 16 or KB, picked from the batch size.
  ZT* gz = list_z + (size_t)bh * list_cap;
  int* gi = list_i + (size_t)bh * list_cap;
  int n_list = 0;
  for (int bbase = 0; bbase < n_cand; bbase += kNT * KB) {
    const int nb_ = min(kNT * KB, n_cand - bbase);
    const int per = (nb_ + kNT - 1) / kNT;
    const GatherArgs<ZT> ga{roff, creg, splits, cap, thr, lz, li, gz, gi, lcap, tmp};
    if (per <= 2) n_list = gather_batch<2>(ga, bbase, nb_, n_list);
    else if (per <= 8) n_list = gather_batch<8>(ga, bbase, nb_, n_list);
    else if (per <= 16)
      n_list = gather_batch_wide<16>(roff, creg, splits, cap, thr, lz, li, gz, gi, lcap, tmp,
                                     bbase, nb_, n_list);
    else
      n_list = gather_batch_wide<KB>(roff, creg, splits, cap, thr, lz, li, gz, gi, lcap, tmp,
                                          bbase, nb_, n_list);
  }
  __syncthreads();
  // (every bound that raised thr is at most tau, so Newton may start there)
  tau_solve_pv<KV, D, kNT>(v_pool, Hkv, g, PS, lz, li, sp, &pvacc[0][0], n_list, lcap, gz, gi,
                           am1, m, mcode, amax, tsh, out + (size_t)bh * D,
                           tau_out ? tau_out + bh : nullptr, sup_out ? sup_out + bh : nullptr,
                           am1 * (double)thr);
}

// One kernel serves the budgeted and the full-cache decode (the step is the
// same over either path's candidates), so a decode step that runs both finds
// its code in the instruction cache the second time.
template <typename KV, int D>
__global__ void __launch_bounds__(kNT)
tau_pv_kernel(TauArgs<KV> args) {
  extern __shared__ __align__(16) unsigned char smem[];
  tau_head<KV, D>(args, blockIdx.x % args.U, blockIdx.x / args.U, smem);
}

// ---------------------------------------------------------------------------
// host launchers (instantiated per cache dtype in decode_*.hip)

template <typename KV>
ScoreArgs<KV> score_args(const LaunchShape& s, const SplitPlan& p, const float* q,
                         const void* k_pool, const int32_t* bt, const int32_t* lens,
                         const int32_t* sel, int budget, float alpha, float window, void* ws,
                         const DecodeWs& L) {
  using ZT = typename KvTraits<KV>::Acc;
  char* w = static_cast<char*>(ws);
  ScoreArgs<KV> a;
  a.q = q;
  a.k_pool = static_cast<const KV*>(k_pool);
  a.block_table = bt;
  a.seq_lens = lens;
  a.sel = sel;
  a.H = s.num_q_heads;
  a.Hkv = s.num_kv_heads;
  a.U = s.batch * s.num_kv_heads;
  a.max_pages = s.max_pages;
  a.num_phys = s.num_phys;
  a.budget = budget;
  a.pps = p.pages_per_split;
  a.splits = p.splits;
  a.cap = p.cap;
  a.window_d = (double)window;
  a.cand = reinterpret_cast<Cand<ZT>*>(w + L.cand);
  a.counts = reinterpret_cast<int*>(w + L.counts);
  a.maxima = reinterpret_cast<ZT*>(w + L.maxima);
  a.spill = reinterpret_cast<Cand<ZT>*>(w + L.spill);
  const ScoreMode mode = score_mode(s, p, sel != nullptr, budget, window);
  a.gmax = mode.share ? reinterpret_cast<uint32_t*>(w + L.gmax) : nullptr;
  a.slots = mode.slots;
  a.local_bound = s.bf16 && kMfmaScores && window >= kWideWindow;
  a.alpha = alpha;
  return a;
}

template <typename KV, int D, int G, int PS, bool SPARSE>
hipError_t launch_score_t(const LaunchShape& s, const SplitPlan& p, const float* q,
                          const void* k_pool, const int32_t* bt, const int32_t* lens,
                          const int32_t* sel, int budget, float alpha, float window, void* ws,
                          const DecodeWs& L, hipStream_t st) {
  using ZT = typename KvTraits<KV>::Acc;
  const int U = s.batch * s.num_kv_heads;
  const ScoreLds lay = score_lds_layout(G, PS, p.pages_per_split, SPARSE, s.max_pages, budget,
                                        sizeof(ZT), score_kbuf_bytes(s.bf16, G, PS, D, SPARSE), D,
                                        score_mode(s, p, SPARSE, budget, window).slots);
  auto kern = score_kernel<KV, D, G, PS, SPARSE>;
  // The LDS limit is a kernel attribute: raised once, to the most any plan
  // asks for (a function-local static is initialised exactly once, also when
  // several host threads launch).
  static const hipError_t lds_raised =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxScoreLdsBytes);
  if (lds_raised != hipSuccess) return lds_raised;
  char* w = static_cast<char*>(ws);
  const ScoreArgs<KV> args =
      score_args<KV>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L);
  hipLaunchKernelGGL(kern, dim3(U * p.splits), dim3(kNT), lay.total, st, args);
  return hipGetLastError();
}

template <typename KV, int D, int G, bool SPARSE>
hipError_t launch_score_ps(const LaunchShape& s, const SplitPlan& p, const float* q,
                           const void* k_pool, const int32_t* bt, const int32_t* lens,
                           const int32_t* sel, int budget, float alpha, float window, void* ws,
                           const DecodeWs& L, hipStream_t st) {
  switch (s.page_size) {
    case 16: return launch_score_t<KV, D, G, 16, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
    case 32: return launch_score_t<KV, D, G, 32, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
    default: return launch_score_t<KV, D, G, 64, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
  }
}

template <typename KV, int D, bool SPARSE>
hipError_t launch_score_g(const LaunchShape& s, const SplitPlan& p, const float* q,
                          const void* k_pool, const int32_t* bt, const int32_t* lens,
                          const int32_t* sel, int budget, float alpha, float window, void* ws,
                          const DecodeWs& L, hipStream_t st) {
  switch (s.group) {
    case 1: return launch_score_ps<KV, D, 1, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
    case 2: return launch_score_ps<KV, D, 2, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
    case 4: return launch_score_ps<KV, D, 4, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
    default: return launch_score_ps<KV, D, 8, SPARSE>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
  }
}

template <typename KV>
hipError_t launch_score_kv(const LaunchShape& s, const SplitPlan& p, const float* q,
                           const void* k_pool, const int32_t* bt, const int32_t* lens,
                           const int32_t* sel, int budget, float alpha, float window, void* ws,
                           const DecodeWs& L, hipStream_t st) {
  if (sel) {
    if (s.head_dim == 64) return launch_score_g<KV, 64, true>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
    return launch_score_g<KV, 128, true>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
  }
  if (s.head_dim == 64) return launch_score_g<KV, 64, false>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
  return launch_score_g<KV, 128, false>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
}

template <typename KV>
TauArgs<KV> tau_args(const LaunchShape& s, const SplitPlan& p, const void* v_pool, float alpha,
                     float window, float* out, float* tau, int32_t* support, void* ws,
                     const DecodeWs& L, int lcap, bool share) {
  using ZT = typename KvTraits<KV>::Acc;
  char* w = static_cast<char*>(ws);
  TauArgs<KV> a;
  a.v_pool = static_cast<const KV*>(v_pool);
  a.H = s.num_q_heads;
  a.Hkv = s.num_kv_heads;
  a.G = s.group;
  a.U = s.batch * s.num_kv_heads;
  a.PS = s.page_size;
  a.splits = p.regions;
  a.cap = p.rcap;
  a.list_cap = p.list_cap;
  a.lcap = lcap;
  a.alpha = alpha;
  a.window_d = (double)window;
  a.cand = reinterpret_cast<const Cand<ZT>*>(w + L.cand);
  a.counts = reinterpret_cast<const int*>(w + L.counts);
  a.maxima = reinterpret_cast<const ZT*>(w + L.maxima);
  a.list_z = reinterpret_cast<ZT*>(w + L.list);
  a.list_i = reinterpret_cast<int*>(a.list_z + (size_t)s.batch * s.num_q_heads * p.list_cap);
  a.out = out;
  a.tau_out = tau;
  a.sup_out = support;
  a.glb = share ? reinterpret_cast<const uint32_t*>(w + L.gmax) : nullptr;
  return a;
}

template <typename KV, int D, bool SPARSE>
hipError_t launch_tau_pv_t(const LaunchShape& s, const SplitPlan& p, const void* v_pool,
                           const int32_t* bt, const int32_t* lens, const int32_t* sel, int budget,
                           float alpha, float window, float* out, float* tau, int32_t* support,
                           void* ws, const DecodeWs& L, hipStream_t st) {
  (void)bt; (void)lens; (void)sel;
  using ZT = typename KvTraits<KV>::Acc;
  constexpr int NG = kNT / (D / (16 / (int)sizeof(KV)));
  const int U = s.batch * s.num_kv_heads;
  // Up to 256 workgroups (one per CU) hold 8192 window members each; larger
  // grids hold 4096 so that two workgroups fit a CU.
  const int lcap = U * s.group > 256 ? kTauMaxList / 2 : kTauMaxList;
  const size_t lds = tau_lds_layout(p.regions, lcap, sizeof(ZT), NG, D).total;
  auto kern = tau_pv_kernel<KV, D>;
  // The LDS limit is a kernel attribute: raised once per launcher, to the
  // most any plan asks for (a function-local static is initialised exactly
  // once, also when several host threads launch; the other path's launcher
  // setting it again is harmless).
  static const hipError_t lds_raised = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)tau_lds_layout(kMaxSplits, kTauMaxList, 8, NG, D).total);
  if (lds_raised != hipSuccess) return lds_raised;
  const TauArgs<KV> args = tau_args<KV>(s, p, v_pool, alpha, window, out, tau, support, ws, L,
                                        lcap, score_mode(s, p, SPARSE, budget, window).share);
  hipLaunchKernelGGL(kern, dim3(U * s.group), dim3(kNT), lds, st, args);
  return hipGetLastError();
}

template <typename KV>
hipError_t launch_tau_pv_kv(const LaunchShape& s, const SplitPlan& p, const void* v_pool,
                            const int32_t* bt, const int32_t* lens, const int32_t* sel,
                            int budget, float alpha, float window, float* out, float* tau,
                            int32_t* support, void* ws, const DecodeWs& L, hipStream_t st) {
  if (sel) {
    if (s.head_dim == 64) return launch_tau_pv_t<KV, 64, true>(s, p, v_pool, bt, lens, sel, budget, alpha, window, out, tau, support, ws, L, st);
    return launch_tau_pv_t<KV, 128, true>(s, p, v_pool, bt, lens, sel, budget, alpha, window, out, tau, support, ws, L, st);
  }
  if (s.head_dim == 64) return launch_tau_pv_t<KV, 64, false>(s, p, v_pool, bt, lens, sel, budget, alpha, window, out, tau, support, ws, L, st);
  return launch_tau_pv_t<KV, 128, false>(s, p, v_pool, bt, lens, sel, budget, alpha, window, out, tau, support, ws, L, st);
}

}  // namespace ekv
