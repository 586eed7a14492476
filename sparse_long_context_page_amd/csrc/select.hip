// Page bounds and fixed-budget top-k page selection.
// EntmaxKV summary page (gist.science paper 2605.21649): section 2.A (the
// box metadata gives a deterministic upper bound on a page's best q.k) and
// section 2.B policy 1 (keep the k pages with the highest bounds).
//
// bounds_kernel: one workgroup per (chunk of pages, sequence, KV head). The
//   G query heads that share the KV head are bounded together, so each page's
//   box is read once. Each page's (k_min, k_max) row pair is split over LP
//   lanes (16 bytes of each per lane). Per coordinate the lane takes k_max
//   where q_d >= 0 and k_min otherwise (the box maximum of q_d k_d), forms the
//   products in float64 (exact: 24-bit x 8- or 24-bit significands) and sums
//   in float64; a multi-value butterfly finishes the G sums across the LP
//   lanes. Result rounded once to float32 (+0 for a zero).
// select_kernel: one workgroup per (sequence, query head). Radix select on
//   the order-preserving 32-bit image of the float32 bound, starting at the
//   highest bit where the bounds differ (so the first histogram is spread),
//   8 bits per pass, stopping as soon as the boundary digit is taken whole.
//   Ties on the full 32 bits go to the lower page index. The kept pages are
//   written in ascending order with two block scans.
#include "launch.hpp"

namespace ekv {

constexpr int kSelNT = 256;
constexpr int kSelLds = 16384;  // bounds staged in LDS when the sequence has at most this many pages
constexpr int kBoundSteps = 4;  // page groups per workgroup

template <typename KV, int D, int G>
__global__ void __launch_bounds__(256)
bounds_kernel(const float* __restrict__ q, const KV* __restrict__ meta,
              const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
              float* __restrict__ ub, int H, int Hkv, int ps, int max_pages, int num_phys, int U) {
  constexpr int VPC = 16 / sizeof(KV);    // box coordinates per lane (per bound side)
  constexpr int LP = D / VPC;             // lanes per page
  constexpr int PPB = 256 / LP;           // pages per block step
  using BF = Butterfly<G, LP>;
  static_assert(BF::CNT == 1, "group size must not exceed lanes per page");

  const int u = blockIdx.x % U;
  const int chunk = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  const int j0 = chunk * PPB * kBoundSteps;
  if (j0 >= P) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int c = threadIdx.x % LP;
  const int h0 = b * H + g * G;

  double qd[G][VPC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VPC; ++e) qd[h][e] = (double)q[(size_t)(h0 + h) * D + c * VPC + e];

  const int my_head = BF::first_index(lane);
  const bool owner = BF::owner(lane);

#pragma unroll
  for (int s = 0; s < kBoundSteps; ++s) {
    const int j = j0 + s * PPB + threadIdx.x / LP;
    int phys = -1;
    if (j < P) phys = block_table[(size_t)b * max_pages + j];
    const bool ok = phys >= 0 && phys < num_phys;
    uint4 xlo = make_uint4(0, 0, 0, 0), xhi = make_uint4(0, 0, 0, 0);
    if (ok) {
      const KV* row = meta + ((size_t)phys * Hkv + g) * 2 * D + c * VPC;
      xlo = *reinterpret_cast<const uint4*>(row);
      xhi = *reinterpret_cast<const uint4*>(row + D);
    }
    float lo[VPC], hi[VPC];
    if constexpr (sizeof(KV) == 2) {
      const uint32_t wl[4] = {xlo.x, xlo.y, xlo.z, xlo.w};
      const uint32_t wh[4] = {xhi.x, xhi.y, xhi.z, xhi.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[2 * i] = bf16_lo(wl[i]);
        lo[2 * i + 1] = bf16_hi(wl[i]);
        hi[2 * i] = bf16_lo(wh[i]);
        hi[2 * i + 1] = bf16_hi(wh[i]);
      }
    } else {
      lo[0] = __uint_as_float(xlo.x); lo[1] = __uint_as_float(xlo.y);
      lo[2] = __uint_as_float(xlo.z); lo[3] = __uint_as_float(xlo.w);
      hi[0] = __uint_as_float(xhi.x); hi[1] = __uint_as_float(xhi.y);
      hi[2] = __uint_as_float(xhi.z); hi[3] = __uint_as_float(xhi.w);
    }
    double acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < VPC; ++e) {
        const float k = qd[h][e] >= 0.0 ? hi[e] : lo[e];
        a = fma(qd[h][e], (double)k, a);
      }
      acc[h] = a;
    }
    BF::reduce(acc, lane);
    if (ok && owner) {
      const float key = (float)acc[0] + 0.0f;
      ub[(size_t)(h0 + my_head) * max_pages + j] = key;
    }
  }
}

// --------------------------------------------------------------------------

__global__ void __launch_bounds__(kSelNT)
select_kernel(const float* __restrict__ ub, const int32_t* __restrict__ seq_lens, int H, int G,
              int Hkv, int U, int ps, int max_pages, int budget, int32_t* __restrict__ sel,
              float* __restrict__ sel_ub) {
  constexpr int NW = kSelNT / kWave;
  __shared__ uint32_t sord[kSelLds];
  __shared__ int hist[256];
  __shared__ unsigned int ured[NW];
  __shared__ int wcnt[NW][2];
  __shared__ int bc[2];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int u = blockIdx.x % U, hh = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int bh = b * H + g * G + hh;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  const float* row = ub + (size_t)bh * max_pages;
  int32_t* out = sel + (size_t)bh * budget;
  float* out_ub = sel_ub ? sel_ub + (size_t)bh * budget : nullptr;

  if (P <= budget) {
    for (int i = tid; i < budget; i += kSelNT) {
      out[i] = i < P ? i : -1;
      if (out_ub) out_ub[i] = i < P ? row[i] : -__builtin_inff();
    }
    return;
  }

  // Order-preserving 32-bit keys; staged in LDS when they fit.
  const bool staged = P <= kSelLds;
  if (staged) {
    for (int i = tid; i < P; i += kSelNT) sord[i] = float_order(row[i] + 0.0f);
    __syncthreads();
  }
  auto ord = [&](int i) -> uint32_t { return staged ? sord[i] : float_order(row[i] + 0.0f); };

  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int i = tid; i < P; i += kSelNT) {
    const uint32_t o = ord(i);
    mn = min(mn, o);
    mx = max(mx, o);
  }
  mn = block_reduce<kSelNT>(mn, ured, [](uint32_t a, uint32_t c) { return min(a, c); });
  mx = block_reduce<kSelNT>(mx, ured, [](uint32_t a, uint32_t c) { return max(a, c); });

  // Radix select of the budget-th largest key, 8 bits per pass from the
  // highest bit where keys differ; stop once the boundary digit is taken whole.
  uint32_t prefix, pmask;
  int k = budget;  // rank still to place among keys matching the prefix
  if (mn == mx) {
    prefix = mx;
    pmask = 0xffffffffu;
  } else {
    int hb = 31 - __clz(mn ^ mx);
    pmask = ~((2u << hb) - 1u);
    prefix = mx & pmask;
    while (true) {
      const int lo = hb >= 7 ? hb - 7 : 0;
      const int width = hb - lo + 1;
      const uint32_t dmask = (1u << width) - 1u;
      hist[tid] = 0;  // kSelNT == 256 bins
      __syncthreads();
      for (int i = tid; i < P; i += kSelNT) {
        const uint32_t o = ord(i);
        if ((o & pmask) == prefix) atomicAdd(&hist[(o >> lo) & dmask], 1);
      }
      __syncthreads();
      if (wave == 0) {
        int c4[4];
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c4[i] = hist[4 * lane + i];
          s += c4[i];
        }
        int suf = s;  // keys in this lane's bins and above
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
          const int o = __shfl_down(suf, d, kWave);
          if (lane + d < kWave) suf += o;
        }
        int above = suf - s;
        if (above < k && k <= suf) {
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if (above < k && k <= above + c4[i]) {
              bc[0] = 4 * lane + i;
              bc[1] = above;
            }
            above += c4[i];
          }
        }
      }
      __syncthreads();
      const int d = bc[0];
      const int cnt_d = hist[d];
      k -= bc[1];
      prefix |= ((uint32_t)d) << lo;
      pmask |= dmask << lo;
      if (cnt_d == k || lo == 0) break;
      hb = lo - 1;
      __syncthreads();
    }
  }

  // Keep keys above the prefix and the first k (by page index) equal to it,
  // written in ascending page order. Wave w owns a contiguous page range and
  // walks it 64 pages at a time (consecutive LDS words, no bank conflicts).
  const int span = ((P + NW * kWave - 1) / (NW * kWave)) * kWave;
  const int j0 = min(P, wave * span), j1 = min(P, j0 + span);
  const uint64_t ltm = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int n_eq = 0, n_gt = 0;
  for (int base = j0; base < j1; base += kWave) {
    const int j = base + lane;
    uint32_t m = 0;
    if (j < j1) m = ord(j) & pmask;
    n_eq += __popcll(__ballot(j < j1 && m == prefix));
    n_gt += __popcll(__ballot(j < j1 && m > prefix));
  }
  if (lane == 0) {
    wcnt[wave][0] = n_eq;
    wcnt[wave][1] = n_gt;
  }
  __syncthreads();
  int eq_base = 0, sel_base = 0;
  for (int w = 0; w < wave; ++w) {
    const int e = wcnt[w][0];
    sel_base += wcnt[w][1] + max(0, min(e, k - eq_base));
    eq_base += e;
  }
  for (int base = j0; base < j1; base += kWave) {
    const int j = base + lane;
    uint32_t m = 0;
    if (j < j1) m = ord(j) & pmask;
    const bool eq = j < j1 && m == prefix;
    const bool gt = j < j1 && m > prefix;
    const uint64_t beq = __ballot(eq);
    const int rank = eq_base + __popcll(beq & ltm);
    const bool take = gt || (eq && rank < k);
    const uint64_t bt = __ballot(take);
    if (take) {
      const int pos = sel_base + __popcll(bt & ltm);
      out[pos] = j;
      if (out_ub) out_ub[pos] = row[j] + 0.0f;
    }
    eq_base += __popcll(beq);
    sel_base += __popcll(bt);
  }
}

template <typename KV, int D, int G>
static hipError_t launch_bounds_t(const LaunchShape& s, const float* q, const void* meta,
                                  const int32_t* bt, const int32_t* lens, float* ub,
                                  hipStream_t st) {
  constexpr int LP = D / (16 / sizeof(KV));
  constexpr int PPW = (256 / LP) * kBoundSteps;
  const int U = s.batch * s.num_kv_heads;
  const int chunks = (s.max_pages + PPW - 1) / PPW;
  hipLaunchKernelGGL((bounds_kernel<KV, D, G>), dim3(U * chunks), dim3(256), 0, st, q,
                     static_cast<const KV*>(meta), bt, lens, ub, s.num_q_heads, s.num_kv_heads,
                     s.page_size, s.max_pages, s.num_phys, U);
  return hipGetLastError();
}

template <typename KV, int D>
static hipError_t launch_bounds_d(const LaunchShape& s, const float* q, const void* meta,
                                  const int32_t* bt, const int32_t* lens, float* ub,
                                  hipStream_t st) {
  switch (s.group) {
    case 1: return launch_bounds_t<KV, D, 1>(s, q, meta, bt, lens, ub, st);
    case 2: return launch_bounds_t<KV, D, 2>(s, q, meta, bt, lens, ub, st);
    case 4: return launch_bounds_t<KV, D, 4>(s, q, meta, bt, lens, ub, st);
    default: return launch_bounds_t<KV, D, 8>(s, q, meta, bt, lens, ub, st);
  }
}

hipError_t launch_bounds(const LaunchShape& s, const float* q, const void* meta,
                         const int32_t* bt, const int32_t* lens, float* ub, hipStream_t st) {
  if (s.bf16) {
    if (s.head_dim == 64) return launch_bounds_d<bf16_t, 64>(s, q, meta, bt, lens, ub, st);
    return launch_bounds_d<bf16_t, 128>(s, q, meta, bt, lens, ub, st);
  }
  if (s.head_dim == 64) return launch_bounds_d<float, 64>(s, q, meta, bt, lens, ub, st);
  return launch_bounds_d<float, 128>(s, q, meta, bt, lens, ub, st);
}

hipError_t launch_select(const LaunchShape& s, const float* ub, const int32_t* lens, int budget,
                         int32_t* sel, float* sel_ub, hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  hipLaunchKernelGGL(select_kernel, dim3(U * s.group), dim3(kSelNT), 0, st, ub, lens,
                     s.num_q_heads, s.group, s.num_kv_heads, U, s.page_size, s.max_pages, budget,
                     sel, sel_ub);
  return hipGetLastError();
}

size_t select_ws_bytes(const LaunchShape& s) {
  return (size_t)s.batch * s.num_q_heads * s.max_pages * sizeof(float);
}

}  // namespace ekv
