// Gaussian-aware entmax page selection ([EntmaxKV page] section 2.A, the
// Gaussian statistics, and section 2.B, policy 2). The pages give the policy
// but not its formulas; the readings implemented here:
//  - a page's token scores under q are taken as N(mu, s^2) with
//    mu = sum_d q_d mean_d and s^2 = sum_d q_d^2 var_d (the page's key
//    moments, coordinates independent); in the units of tau,
//    a ~ N(mu_a, s_a^2) with mu_a = (alpha-1) mu and s_a = (alpha-1) s;
//  - tau_hat solves sum_p n_p E[(A_p - t)_+^m] = 1 (n_p the page's valid
//    tokens, m = 1/(alpha-1) an integer 1..4), E in closed form from the
//    truncated moments of the standard normal;
//  - a page's estimated maximum is mu_a + s_a sqrt(2 ln n_p), and the page
//    is a candidate when that exceeds tau_hat - Delta.
//
// gauss_stats_kernel: one workgroup per (chunk of 32 pages, (b, KV head));
//   a page's moment record [mean | var] is split over D/4 lanes, the G
//   heads' two dot products are formed in float64 and finished by a
//   multi-value butterfly; (mu_a, s_a) per (b, h, page) go to the workspace.
// gauss_solve_kernel: one workgroup per (b, h): tau_hat by Newton's method
//   from the left end of the bracket (the left side of the equation is convex
//   and decreasing in t, so the iterates rise monotonically to the root),
//   over the pages that can contribute (held in LDS); then one key per page
//   (its estimated maximum as float32, or -inf when it fails the rule) for
//   the top-cap select kernel.
#include <cfloat>
#include <type_traits>

#include "launch.hpp"

namespace ekv {

constexpr int kGaussPages = 32;    // pages per workgroup of the statistics kernel
constexpr int kGaussList = 2048;   // contributing pages a solve workgroup holds in LDS
constexpr int kGaussIters = 64;    // most Newton steps
constexpr double kGaussReach = 9.0;  // pages with mu_a + 9 s_a <= the bracket's left end
                                     // contribute below 1e-19 n_p s_a^m: left out of the sums

template <typename KV, int D, int G>
__global__ void __launch_bounds__(256)
gauss_stats_kernel(const float* __restrict__ q, const KV* __restrict__ moments,
                   const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                   double2* __restrict__ stats, int H, int Hkv, int ps, int max_pages,
                   int num_phys, int U, int ldu, double am1) {
  constexpr int VPC = 4;       // coordinates per lane (per record half)
  constexpr int LP = D / VPC;  // lanes per page
  constexpr int PPB = 256 / LP;
  constexpr int STEPS = kGaussPages / PPB;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  using Chunk = typename std::conditional<sizeof(KV) == 2, u32x2, u32x4>::type;
  using BF = Butterfly<G, LP>;
  static_assert(BF::CNT == 1, "group size must not exceed lanes per page");
  static_assert(kGaussPages % PPB == 0, "whole block steps");
  __shared__ int sphys[kGaussPages];

  const int u = blockIdx.x % U;
  const int chunk = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int j0 = chunk * kGaussPages;
  const int jt = j0 + (int)threadIdx.x;
  const int bt_entry = threadIdx.x < kGaussPages && jt < max_pages
                           ? block_table[(size_t)b * max_pages + jt] : -1;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  if (j0 >= P) return;
  const int n = min(kGaussPages, P - j0);
  if (threadIdx.x < kGaussPages) sphys[threadIdx.x] = (int)threadIdx.x < n ? bt_entry : -1;

  const int lane = threadIdx.x & (kWave - 1);
  const int c = threadIdx.x % LP;
  const int h0 = b * H + g * G;
  float qf[G][VPC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4 v = *reinterpret_cast<const float4*>(q + (size_t)(h0 + h) * D + c * VPC);
    qf[h][0] = v.x; qf[h][1] = v.y; qf[h][2] = v.z; qf[h][3] = v.w;
  }
  const int my_head = BF::first_index(lane);
  const bool owner = BF::owner(lane);
  __syncthreads();

  // every record load of the workgroup in flight before the first is used
  Chunk xm[STEPS], xv[STEPS];
  bool ok[STEPS];
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    const int phys = sphys[t * PPB + threadIdx.x / LP];
    ok[t] = phys >= 0 && phys < num_phys;
    // page 0 stands in for an empty slot; its result is dropped
    const KV* row = moments + ((size_t)(ok[t] ? phys : 0) * Hkv + g) * 2 * D + c * VPC;
    xm[t] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(row));
    xv[t] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(row + D));
  }
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    float mean[VPC], var[VPC];
    if constexpr (sizeof(KV) == 2) {
      mean[0] = bf16_lo(xm[t].x); mean[1] = bf16_hi(xm[t].x);
      mean[2] = bf16_lo(xm[t].y); mean[3] = bf16_hi(xm[t].y);
      var[0] = bf16_lo(xv[t].x); var[1] = bf16_hi(xv[t].x);
      var[2] = bf16_lo(xv[t].y); var[3] = bf16_hi(xv[t].y);
    } else {
      mean[0] = __uint_as_float(xm[t].x); mean[1] = __uint_as_float(xm[t].y);
      mean[2] = __uint_as_float(xm[t].z); mean[3] = __uint_as_float(xm[t].w);
      var[0] = __uint_as_float(xv[t].x); var[1] = __uint_as_float(xv[t].y);
      var[2] = __uint_as_float(xv[t].z); var[3] = __uint_as_float(xv[t].w);
    }
    double mu[G], s2[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double a = 0.0, v = 0.0;
#pragma unroll
      for (int e = 0; e < VPC; ++e) {
        const double qd = (double)qf[h][e];
        a = fma(qd, (double)mean[e], a);
        v = fma(qd * qd, (double)var[e], v);
      }
      mu[h] = a;
      s2[h] = v;
    }
    BF::reduce(mu, lane);
    BF::reduce(s2, lane);
    const int jj = t * PPB + threadIdx.x / LP;
    if (ok[t] && owner)
      stats[(size_t)(h0 + my_head) * ldu + j0 + jj] =
          make_double2(am1 * mu[0], am1 * sqrt(fmax(s2[0], 0.0)));
  }
}

// E[(Y - c)_+^k] for Y ~ N(0, 1), k = M and M - 1 (M in 1..4), from the
// truncated moments J_k = E[Y^k; Y > c]: J_0 = Q(c), J_1 = phi(c),
// J_k = c^(k-1) phi(c) + (k-1) J_(k-2), and the binomial expansion of
// (Y - c)^k. Clamped at 0 (the expansion cancels to rounding noise where
// phi underflows).
template <int M>
__device__ __forceinline__ void normal_partial_moments(double c, double& pm, double& pm1) {
  const double phi = 0.3989422804014327 * exp(-0.5 * c * c);  // 1/sqrt(2 pi)
  double J[M + 1];
  J[0] = 0.5 * erfc(c * 0.7071067811865476);  // Q(c) = erfc(c / sqrt 2) / 2
  if constexpr (M >= 1) J[1] = phi;
#pragma unroll
  for (int k = 2; k <= M; ++k) {
    double ck = 1.0;
#pragma unroll
    for (int i = 0; i < k - 1; ++i) ck *= c;
    J[k] = ck * phi + (double)(k - 1) * J[k - 2];
  }
  auto expand = [&](int m) {
    // sum_k binom(m, k) (-c)^(m-k) J_k
    double s = 0.0, binom = 1.0;
    for (int k = m; k >= 0; --k) {
      double p = 1.0;
      for (int i = 0; i < m - k; ++i) p *= -c;
      s += binom * p * J[k];
      binom = binom * (double)k / (double)(m - k + 1);
    }
    return fmax(s, 0.0);
  };
  pm = expand(M);
  pm1 = expand(M - 1);
}

template <int M>
__global__ void __launch_bounds__(256)
gauss_solve_kernel(const double2* __restrict__ stats, const int32_t* __restrict__ seq_lens,
                   int H, int ps, int max_pages, int ldu, double delta, float* __restrict__ keys,
                   float* __restrict__ tau_hat) {
  constexpr int NT = 256;
  __shared__ double lmu[kGaussList];
  __shared__ double ls[kGaussList];
  __shared__ float ln[kGaussList];
  __shared__ double red[2 * (NT / kWave)];
  __shared__ int tmp[NT / kWave + 2];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int bh = blockIdx.x, b = bh / H;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  const double2* row = stats + (size_t)bh * ldu;
  float* krow = keys + (size_t)bh * ldu;
  if (P == 0) {
    if (tid == 0 && tau_hat) tau_hat[bh] = __builtin_nanf("");
    return;
  }
  auto rows_of = [&](int j) { return (double)min(ps, L - j * ps); };

  // bracket: the root lies in [max mu_a - 1, max (mu_a + 40 s_a)]
  double mx = -DBL_MAX;
  for (int j = tid; j < P; j += NT) mx = fmax(mx, row[j].x);
  mx = block_reduce<NT>(mx, red, [](double a, double c) { return fmax(a, c); });
  const double lo = mx - 1.0;

  // the pages that can contribute at t >= lo, compacted into LDS when they fit
  auto reaches = [&](const double2& v) {
    return v.y > 0.0 ? v.x + kGaussReach * v.y > lo : v.x > lo;
  };
  int cnt = 0;
  for (int j = tid; j < P; j += NT) cnt += reaches(row[j]) ? 1 : 0;
  int n_act;
  int pos = block_excl_scan<NT>(cnt, tmp, &n_act);
  const bool in_lds = n_act <= kGaussList;
  if (in_lds) {
    for (int j = tid; j < P; j += NT) {
      const double2 v = row[j];
      if (reaches(v)) {
        lmu[pos] = v.x;
        ls[pos] = v.y;
        ln[pos] = (float)rows_of(j);
        ++pos;
      }
    }
  }
  __syncthreads();

  // f(t) = sum_p n_p E[(A_p - t)_+^M] and g(t) = -f'(t) / M
  auto term = [&](double mu, double s, double n, double t, double& f, double& g) {
    if (s > 0.0) {
      double pm, pm1;
      normal_partial_moments<M>((t - mu) / s, pm, pm1);
      double sm1 = 1.0;
#pragma unroll
      for (int i = 0; i < M - 1; ++i) sm1 *= s;
      f += n * sm1 * s * pm;
      g += n * sm1 * pm1;
    } else if (mu > t) {
      const double d = mu - t;
      double dm1 = 1.0;
#pragma unroll
      for (int i = 0; i < M - 1; ++i) dm1 *= d;
      f += n * dm1 * d;
      g += n * dm1;
    }
  };
  double t = lo;
  for (int it = 0; it < kGaussIters; ++it) {
    double f = 0.0, g = 0.0;
    if (in_lds) {
      for (int i = tid; i < n_act; i += NT) term(lmu[i], ls[i], (double)ln[i], t, f, g);
    } else {
      for (int j = tid; j < P; j += NT) {
        const double2 v = row[j];
        if (reaches(v)) term(v.x, v.y, rows_of(j), t, f, g);
      }
    }
    f = wave_allsum(f);
    g = wave_allsum(g);
    if (lane == 0) {
      red[2 * wid] = f;
      red[2 * wid + 1] = g;
    }
    __syncthreads();
    f = 0.0;
    g = 0.0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
      f += red[2 * w];
      g += red[2 * w + 1];
    }
    __syncthreads();
    // Newton step from the left (f - 1 >= 0 here, f' = -M g < 0)
    if (!(f > 1.0) || !(g > 0.0)) break;
    const double step = (f - 1.0) / ((double)M * g);
    t += step;
    if (step <= 1e-15 * fmax(1.0, fabs(t))) break;
  }

  // one key per page: the estimated maximum, or -inf off the rule
  const double cut = t - delta;
  for (int j = tid; j < P; j += NT) {
    const double2 v = row[j];
    const double n = rows_of(j);
    const double est = n >= 2.0 ? v.x + v.y * sqrt(2.0 * log(n)) : v.x;
    krow[j] = est > cut ? (float)est + 0.0f : -__builtin_inff();
  }
  if (tid == 0 && tau_hat) tau_hat[bh] = (float)t;
}

template <typename KV, int D, int G>
static hipError_t launch_stats_g(const LaunchShape& s, const float* q, const void* moments,
                                 const int32_t* bt, const int32_t* lens, double am1, void* stats,
                                 hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  const int chunks = (s.max_pages + kGaussPages - 1) / kGaussPages;
  hipLaunchKernelGGL((gauss_stats_kernel<KV, D, G>), dim3(U * chunks), dim3(256), 0, st, q,
                     static_cast<const KV*>(moments), bt, lens, static_cast<double2*>(stats),
                     s.num_q_heads, s.num_kv_heads, s.page_size, s.max_pages, s.num_phys, U,
                     ub_ld(s.max_pages), am1);
  return hipGetLastError();
}

template <typename KV, int D>
static hipError_t launch_stats_d(const LaunchShape& s, const float* q, const void* moments,
                                 const int32_t* bt, const int32_t* lens, double am1, void* stats,
                                 hipStream_t st) {
  switch (s.group) {
    case 1: return launch_stats_g<KV, D, 1>(s, q, moments, bt, lens, am1, stats, st);
    case 2: return launch_stats_g<KV, D, 2>(s, q, moments, bt, lens, am1, stats, st);
    case 4: return launch_stats_g<KV, D, 4>(s, q, moments, bt, lens, am1, stats, st);
    default: return launch_stats_g<KV, D, 8>(s, q, moments, bt, lens, am1, stats, st);
  }
}

hipError_t launch_gauss_stats(const LaunchShape& s, const float* q, const void* moments,
                              const int32_t* bt, const int32_t* lens, double am1, void* stats,
                              hipStream_t st) {
  if (s.bf16) {
    if (s.head_dim == 64) return launch_stats_d<bf16_t, 64>(s, q, moments, bt, lens, am1, stats, st);
    return launch_stats_d<bf16_t, 128>(s, q, moments, bt, lens, am1, stats, st);
  }
  if (s.head_dim == 64) return launch_stats_d<float, 64>(s, q, moments, bt, lens, am1, stats, st);
  return launch_stats_d<float, 128>(s, q, moments, bt, lens, am1, stats, st);
}

hipError_t launch_gauss_solve(const LaunchShape& s, const void* stats, const int32_t* lens, int m,
                              double delta, float* keys, float* tau_hat, hipStream_t st) {
  const int heads = s.batch * s.num_q_heads;
  const double2* st2 = static_cast<const double2*>(stats);
  const int ldu = ub_ld(s.max_pages);
  switch (m) {
    case 1:
      hipLaunchKernelGGL(gauss_solve_kernel<1>, dim3(heads), dim3(256), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
    case 2:
      hipLaunchKernelGGL(gauss_solve_kernel<2>, dim3(heads), dim3(256), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
    case 3:
      hipLaunchKernelGGL(gauss_solve_kernel<3>, dim3(heads), dim3(256), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
    default:
      hipLaunchKernelGGL(gauss_solve_kernel<4>, dim3(heads), dim3(256), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
  }
  return hipGetLastError();
}

// stats (double2) then keys (float), each [batch * num_q_heads, ub_ld] and
// 256-byte aligned
size_t gauss_ws_bytes(const LaunchShape& s) {
  const size_t rows = (size_t)s.batch * s.num_q_heads * ub_ld(s.max_pages);
  const size_t a = (rows * 16 + 255) & ~(size_t)255;
  return a + rows * 4;
}

}  // namespace ekv
