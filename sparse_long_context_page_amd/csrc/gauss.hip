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
// gauss_solve_kernel: one workgroup of 1024 threads per (b, h), the head's
//   page statistics staged in LDS: tau_hat by Newton steps on the logarithm
//   of the equation's left side (nearly quadratic in t for Gaussian tails),
//   safeguarded by a bracket that bisects when a step would leave it; then
//   one key per page (its estimated maximum as float32, or -inf when it fails
//   the rule) for the top-cap select kernel.
#include <cfloat>
#include <type_traits>

#include "launch.hpp"

namespace ekv {

constexpr int kGaussPages = 32;    // pages per workgroup of the statistics kernel
constexpr int kGaussNT = 1024;     // threads of a solve workgroup (one per (b, h))
constexpr int kGaussLds = 4096;    // pages of a head a solve workgroup holds in LDS
constexpr int kGaussIters = 100;   // most solve steps
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
    // a page past the block table's valid range (an input outside the
    // contract) gets a neutral entry: it adds nothing to tau_hat's sum and
    // its key is -inf
    if (jj < n && owner)
      stats[(size_t)(h0 + my_head) * ldu + j0 + jj] =
          ok[t] ? make_double2(am1 * mu[0], am1 * sqrt(fmax(s2[0], 0.0)))
                : make_double2(-DBL_MAX, 0.0);
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

// The same in float32 (a cheaper first approximation of tau_hat; the
// expansion's cancellation in the far tail only touches pages whose share
// of the sum is negligible there).
template <int M>
__device__ __forceinline__ void normal_partial_moments_f(float c, float& pm, float& pm1) {
  const float phi = 0.39894228f * __expf(-0.5f * c * c);
  float J[M + 1];
  J[0] = 0.5f * erfcf(c * 0.70710678f);
  if constexpr (M >= 1) J[1] = phi;
#pragma unroll
  for (int k = 2; k <= M; ++k) {
    float ck = 1.0f;
#pragma unroll
    for (int i = 0; i < k - 1; ++i) ck *= c;
    J[k] = ck * phi + (float)(k - 1) * J[k - 2];
  }
  auto expand = [&](int m) {
    float s = 0.0f, binom = 1.0f;
    for (int k = m; k >= 0; --k) {
      float p = 1.0f;
      for (int i = 0; i < m - k; ++i) p *= -c;
      s += binom * p * J[k];
      binom = binom * (float)k / (float)(m - k + 1);
    }
    return fmaxf(s, 0.0f);
  };
  pm = expand(M);
  pm1 = expand(M - 1);
}

template <int M>
__global__ void __launch_bounds__(kGaussNT)
gauss_solve_kernel(const double2* __restrict__ stats, const int32_t* __restrict__ seq_lens,
                   int H, int ps, int max_pages, int ldu, double delta, float* __restrict__ keys,
                   float* __restrict__ tau_hat) {
  constexpr int NT = kGaussNT, NW = NT / kWave;
  __shared__ double red[2 * NW];
  __shared__ double smu[kGaussLds];
  __shared__ double ss[kGaussLds];

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
  // two sums (or maxima) over the workgroup, the same on every thread
  auto block2 = [&](double& x, double& y, bool is_max) {
    if (is_max) {
      x = wave_max(x);
      y = wave_max(y);
    } else {
      x = wave_allsum(x);
      y = wave_allsum(y);
    }
    if (lane == 0) {
      red[2 * wid] = x;
      red[2 * wid + 1] = y;
    }
    __syncthreads();
    x = red[0];
    y = red[1];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      x = is_max ? fmax(x, red[2 * w]) : x + red[2 * w];
      y = is_max ? fmax(y, red[2 * w + 1]) : y + red[2 * w + 1];
    }
    __syncthreads();
  };

  // (mu_a, s_a) of the head's pages: staged in LDS when the sequence has at
  // most kGaussLds pages, else read from the workspace row at every step
  const bool in_lds = P <= kGaussLds;
  double mx = -DBL_MAX, hx = -DBL_MAX;
  for (int j = tid; j < P; j += NT) {
    const double2 v = row[j];
    if (in_lds) {
      smu[j] = v.x;
      ss[j] = v.y;
    }
    mx = fmax(mx, v.x);
    hx = fmax(hx, v.x + 40.0 * v.y);
  }
  block2(mx, hx, true);
  // bracket: f(a) >= 1 at a = max mu - 1 (the top page alone gives
  // n (E[A] - a)^M >= 1 by Jensen), f < 1 at the right end
  double a = mx - 1.0, z = fmax(hx, a + 1.0);

  // Starting point: the root for one Gaussian pooled over the head's tokens
  // (mean and variance of the page mixture, taken about mx), i.e.
  // N sbar^M E[(Y - c)_+^M] = 1 solved for c by Newton steps on the log of
  // the left side (concave and decreasing in c), then t0 = mubar + c sbar.
  double s1 = 0.0, s2 = 0.0;
  for (int j = tid; j < P; j += NT) {
    const double mu = in_lds ? smu[j] : row[j].x;
    const double sd = in_lds ? ss[j] : row[j].y;
    if (mu > -DBL_MAX) {
      const double n = rows_of(j), d = mu - mx;
      s1 += n * d;
      s2 += n * (sd * sd + d * d);
    }
  }
  block2(s1, s2, false);
  double t0 = a;
  {
    const double N = (double)L;
    const double m1 = s1 / N;
    const double var = s2 / N - m1 * m1;
    if (var > 0.0) {
      const double sbar = sqrt(var);
      const double target = -log(N) - (double)M * log(sbar);  // ln E[(Y - c)_+^M] at the root
      double c = 0.0;
      for (int it = 0; it < 12; ++it) {
        double pm, pm1;
        normal_partial_moments<M>(c, pm, pm1);
        if (!(pm > 0.0)) break;
        const double h = log(pm) - target;
        const double dh = -(double)M * pm1 / pm;
        const double step = -h / dh;
        c += step;
        if (fabs(step) <= 1e-6 * fmax(1.0, fabs(c))) break;
      }
      t0 = fmin(fmax(mx + m1 + c * sbar, a), z);
    }
  }

  // f(t) = sum_p n_p E[(A_p - t)_+^M] and g(t) = -f'(t) / M, over the pages
  // that can reach t (a page with mu + 9 s below the bracket's left end adds
  // less than 1e-19 n s^M). sums64 in float64; sums32 entirely in float32, a
  // cheaper first approximation (its cancellation in the far tail only
  // touches pages whose share of the sum is negligible there).
  auto term64 = [&](double mu, double s, double n, double t, double& f, double& g) {
    if (s > 0.0) {
      if (mu + kGaussReach * s <= a) return;
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
  auto term32 = [&](float mu, float s, float n, float t, float a32, float& f, float& g) {
    if (s > 0.0f) {
      if (mu + (float)kGaussReach * s <= a32) return;
      float pm, pm1;
      // (clamped so that its powers stay finite in float32; only the float64
      // steps that follow decide tau_hat)
      const float c = fminf(fmaxf((t - mu) * __frcp_rn(s), -1.0e4f), 1.0e4f);
      normal_partial_moments_f<M>(c, pm, pm1);
      float sm1 = 1.0f;
#pragma unroll
      for (int i = 0; i < M - 1; ++i) sm1 *= s;
      f += n * sm1 * s * pm;
      g += n * sm1 * pm1;
    } else if (mu > t) {
      const float d = mu - t;
      float dm1 = 1.0f;
#pragma unroll
      for (int i = 0; i < M - 1; ++i) dm1 *= d;
      f += n * dm1 * d;
      g += n * dm1;
    }
  };
  auto sums = [&](auto f32, double t, double& f, double& g) {
    constexpr bool F32 = decltype(f32)::value;
    f = 0.0;
    g = 0.0;
    if constexpr (F32) {
      float ff = 0.0f, gg = 0.0f;
      const float tf = (float)t, af = (float)a;
#pragma unroll 1
      for (int j = tid; j < P; j += NT) {
        double mu, sd;
        if (in_lds) {
          mu = smu[j];
          sd = ss[j];
        } else {
          const double2 v = row[j];
          mu = v.x;
          sd = v.y;
        }
        term32((float)mu, (float)sd, (float)rows_of(j), tf, af, ff, gg);
      }
      f = ff;
      g = gg;
    } else {
#pragma unroll 1
      for (int j = tid; j < P; j += NT) {
        if (in_lds) {
          term64(smu[j], ss[j], rows_of(j), t, f, g);
        } else {
          const double2 v = row[j];
          term64(v.x, v.y, rows_of(j), t, f, g);
        }
      }
    }
    block2(f, g, false);
  };
  // Newton steps on ln f (nearly quadratic for Gaussian tails, so few steps)
  // inside a bracket [lo, hi] that every step shrinks; a step that would
  // leave it bisects instead. First in float32 from the pooled start, to
  // about 1e-4 of f (on a bracket of its own: float32 may misjudge which side
  // of the root a point is on), then in float64 from there on the float64
  // bracket: from that start Newton's quadratic convergence reaches the
  // sum's rounding level in two steps.
  // tol: stop when |f - 1| <= tol; last: when |f - 1| <= last, take that
  // step and stop (from there one quadratic step reaches the rounding
  // level); rel: stop when a step or the bracket is below rel of t.
  auto newton = [&](auto f32, double t, double lo, double hi, double tol, double last,
                    double rel, int iters) {
    for (int it = 0; it < iters; ++it) {
      double f, g;
      sums(f32, t, f, g);
      if (f >= 1.0) lo = t;
      else hi = t;
      if (fabs(f - 1.0) <= tol) break;
      double tn = 0.5 * (lo + hi);
      if (f > 0.0 && g > 0.0) {
        const double tt = t + log(f) * f / ((double)M * g);
        if (tt > lo && tt < hi) tn = tt;
      }
      const double scale = fmax(1.0, fabs(t));
      if (fabs(f - 1.0) <= last || fabs(tn - t) <= rel * scale || hi - lo <= rel * scale) {
        t = tn;
        break;
      }
      t = tn;
    }
    return t;
  };
  double t = newton(std::true_type{}, t0, a, z, 1e-4, 0.0, 1e-6, kGaussIters);
  t = newton(std::false_type{}, fmin(fmax(t, a), z), a, z, 1e-13, 1e-7, 1e-14, kGaussIters);

  // one key per page: the estimated maximum, or -inf off the rule
  const double cut = t - delta;
  const double spread_full = sqrt(2.0 * log((double)ps));  // every page but the last is full
  auto key = [&](double mu, double s, double n) {
    const double spread = n == (double)ps ? spread_full : (n >= 2.0 ? sqrt(2.0 * log(n)) : 0.0);
    const double est = mu + s * spread;
    return est > cut ? (float)est + 0.0f : -__builtin_inff();
  };
  for (int j = tid; j < P; j += NT) {
    if (in_lds) {
      krow[j] = key(smu[j], ss[j], rows_of(j));
    } else {
      const double2 v = row[j];
      krow[j] = key(v.x, v.y, rows_of(j));
    }
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
      hipLaunchKernelGGL(gauss_solve_kernel<1>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
    case 2:
      hipLaunchKernelGGL(gauss_solve_kernel<2>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
    case 3:
      hipLaunchKernelGGL(gauss_solve_kernel<3>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat);
      break;
    default:
      hipLaunchKernelGGL(gauss_solve_kernel<4>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
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
