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
// gauss_stats_kernel: one workgroup per (chunk of 64 pages, (b, KV head));
//   a page's moment record [mean | var] is split over D/4 lanes, the G
//   heads' two dot products are formed in float64, and each wave's partials
//   are transposed through LDS so that a lane adds up 2G of one sum before a
//   short DPP butterfly; (mu_a, s_a) per (b, h, page) go to the workspace.
// gauss_solve_kernel: one workgroup of 512 threads per (b, h), the head's
//   page statistics staged in LDS: tau_hat by Halley steps on the logarithm
//   of the equation's left side (nearly quadratic in t for Gaussian tails),
//   safeguarded by a bracket that bisects when a step would leave it; then
//   one key per page (its estimated maximum as float32, or -inf when it fails
//   the rule), and the top-cap select over those keys by the same workgroup
//   (the radix select of the top-k path, -inf keys not candidates).
#include <cfloat>
#include <type_traits>

#include "erfc_fit.hpp"
#include "launch.hpp"
#include "select_impl.hpp"

namespace ekv {

constexpr int kGaussPages = 64;    // pages per workgroup of the statistics kernel
constexpr int kGaussNT = 512;      // threads of a solve workgroup (one per (b, h))
constexpr int kGaussLds = 4096;    // pages of a head a solve workgroup holds in LDS
constexpr int kGaussIters = 100;   // most solve steps
constexpr double kGaussReach = 9.0;  // pages with mu_a + 9 s_a <= the bracket's left end
                                     // contribute below 1e-19 n_p s_a^m: left out of the sums

// Orders a wave's LDS writes before its later LDS reads (a wave's LDS
// instructions execute in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
  // a wave's partial sums are transposed through LDS: each lane writes its
  // NV partials (mu and s^2 of every head) of its page, then adds up NV
  // partials of one sum, and the R lanes that share a sum combine theirs
  // by DPP lane swaps
  constexpr int NW = 256 / kWave;
  constexpr int PPW = kWave / LP;        // pages per wave and step
  constexpr int NV = 2 * G;              // sums per page: rows 2h (mu), 2h + 1 (s^2)
  constexpr int R = LP / NV;             // lanes per sum
  constexpr int ROW = LP * 8 + 16;       // bytes per row of LP partials, padded
  static_assert(R >= 1 && R * NV == LP && R * PPW * NV == kWave, "group size must not exceed lanes per page");
  static_assert(kGaussPages % PPB == 0, "whole block steps");
  __shared__ int sphys[kGaussPages];
  __shared__ __align__(16) unsigned char red[NW][PPW * NV * ROW];

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
  const int wv = (int)threadIdx.x / kWave;
  unsigned char* wred = red[wv];
  const int o = lane / R, k = lane % R;  // the sum this lane adds up, its part
  const int po = o / NV, ro = o % NV;     // its page in the wave, its row
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
    const int pw = lane / LP;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<double*>(wred + (pw * NV + 2 * h) * ROW + c * 8) = mu[h];
      *reinterpret_cast<double*>(wred + (pw * NV + 2 * h + 1) * ROW + c * 8) = s2[h];
    }
    wave_lds_sync();
    const double2* part = reinterpret_cast<const double2*>(wred + o * ROW + k * NV * 8);
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
      const double2 d = part[i];
      sum += d.x;
      sum += d.y;
    }
    wave_lds_sync();  // the next step's partials go to the same rows
    if constexpr (R >= 2) sum += partner<1>(sum);
    if constexpr (R >= 4) sum += partner<2>(sum);
    if constexpr (R >= 8) sum += partner<4>(sum);
    if constexpr (R >= 16) sum += partner<8>(sum);
    if constexpr (R >= 32) sum += partner<16>(sum);
    const double s2sum = partner<R>(sum);  // row 2h + 1 (every lane of it holds the sum)
    const int jj = t * PPB + wv * PPW + po;
    // a page past the block table's valid range (an input outside the
    // contract) gets a neutral entry: it adds nothing to tau_hat's sum and
    // its key is -inf
    if (jj < n && k == 0 && (ro & 1) == 0) {
      const int phys = sphys[jj];
      stats[(size_t)(h0 + ro / 2) * ldu + j0 + jj] =
          phys >= 0 && phys < num_phys ? make_double2(am1 * sum, am1 * sqrt(fmax(s2sum, 0.0)))
                                       : make_double2(-DBL_MAX, 0.0);
    }
  }
}

// Clenshaw's recurrence for sum_k coef[k] T_k(x).
template <typename T, int N>
__device__ __forceinline__ T cheb_series(const T (&coef)[N], T x) {
  T b1 = 0, b2 = 0;
  const T x2 = x + x;
#pragma unroll
  for (int k = N - 1; k >= 1; --k) {
    const T b0 = fma(x2, b1, -b2) + coef[k];
    b2 = b1;
    b1 = b0;
  }
  return fma(x, b1, -b2) + coef[0];
}

// Q(c) = P(Y > c) for Y ~ N(0, 1), given e = exp(-c^2 / 2) (the normal
// density's exponential, which the caller needs too): for z = |c| / sqrt 2,
// erfc(z) = t h(t) e with t = 1 / (1 + z / K) and h the fitted Chebyshev
// series of erfc_fit.hpp (no branches; one reciprocal), and Q(c) = erfc(z)
// / 2 for c >= 0, 1 - erfc(z) / 2 below.
__device__ __forceinline__ double normal_tail(double c, double e) {
  const double t = 1.0 / (1.0 + fabs(c) * (0.7071067811865476 / kErfcK));
  const double q = 0.5 * t * cheb_series(kErfcC64, 2.0 * t - 1.0) * e;
  return c >= 0.0 ? q : 1.0 - q;
}
__device__ __forceinline__ float normal_tail_f(float c, float e) {
  const float t = __builtin_amdgcn_rcpf(1.0f + fabsf(c) * (float)(0.7071067811865476 / kErfcK));
  const float q = 0.5f * t * cheb_series(kErfcC32, 2.0f * t - 1.0f) * e;
  return c >= 0.0f ? q : 1.0f - q;
}

constexpr int binomial(int m, int k) {
  int r = 1;
  for (int i = 0; i < k; ++i) r = r * (m - i) / (i + 1);
  return r;
}

// E[(Y - c)_+^k] for Y ~ N(0, 1) and k = M, M - 1, M - 2 (M in 1..4) in
// pm[0..2] (for M = 1, pm[2] is the density phi(c), the derivative of
// pm[1] = Q(c) with the sign flipped), from the truncated moments
// J_k = E[Y^k; Y > c]: J_0 = Q(c), J_1 = phi(c),
// J_k = c^(k-1) phi(c) + (k-1) J_(k-2), and the binomial expansion of
// (Y - c)^k. Clamped at 0 (the expansion cancels to rounding noise where
// phi underflows). T = double, or float for a cheaper first approximation
// of tau_hat (the expansion's cancellation in the far tail only touches
// pages whose share of the sum is negligible there).
template <int M, typename T>
__device__ __forceinline__ void normal_partial_moments(T c, T (&pm)[3]) {
  constexpr bool F64 = std::is_same<T, double>::value;
  T e, q;
  if constexpr (F64) {
    e = exp(-0.5 * c * c);
    q = normal_tail(c, e);
  } else {
    e = __expf(-0.5f * c * c);
    q = normal_tail_f(c, e);
  }
  const T phi = (T)0.3989422804014327 * e;  // 1/sqrt(2 pi)
  T J[M + 1];
  J[0] = q;
  J[1] = phi;
#pragma unroll
  for (int k = 2; k <= M; ++k) {
    T ck = 1;
#pragma unroll
    for (int i = 0; i < k - 1; ++i) ck *= c;
    J[k] = ck * phi + (T)(k - 1) * J[k - 2];
  }
  auto expand = [&](auto mc) {
    constexpr int m = decltype(mc)::value;
    // sum_k binom(m, k) (-c)^(m-k) J_k
    T s = 0;
#pragma unroll
    for (int k = m; k >= 0; --k) {
      T p = 1;
#pragma unroll
      for (int i = 0; i < m - k; ++i) p *= -c;
      s += (T)binomial(m, k) * p * J[k];
    }
    return s > 0 ? s : (T)0;
  };
  pm[0] = expand(std::integral_constant<int, M>{});
  pm[1] = expand(std::integral_constant<int, M - 1>{});
  if constexpr (M >= 2) pm[2] = expand(std::integral_constant<int, M - 2>{});
  else pm[2] = phi;
}

// Halley's step for the root of F(x) = ln E(x) - const, where E(x) =
// sum n (A - x)_+^M-type terms with E' = -M E1 and E'' = kH E2 (kH =
// M (M - 1), or 1 for M = 1): F' = -M E1 / E, F'' = kH E2 / E - F'^2, and
// the step is -2 F F' / (2 F'^2 - F F'') (Newton's -F / F' where that
// denominator is not positive). Fv = F(x), e0..e2 = E, E1, E2 at x.
template <int M>
__device__ __forceinline__ double halley_step(double Fv, double e0, double e1, double e2) {
  constexpr double kH = M >= 2 ? (double)(M * (M - 1)) : 1.0;
  const double F1 = -(double)M * e1 / e0;
  const double F2 = kH * e2 / e0 - F1 * F1;
  const double den = 2.0 * F1 * F1 - Fv * F2;
  return den > 0.0 ? -2.0 * Fv * F1 / den : -Fv / F1;
}

template <int M>
__global__ void __launch_bounds__(kGaussNT)
gauss_solve_kernel(const double2* __restrict__ stats, const int32_t* __restrict__ seq_lens,
                   int H, int ps, int max_pages, int ldu, double delta, float* __restrict__ keys,
                   float* __restrict__ tau_hat, int cap, int32_t* __restrict__ sel) {
  constexpr int NT = kGaussNT, NW = NT / kWave;
  static_assert(3 * kGaussLds * sizeof(double) >= kSelLds * sizeof(uint32_t),
                "the select's staging reuses the statistics' LDS");
  __shared__ double red[3 * NW];
  // (mu, s, 1/s) of the head's pages; after the keys are written, the
  // select's key staging
  __shared__ __align__(16) double lds_d[3 * kGaussLds];
  __shared__ SelectScratch<NT> sel_sh;
  double* smu = lds_d;
  double* ss = lds_d + kGaussLds;
  double* sinv = lds_d + 2 * kGaussLds;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int bh = blockIdx.x, b = bh / H;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  const double2* row = stats + (size_t)bh * ldu;
  float* krow = keys + (size_t)bh * ldu;
  int32_t* srow = sel + (size_t)bh * cap;
  if (P == 0) {
    if (tid == 0 && tau_hat) tau_hat[bh] = __builtin_nanf("");
    for (int i = tid; i < cap; i += NT) srow[i] = -1;
    return;
  }
  auto rows_of = [&](int j) { return (double)min(ps, L - j * ps); };
  // N sums (or maxima) over the workgroup, the same on every thread
  auto block_reduce = [&](auto nc, double(&x)[decltype(nc)::value], bool is_max) {
    constexpr int N = decltype(nc)::value;
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = is_max ? wave_max(x[i]) : wave_allsum(x[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) red[N * wid + i] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = red[i];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] = is_max ? fmax(x[i], red[N * w + i]) : x[i] + red[N * w + i];
    }
    __syncthreads();
  };
  auto block2 = [&](double& x, double& y, bool is_max) {
    double v[2] = {x, y};
    block_reduce(std::integral_constant<int, 2>{}, v, is_max);
    x = v[0];
    y = v[1];
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
      sinv[j] = v.y > 0.0 ? 1.0 / v.y : 0.0;
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
  // N sbar^M E[(Y - c)_+^M] = 1 solved for c by Halley steps on the log of
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
        double pm[3];
        normal_partial_moments<M>(c, pm);
        if (!(pm[0] > 0.0)) break;
        const double step = halley_step<M>(log(pm[0]) - target, pm[0], pm[1], pm[2]);
        c += step;
        if (fabs(step) <= 1e-6 * fmax(1.0, fabs(c))) break;
      }
      t0 = fmin(fmax(mx + m1 + c * sbar, a), z);
    }
  }

  // f(t) = sum_p n_p E[(A_p - t)_+^M], g(t) = -f'(t) / M and h(t) =
  // f''(t) / kH over the pages that can reach t (a page with mu + 9 s below
  // the bracket's left end adds less than 1e-19 n s^M). In float64, or
  // entirely in float32 for a cheaper first approximation (its cancellation
  // in the far tail only touches pages whose share of the sum is negligible
  // there; c is clamped so that its powers stay finite, and only the float64
  // step that follows decides tau_hat).
  auto term = [&](auto mu, auto s, auto inv_s, auto n, auto t, auto lo, auto (&acc)[3]) {
    using T = decltype(mu);
    T v0 = 0, v1 = 0, v2 = 0;  // this page's f, g and h
    if (s > (T)0) {
      if (mu + (T)kGaussReach * s <= lo) return;
      T c = (t - mu) * inv_s;
      if constexpr (!std::is_same<T, double>::value) c = fminf(fmaxf(c, -1.0e4f), 1.0e4f);
      T pm[3];
      normal_partial_moments<M>(c, pm);
      T sm2 = 1;  // s^(M-2) for M >= 2
#pragma unroll
      for (int i = 0; i < M - 2; ++i) sm2 *= s;
      const T sm1 = M >= 2 ? sm2 * s : (T)1;  // s^(M-1)
      v0 = n * sm1 * s * pm[0];
      v1 = n * sm1 * pm[1];
      v2 = n * (M >= 2 ? sm2 : inv_s) * pm[2];
    } else if (mu > t) {
      const T d = mu - t;
      T dm2 = 1;  // d^(M-2) for M >= 2
#pragma unroll
      for (int i = 0; i < M - 2; ++i) dm2 *= d;
      v0 = M >= 2 ? n * dm2 * d * d : n * d;
      v1 = M >= 2 ? n * dm2 * d : n;
      v2 = M >= 2 ? n * dm2 : (T)0;
    }
    acc[0] += v0;
    acc[1] += v1;
    acc[2] += v2;
  };
  auto sums = [&](auto f32, double t, double (&fgh)[3]) {
    constexpr bool F32 = decltype(f32)::value;
    if constexpr (F32) {
      float acc[3] = {0.0f, 0.0f, 0.0f};
      const float tf = (float)t, af = (float)a;
#pragma unroll 1
      for (int j = tid; j < P; j += NT) {
        double mu, sd, si;
        if (in_lds) {
          mu = smu[j];
          sd = ss[j];
          si = sinv[j];
        } else {
          const double2 v = row[j];
          mu = v.x;
          sd = v.y;
          si = sd > 0.0 ? 1.0 / sd : 0.0;
        }
        term((float)mu, (float)sd, (float)si, (float)rows_of(j), tf, af, acc);
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) fgh[i] = acc[i];
    } else {
#pragma unroll
      for (int i = 0; i < 3; ++i) fgh[i] = 0.0;
#pragma unroll 1
      for (int j = tid; j < P; j += NT) {
        if (in_lds) {
          term(smu[j], ss[j], sinv[j], rows_of(j), t, a, fgh);
        } else {
          const double2 v = row[j];
          term(v.x, v.y, v.y > 0.0 ? 1.0 / v.y : 0.0, rows_of(j), t, a, fgh);
        }
      }
    }
    block_reduce(std::integral_constant<int, 3>{}, fgh, false);
  };
  // Halley steps on ln f (cubic convergence; ln f is nearly quadratic in t
  // for Gaussian tails) inside a bracket [lo, hi] that every step shrinks; a
  // step that would leave it bisects instead. First in float32 from the
  // pooled start, to about 1e-5 of f (on a bracket of its own: float32 may
  // misjudge which side of the root a point is on), then in float64 from
  // there on the float64 bracket: from within 1e-5 one cubic step reaches
  // the sum's rounding level.
  // tol: stop when |f - 1| <= tol; last: when |f - 1| <= last, take that
  // step and stop; rel: stop when a step or the bracket is below rel of t.
  auto solve = [&](auto f32, double t, double lo, double hi, double tol, double last,
                   double rel, int iters) {
    for (int it = 0; it < iters; ++it) {
      double fgh[3];
      sums(f32, t, fgh);
      const double f = fgh[0];
      if (f >= 1.0) lo = t;
      else hi = t;
      if (fabs(f - 1.0) <= tol) break;
      double tn = 0.5 * (lo + hi);
      if (f > 0.0 && fgh[1] > 0.0) {
        const double tt = t + halley_step<M>(log(f), f, fgh[1], fgh[2]);
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
  double t = solve(std::true_type{}, t0, a, z, 1e-5, 0.0, 1e-6, kGaussIters);
  t = solve(std::false_type{}, fmin(fmax(t, a), z), a, z, 1e-13, 1e-5, 1e-14, kGaussIters);

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

  // the capped select over the keys just written (a workgroup-scope barrier
  // orders their stores before its loads; the statistics' LDS is dead)
  __syncthreads();
  const int kept = select_row<NT, true, false>(
      krow, reinterpret_cast<const uint64_t*>(krow), P, cap, 0, 0, ldu,
      reinterpret_cast<uint32_t*>(lds_d), sel_sh,
      [&](int pos, int page, uint32_t) { srow[pos] = page; });
  for (int i = kept + tid; i < cap; i += NT) srow[i] = -1;
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
                              double delta, float* keys, float* tau_hat, int cap, int32_t* sel,
                              hipStream_t st) {
  const int heads = s.batch * s.num_q_heads;
  const double2* st2 = static_cast<const double2*>(stats);
  const int ldu = ub_ld(s.max_pages);
  switch (m) {
    case 1:
      hipLaunchKernelGGL(gauss_solve_kernel<1>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat, cap, sel);
      break;
    case 2:
      hipLaunchKernelGGL(gauss_solve_kernel<2>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat, cap, sel);
      break;
    case 3:
      hipLaunchKernelGGL(gauss_solve_kernel<3>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat, cap, sel);
      break;
    default:
      hipLaunchKernelGGL(gauss_solve_kernel<4>, dim3(heads), dim3(kGaussNT), 0, st, st2, lens,
                         s.num_q_heads, s.page_size, s.max_pages, ldu, delta, keys, tau_hat, cap, sel);
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
