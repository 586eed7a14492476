// Page bounding-box metadata: per (page, KV head) coordinate-wise min and max
// of the page's valid keys, built for whole sequences (meta_kernel) or
// updated after tokens are appended (append_meta_kernel). EntmaxKV summary
// page (gist.science paper 2605.21649), section 2.A: the box is the
// lightweight per-page metadata that bounds a page's best score.
//
// Each lane owns one 16-byte column chunk of one (page, KV head) item and
// walks all of the page's valid rows, so no cross-lane reduction is needed:
// a wave covers 64 / (head_dim chunks) items at once, and the items of a
// wave are consecutive KV heads of one page (contiguous in the pool). Rows
// are read sixteen at a time with streaming loads. min/max does no rounding,
// so the output is the stored key values.
#include "launch.hpp"
#include "mfma.hpp"

namespace ekv {

template <typename KV, int D>
__global__ void __launch_bounds__(256)
meta_kernel(const KV* __restrict__ k_pool, const int32_t* __restrict__ block_table,
            const int32_t* __restrict__ seq_lens, KV* __restrict__ meta, int B, int Hkv, int ps,
            int max_pages, int num_phys) {
  constexpr int VPC = 16 / sizeof(KV);  // values per 16-byte chunk
  constexpr int CPR = D / VPC;          // lanes per item (chunks per row)
  constexpr int IPW = kWave / CPR;      // items per wave
  constexpr int RB = 16;                // rows per batch of loads
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c = lane % CPR;
  const long long item = ((long long)blockIdx.x * (256 / kWave) + wave) * IPW + lane / CPR;
  const int g = (int)(item % Hkv);
  const long long bj = item / Hkv;
  const int j = (int)(bj % max_pages);
  const int b = (int)(bj / max_pages);
  if (b >= B) return;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  if (j * ps >= L) return;
  const int phys = block_table[(size_t)b * max_pages + j];
  if (phys < 0 || phys >= num_phys) return;
  const int nv = min(ps, L - j * ps);
  const KV* base = k_pool + ((size_t)phys * Hkv + g) * (size_t)ps * D + c * VPC;

  float lo[VPC], hi[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) {
    lo[e] = __builtin_inff();
    hi[e] = -__builtin_inff();
  }
  for (int r0 = 0; r0 < nv; r0 += RB) {
    // every load of the batch issued unconditionally (rows past the valid
    // ones re-read the last valid row, which leaves min and max unchanged),
    // so all RB are in flight before the first is used
    u32x4 x[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
      x[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(base + (size_t)min(r0 + i, nv - 1) * D));
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float f[VPC];
      if constexpr (sizeof(KV) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          f[2 * w] = bf16_lo(x[i][w]);
          f[2 * w + 1] = bf16_hi(x[i][w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) f[w] = __uint_as_float(x[i][w]);
      }
#pragma unroll
      for (int e = 0; e < VPC; ++e) {
        lo[e] = fminf(lo[e], f[e]);
        hi[e] = fmaxf(hi[e], f[e]);
      }
    }
  }
  KV* dst = meta + ((size_t)phys * Hkv + g) * 2 * D + c * VPC;
  uint4 o[2];
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const float* a = side ? hi : lo;
    if constexpr (sizeof(KV) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (__float_as_uint(a[2 * i]) >> 16) | (__float_as_uint(a[2 * i + 1]) & 0xffff0000u);
      o[side] = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      o[side] = make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                           __float_as_uint(a[3]));
    }
  }
  // streaming stores: plain ones made the build ~5 % slower (and the key
  // stream alone, with no store at all, takes ~70 % of the time)
  __builtin_nontemporal_store((u32x4){o[0].x, o[0].y, o[0].z, o[0].w},
                              reinterpret_cast<u32x4*>(dst));
  __builtin_nontemporal_store((u32x4){o[1].x, o[1].y, o[1].z, o[1].w},
                              reinterpret_cast<u32x4*>(dst + D));
}

// Page key moments ([EntmaxKV page] section 2.A, the Gaussian statistics):
// per (page, KV head) and coordinate, the mean and the population variance of
// the page's valid keys. Same lane layout as meta_kernel. The sums run in
// float64 around the page's first row k0 (d = k - k0), so the variance
// s2/n - (s1/n)^2 does not cancel; for bf16 keys every d, d^2 and sum of a
// page is exact. Results are rounded to float32 and then, for bf16 caches,
// to bf16 (each to nearest even).
// kAppend: after tokens [L0, L1) were appended (seq_lens holds L1), items are
// (sequence, KV head, i-th page those tokens touch) as in append_meta_kernel,
// and each touched page is recomputed from all its valid rows: the stored,
// rounded moments cannot be updated in place, and a page's result is the
// same bits as a full build at L1.
template <typename KV, int D, bool kAppend>
__global__ void __launch_bounds__(256)
moments_kernel(const KV* __restrict__ k_pool, const int32_t* __restrict__ block_table,
               const int32_t* __restrict__ old_lens, const int32_t* __restrict__ seq_lens,
               KV* __restrict__ moments, int B, int Hkv, int ps, int max_pages, int num_phys,
               int slots) {
  constexpr int VPC = 16 / sizeof(KV);
  constexpr int CPR = D / VPC;
  constexpr int IPW = kWave / CPR;
  constexpr int RB = 8;  // rows per batch of loads (two float64 sums per value)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c = lane % CPR;
  const long long item = ((long long)blockIdx.x * (256 / kWave) + wave) * IPW + lane / CPR;
  const int g = (int)(item % Hkv);
  const long long rest = item / Hkv;
  const int per_seq = kAppend ? slots : max_pages;
  const int b = (int)(rest / per_seq);
  if (b >= B) return;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  int j = (int)(rest % per_seq);
  if constexpr (kAppend) {
    const int L0 = min(clamp_len(old_lens[b], max_pages * ps), L);
    if (L0 == L) return;
    j += L0 / ps;
  }
  if (j * ps >= L) return;
  const int phys = block_table[(size_t)b * max_pages + j];
  if (phys < 0 || phys >= num_phys) return;
  const int nv = min(ps, L - j * ps);
  const KV* base = k_pool + ((size_t)phys * Hkv + g) * (size_t)ps * D + c * VPC;

  auto widen8 = [](const u32x4& x, float (&f)[VPC]) {
    if constexpr (sizeof(KV) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[2 * w] = bf16_lo(x[w]);
        f[2 * w + 1] = bf16_hi(x[w]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) f[w] = __uint_as_float(x[w]);
    }
  };
  float k0[VPC];
  widen8(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base)), k0);
  double s1[VPC], s2[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) {
    s1[e] = 0.0;
    s2[e] = 0.0;
  }
  for (int r0 = 0; r0 < nv; r0 += RB) {
    // every load of the batch issued (rows past the valid ones re-read the
    // last valid row and are not summed)
    u32x4 x[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
      x[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(base + (size_t)min(r0 + i, nv - 1) * D));
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (r0 + i < nv) {
        float f[VPC];
        widen8(x[i], f);
#pragma unroll
        for (int e = 0; e < VPC; ++e) {
          const double d = (double)f[e] - (double)k0[e];
          s1[e] += d;
          s2[e] = fma(d, d, s2[e]);
        }
      }
    }
  }
  const double n = (double)nv;
  float mean[VPC], var[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) {
    const double m1 = s1[e] / n;
    mean[e] = (float)((double)k0[e] + m1);
    var[e] = (float)fmax(s2[e] / n - m1 * m1, 0.0);
  }
  KV* dst = moments + ((size_t)phys * Hkv + g) * 2 * D + c * VPC;
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const float* a = side ? var : mean;
    u32x4 o;
    if constexpr (sizeof(KV) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = bf16_rne_bits(a[2 * k]) | (bf16_rne_bits(a[2 * k + 1]) << 16);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(a[k]);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + side * D));
  }
}

// Boxes after an append: item = (sequence, KV head, i-th page touched by the
// new tokens [L0, L1)). Same lane layout as meta_kernel; a page whose first
// valid row is new starts from +-inf, a page that already held tokens starts
// from its current box, and both take the min/max of the new rows.
template <typename KV, int D>
__global__ void __launch_bounds__(256)
append_meta_kernel(const KV* __restrict__ k_pool, const int32_t* __restrict__ block_table,
                   const int32_t* __restrict__ old_lens, const int32_t* __restrict__ new_lens,
                   KV* __restrict__ meta, int B, int Hkv, int ps, int max_pages, int num_phys,
                   int slots) {
  constexpr int VPC = 16 / sizeof(KV);
  constexpr int CPR = D / VPC;
  constexpr int IPW = kWave / CPR;
  constexpr int RB = 8;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c = lane % CPR;
  const long long item = ((long long)blockIdx.x * (256 / kWave) + wave) * IPW + lane / CPR;
  const int i = (int)(item % slots);
  const long long bg = item / slots;
  const int g = (int)(bg % Hkv);
  const int b = (int)(bg / Hkv);
  if (b >= B) return;
  const int L1 = clamp_len(new_lens[b], max_pages * ps);
  const int L0 = min(clamp_len(old_lens[b], max_pages * ps), L1);
  if (L0 == L1) return;
  const int j = L0 / ps + i;
  if (j * ps >= L1) return;
  const int phys = block_table[(size_t)b * max_pages + j];
  if (phys < 0 || phys >= num_phys) return;
  const int r0 = max(0, L0 - j * ps), r1 = min(ps, L1 - j * ps);
  const KV* base = k_pool + ((size_t)phys * Hkv + g) * (size_t)ps * D + c * VPC;
  KV* dst = meta + ((size_t)phys * Hkv + g) * 2 * D + c * VPC;

  float lo[VPC], hi[VPC];
  auto widen4 = [](const uint4& x, float (&f)[VPC]) {
    if constexpr (sizeof(KV) == 2) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_lo(w[k]);
        f[2 * k + 1] = bf16_hi(w[k]);
      }
    } else {
      f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
      f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
    }
  };
  if (r0 == 0) {
#pragma unroll
    for (int e = 0; e < VPC; ++e) {
      lo[e] = __builtin_inff();
      hi[e] = -__builtin_inff();
    }
  } else {
    widen4(*reinterpret_cast<const uint4*>(dst), lo);
    widen4(*reinterpret_cast<const uint4*>(dst + D), hi);
  }
  for (int rr = r0; rr < r1; rr += RB) {
    u32x4 x[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k)
      if (rr + k < r1) x[k] = *reinterpret_cast<const u32x4*>(base + (size_t)(rr + k) * D);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      if (rr + k >= r1) break;
      float f[VPC];
      widen4(make_uint4(x[k][0], x[k][1], x[k][2], x[k][3]), f);
#pragma unroll
      for (int e = 0; e < VPC; ++e) {
        lo[e] = fminf(lo[e], f[e]);
        hi[e] = fmaxf(hi[e], f[e]);
      }
    }
  }
  uint4 o[2];
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const float* a = side ? hi : lo;
    if constexpr (sizeof(KV) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = (__float_as_uint(a[2 * k]) >> 16) | (__float_as_uint(a[2 * k + 1]) & 0xffff0000u);
      o[side] = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      o[side] = make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                           __float_as_uint(a[3]));
    }
  }
  *reinterpret_cast<uint4*>(dst) = o[0];
  *reinterpret_cast<uint4*>(dst + D) = o[1];
}

template <typename KV, int D>
static hipError_t launch_append_meta_t(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                                       const int32_t* old_lens, const int32_t* new_lens,
                                       int max_new, void* meta, hipStream_t st) {
  constexpr int IPB = (256 / kWave) * (kWave / (D / (16 / sizeof(KV))));  // items per block
  // pages one sequence's new tokens can touch: the partly filled last page
  // plus ceil(max_new / ps) more, never more than the table has
  long long slots = ((long long)max_new + s.page_size - 1) / s.page_size + 1;
  if (slots > s.max_pages) slots = s.max_pages;
  const long long items = (long long)s.batch * s.num_kv_heads * slots;
  const long long blocks = (items + IPB - 1) / IPB;
  hipLaunchKernelGGL((append_meta_kernel<KV, D>), dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const KV*>(k_pool), bt, old_lens, new_lens, static_cast<KV*>(meta),
                     s.batch, s.num_kv_heads, s.page_size, s.max_pages, s.num_phys, (int)slots);
  return hipGetLastError();
}

hipError_t launch_append_meta(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                              const int32_t* old_lens, const int32_t* new_lens, int max_new,
                              void* meta, hipStream_t st) {
  if (s.bf16) {
    if (s.head_dim == 64)
      return launch_append_meta_t<bf16_t, 64>(s, k_pool, bt, old_lens, new_lens, max_new, meta, st);
    return launch_append_meta_t<bf16_t, 128>(s, k_pool, bt, old_lens, new_lens, max_new, meta, st);
  }
  if (s.head_dim == 64)
    return launch_append_meta_t<float, 64>(s, k_pool, bt, old_lens, new_lens, max_new, meta, st);
  return launch_append_meta_t<float, 128>(s, k_pool, bt, old_lens, new_lens, max_new, meta, st);
}

template <typename KV, int D>
static hipError_t launch_meta_t(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                                const int32_t* lens, void* meta, hipStream_t st) {
  constexpr int IPB = (256 / kWave) * (kWave / (D / (16 / sizeof(KV))));  // items per block
  const long long items = (long long)s.batch * s.max_pages * s.num_kv_heads;
  const long long blocks = (items + IPB - 1) / IPB;
  hipLaunchKernelGGL((meta_kernel<KV, D>), dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const KV*>(k_pool), bt, lens, static_cast<KV*>(meta), s.batch,
                     s.num_kv_heads, s.page_size, s.max_pages, s.num_phys);
  return hipGetLastError();
}

// old_lens == nullptr: every page of every sequence; else only the pages the
// tokens [old_lens, lens) touch, at most max_new tokens per sequence.
template <typename KV, int D>
static hipError_t launch_moments_t(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                                   const int32_t* old_lens, const int32_t* lens, int max_new,
                                   void* moments, hipStream_t st) {
  constexpr int IPB = (256 / kWave) * (kWave / (D / (16 / sizeof(KV))));  // items per block
  long long slots = s.max_pages;
  if (old_lens) {
    // the partly filled last page plus ceil(max_new / ps) more
    slots = ((long long)max_new + s.page_size - 1) / s.page_size + 1;
    if (slots > s.max_pages) slots = s.max_pages;
  }
  const long long items = (long long)s.batch * slots * s.num_kv_heads;
  const long long blocks = (items + IPB - 1) / IPB;
  if (old_lens)
    hipLaunchKernelGGL((moments_kernel<KV, D, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const KV*>(k_pool), bt, old_lens, lens,
                       static_cast<KV*>(moments), s.batch, s.num_kv_heads, s.page_size,
                       s.max_pages, s.num_phys, (int)slots);
  else
    hipLaunchKernelGGL((moments_kernel<KV, D, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const KV*>(k_pool), bt, nullptr, lens,
                       static_cast<KV*>(moments), s.batch, s.num_kv_heads, s.page_size,
                       s.max_pages, s.num_phys, (int)slots);
  return hipGetLastError();
}

hipError_t launch_moments(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                          const int32_t* old_lens, const int32_t* lens, int max_new,
                          void* moments, hipStream_t st) {
  if (s.bf16) {
    if (s.head_dim == 64)
      return launch_moments_t<bf16_t, 64>(s, k_pool, bt, old_lens, lens, max_new, moments, st);
    return launch_moments_t<bf16_t, 128>(s, k_pool, bt, old_lens, lens, max_new, moments, st);
  }
  if (s.head_dim == 64)
    return launch_moments_t<float, 64>(s, k_pool, bt, old_lens, lens, max_new, moments, st);
  return launch_moments_t<float, 128>(s, k_pool, bt, old_lens, lens, max_new, moments, st);
}

hipError_t launch_meta(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                       const int32_t* lens, void* meta, hipStream_t st) {
  if (s.bf16) {
    if (s.head_dim == 64) return launch_meta_t<bf16_t, 64>(s, k_pool, bt, lens, meta, st);
    return launch_meta_t<bf16_t, 128>(s, k_pool, bt, lens, meta, st);
  }
  if (s.head_dim == 64) return launch_meta_t<float, 64>(s, k_pool, bt, lens, meta, st);
  return launch_meta_t<float, 128>(s, k_pool, bt, lens, meta, st);
}

}  // namespace ekv
