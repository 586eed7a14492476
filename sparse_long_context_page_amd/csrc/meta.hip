// Page bounding-box metadata: per (page, KV head) coordinate-wise min and max
// of the page's valid keys. EntmaxKV summary page (gist.science paper
// 2605.21649), section 2.A: the box is the lightweight per-page metadata
// that bounds a page's best score.
//
// One workgroup per (logical page, sequence, KV head); the page's keys are a
// contiguous page_size x head_dim block. Threads own one 16-byte column
// chunk each and walk a strided subset of the rows; partial results meet in
// LDS. min/max does no rounding, so the output is the stored key values.
#include "launch.hpp"

namespace ekv {

template <typename KV, int D>
__global__ void __launch_bounds__(256)
meta_kernel(const KV* __restrict__ k_pool, const int32_t* __restrict__ block_table,
            const int32_t* __restrict__ seq_lens, KV* __restrict__ meta, int Hkv, int ps,
            int max_pages, int num_phys) {
  constexpr int VPC = 16 / sizeof(KV);  // values per 16-byte chunk
  constexpr int CPR = D / VPC;          // chunks per row
  constexpr int RG = 256 / CPR;         // row groups
  __shared__ float smin[RG][CPR][VPC];
  __shared__ float smax[RG][CPR][VPC];

  const int j = blockIdx.x, b = blockIdx.y, g = blockIdx.z;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  if (j * ps >= L) return;
  const int phys = block_table[(size_t)b * max_pages + j];
  if (phys < 0 || phys >= num_phys) return;
  const int nv = min(ps, L - j * ps);

  const int c = threadIdx.x % CPR;
  const int r0 = threadIdx.x / CPR;
  const KV* base = k_pool + ((size_t)phys * Hkv + g) * (size_t)ps * D + c * VPC;

  float lo[VPC], hi[VPC];
#pragma unroll
  for (int e = 0; e < VPC; ++e) {
    lo[e] = __builtin_inff();
    hi[e] = -__builtin_inff();
  }
  for (int r = r0; r < nv; r += RG) {
    uint4 x = *reinterpret_cast<const uint4*>(base + (size_t)r * D);
    float f[VPC];
    if constexpr (sizeof(KV) == 2) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      f[0] = __uint_as_float(x.x);
      f[1] = __uint_as_float(x.y);
      f[2] = __uint_as_float(x.z);
      f[3] = __uint_as_float(x.w);
    }
#pragma unroll
    for (int e = 0; e < VPC; ++e) {
      lo[e] = fminf(lo[e], f[e]);
      hi[e] = fmaxf(hi[e], f[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VPC; ++e) {
    smin[r0][c][e] = lo[e];
    smax[r0][c][e] = hi[e];
  }
  __syncthreads();
  if (threadIdx.x < 2 * CPR) {
    const bool want_max = threadIdx.x >= CPR;
    const int cc = threadIdx.x % CPR;
    float acc[VPC];
#pragma unroll
    for (int e = 0; e < VPC; ++e) acc[e] = want_max ? smax[0][cc][e] : smin[0][cc][e];
    const int used = min(RG, nv);
    for (int rg = 1; rg < used; ++rg) {
#pragma unroll
      for (int e = 0; e < VPC; ++e)
        acc[e] = want_max ? fmaxf(acc[e], smax[rg][cc][e]) : fminf(acc[e], smin[rg][cc][e]);
    }
    KV* dst = meta + (((size_t)phys * Hkv + g) * 2 + (want_max ? 1 : 0)) * D + cc * VPC;
    uint4 o;
    if constexpr (sizeof(KV) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (__float_as_uint(acc[2 * i]) >> 16) | (__float_as_uint(acc[2 * i + 1]) & 0xffff0000u);
      o = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3]));
    }
    *reinterpret_cast<uint4*>(dst) = o;
  }
}

template <typename KV, int D>
static hipError_t launch_meta_t(const LaunchShape& s, const void* k_pool, const int32_t* bt,
                                const int32_t* lens, void* meta, hipStream_t st) {
  dim3 grid(s.max_pages, s.batch, s.num_kv_heads);
  hipLaunchKernelGGL((meta_kernel<KV, D>), grid, dim3(256), 0, st,
                     static_cast<const KV*>(k_pool), bt, lens, static_cast<KV*>(meta),
                     s.num_kv_heads, s.page_size, s.max_pages, s.num_phys);
  return hipGetLastError();
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
