// Matrix-core and direct-to-LDS helpers shared by the page-bound and the
// score kernels (gfx950).
#pragma once

#include "common.hpp"

namespace ekv {

// Matrix-core operand types (v_mfma_f32_16x16x32_bf16): lane l holds
// A[l % 16][(l / 16) * 8 + j] and B[(l / 16) * 8 + j][l % 16] for j < 8, and
// D[(l / 16) * 4 + i][l % 16] for i < 4.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 bits of x rounded to nearest even (x finite).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// Part `part` (0, 1, 2; 0 bits otherwise) of the exact split
// x = p0 + p1 + p2 into bf16 values: p0 = rne(x), p1 = rne(x - p0),
// p2 = x - p0 - p1. Each remainder is exact in float32 and the last one has
// at most 8 significant bits, so it is itself a bf16 value.
__device__ __forceinline__ uint32_t bf16_part(float x, int part) {
  const uint32_t p0 = bf16_rne_bits(x);
  const float r1 = x - __uint_as_float(p0 << 16);
  const uint32_t p1 = bf16_rne_bits(r1);
  const float r2 = r1 - __uint_as_float(p1 << 16);
  const uint32_t p2 = bf16_rne_bits(r2);
  return part == 0 ? p0 : (part == 1 ? p1 : (part == 2 ? p2 : 0u));
}

// bf16_part(x, part) when `live`, else 0, computed without branches (all
// three parts, then selects).
__device__ __forceinline__ uint32_t bf16_part_sel(float x, int part, bool live) {
  const uint32_t p0 = bf16_rne_bits(x);
  const float r1 = x - __uint_as_float(p0 << 16);
  const uint32_t p1 = bf16_rne_bits(r1);
  const float r2 = r1 - __uint_as_float(p1 << 16);
  const uint32_t p2 = bf16_rne_bits(r2);
  uint32_t v = p0;
  v = part == 1 ? p1 : v;
  v = part == 2 ? p2 : v;
  return (live && part < 3) ? v : 0u;
}

// Direct-to-LDS 16-byte streaming load: lane i of the wave writes the 16
// bytes at its `src` to LDS bytes [16i, 16i + 16) past `lds` (uniform across
// the wave). Marked non-temporal (cache-policy bit 2): the data is read
// once, and without the hint these loads stream at well under HBM speed.
// Counted by vmcnt like any vector-memory load.
__device__ __forceinline__ void lds_load16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 2);
}

// s_waitcnt that waits until at most n vector-memory operations of this wave
// are outstanding (other counters left alone); n < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((((N >> 4) & 3) << 14) | (0xF << 8) | (0x7 << 4) | (N & 15));
}

// s_waitcnt for at most N + extra outstanding vector-memory operations,
// extra a wave-uniform count of stores issued after the operations waited
// for (more than 8 waits as for 8, i.e. longer: never too short).
template <int N>
__device__ __forceinline__ void wait_vmcnt_plus(int extra) {
  switch (extra) {
    case 0: wait_vmcnt<N>(); break;
    case 1: wait_vmcnt<N + 1>(); break;
    case 2: wait_vmcnt<N + 2>(); break;
    case 3: wait_vmcnt<N + 3>(); break;
    case 4: wait_vmcnt<N + 4>(); break;
    case 5: wait_vmcnt<N + 5>(); break;
    case 6: wait_vmcnt<N + 6>(); break;
    case 7: wait_vmcnt<N + 7>(); break;
    default: wait_vmcnt<N + 8>(); break;
  }
}

}  // namespace ekv
