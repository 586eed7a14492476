// Device helpers shared by the kernels: bf16 widening, wave64 shuffles and
// reductions, block scans, and the multi-value butterfly used to finish
// several dot products at once across the lanes that share a row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ekv {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // bf16 bit pattern

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

template <>
__device__ __forceinline__ double shfl_xor<double>(double v, int mask) {
  int2 p = *reinterpret_cast<int2*>(&v);
  p.x = __shfl_xor(p.x, mask, kWave);
  p.y = __shfl_xor(p.y, mask, kWave);
  return *reinterpret_cast<double*>(&p);
}

// Larger float -> larger unsigned key (total order on finite values, +0 > -0;
// callers fold -0 into +0 first).
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, shfl_xor(v, m));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, shfl_xor(v, m));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive block prefix sum of one int per thread. `tmp` holds at least
// NT/64 ints of LDS. Returns the exclusive prefix; *total gets the sum.
// Contains barriers: every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  constexpr int NW = NT / kWave;
  int inc = wave_incl_scan(v, lane);
  if (lane == kWave - 1) tmp[wid] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int s = tmp[w];
    base += (w < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* tmp, Op op) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = op(v, shfl_xor(v, m));
  if (lane == 0) tmp[wid] = v;
  __syncthreads();
  T r = tmp[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = op(r, tmp[w]);
  __syncthreads();
  return r;
}

// Multi-value butterfly. NV partial sums v[0..NV) are spread over groups of
// LT lanes (lane bits below log2(LT) pick the lane within a group; LT and NV
// are powers of two). After the call each lane holds CNT = max(1, NV/LT)
// complete sums in v[0..CNT): value indices first_index(lane) + i. Each
// halving step exchanges half of the values still held, so the work is
// NV/2 + NV/4 + ... shuffles instead of NV*log2(LT).
template <int NV, int LT>
struct Butterfly {
  static constexpr int CNT = NV > LT ? NV / LT : 1;

  template <typename T>
  __device__ __forceinline__ static void reduce(T (&v)[NV], int lane) {
    step<T, LT / 2, NV>(v, lane);
  }

  template <typename T, int W, int C>
  __device__ __forceinline__ static void step(T (&v)[NV], int lane) {
    if constexpr (W >= 1) {
      if constexpr (C > 1) {
        constexpr int H = C / 2;
        const bool up = (lane & W) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          T send = up ? v[i] : v[H + i];
          T keep = up ? v[H + i] : v[i];
          v[i] = keep + shfl_xor(send, W);
        }
        step<T, W / 2, H>(v, lane);
      } else {
        v[0] += shfl_xor(v[0], W);
        step<T, W / 2, C>(v, lane);
      }
    }
  }

  // Value index of v[0] on this lane after reduce().
  __device__ __forceinline__ static int first_index(int lane) {
    int idx = 0;
    int c = NV;
#pragma unroll
    for (int w = LT / 2; w >= 1; w >>= 1) {
      if (c > 1) {
        c >>= 1;
        if (lane & w) idx += c;
      }
    }
    return idx;
  }

  // Lanes whose bits below DUP are zero own their sums; the others hold copies.
  static constexpr int DUP = NV >= LT ? 1 : LT / NV;
  __device__ __forceinline__ static bool owner(int lane) { return (lane & (DUP - 1)) == 0; }
};

// MFMA operand types (gfx950 v_mfma_f32_16x16x32_bf16). Lane l holds
// A[l % 16][(l / 16) * 8 + j], B[(l / 16) * 8 + j][l % 16] for j < 8, and
// D[(l / 16) * 4 + i][l % 16] for i < 4.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// Part `part` (0, 1, 2) of the exact split x = p0 + p1 + p2 into bf16 values:
// p0 = rne(x), p1 = rne(x - p0), p2 = x - p0 - p1. Each difference is exact
// in float32 (the operands are within a factor of two), and the last
// remainder has at most 8 significant bits, so it is a bf16 value.
__device__ __forceinline__ uint32_t bf16_part(float x, int part) {
  const uint32_t p0 = bf16_rne_bits(x);
  const float r1 = x - __uint_as_float(p0 << 16);
  const uint32_t p1 = bf16_rne_bits(r1);
  const float r2 = r1 - __uint_as_float(p1 << 16);
  const uint32_t p2 = bf16_rne_bits(r2);
  return part == 0 ? p0 : (part == 1 ? p1 : (part == 2 ? p2 : 0u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int clamp_len(int L, int max_tokens) {
  return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

}  // namespace ekv
