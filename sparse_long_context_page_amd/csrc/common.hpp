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

// Inverse of float_order.
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active), with
// DPP only: shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the
// last lane of row 0 (and 2) is added to row 1 (and 3), and that of row 1 to
// rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  (void)lane;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Value held by a partner lane whose index differs from this lane's in bit W
// (W < 16: in bits 0..log2(W) -- a DPP lane swap within a row, no LDS
// traffic). The partners used are lane^1, lane^2 (quad permutes), lane^7
// (row half-mirror) and lane^15 (row mirror); W >= 16 uses lane^W.
template <int W>
__device__ __forceinline__ int partner_i32(int v) {
  if constexpr (W == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  else if constexpr (W == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  else if constexpr (W == 4) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  else if constexpr (W == 8) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  else return __shfl_xor(v, W, kWave);
}

template <int W, typename T>
__device__ __forceinline__ T partner(T v) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, partner_i32<W>(__builtin_bit_cast(int, v)));
  } else {
    int2 p = __builtin_bit_cast(int2, v);
    p.x = partner_i32<W>(p.x);
    p.y = partner_i32<W>(p.y);
    return __builtin_bit_cast(T, p);
  }
}

// Value of v on lane `src` (uniform), for 4- and 8-byte types.
template <typename T>
__device__ __forceinline__ T lane_value(T v, int src) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
  } else {
    int2 p = __builtin_bit_cast(int2, v);
    p.x = __builtin_amdgcn_readlane(p.x, src);
    p.y = __builtin_amdgcn_readlane(p.y, src);
    return __builtin_bit_cast(T, p);
  }
}

// Sum over the 64 lanes, the same value in every lane, with no LDS traffic:
// DPP lane swaps add up each row of 16 lanes, then the four row sums are
// read from lanes 0, 16, 32, 48 and added in a fixed order.
template <typename T>
__device__ __forceinline__ T wave_allsum(T v) {
  v += partner<1>(v);
  v += partner<2>(v);
  v += partner<4>(v);
  v += partner<8>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// op over the 64 lanes (every lane active), the same value in every lane:
// DPP lane swaps within each row of 16, then the four row results.
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
  v = op(v, partner<1>(v));
  v = op(v, partner<2>(v));
  v = op(v, partner<4>(v));
  v = op(v, partner<8>(v));
  return op(op(lane_value(v, 0), lane_value(v, 16)), op(lane_value(v, 32), lane_value(v, 48)));
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_allreduce(v, [](T a, T b) { return a + b; });
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_allreduce(v, [](T a, T b) { return max(a, b); });
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_allreduce(v, [](T a, T b) { return min(a, b); });
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

// Exclusive block prefix sums of two ints per thread at once (one barrier
// pair). `tmp` holds at least 2 * NT/64 ints of LDS. Every thread of the
// block must call it.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(int a, int b, int* tmp, int* ea, int* eb) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  constexpr int NW = NT / kWave;
  const int ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
  if (lane == kWave - 1) {
    tmp[2 * wid] = ia;
    tmp[2 * wid + 1] = ib;
  }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    ba += (w < wid) ? tmp[2 * w] : 0;
    bb += (w < wid) ? tmp[2 * w + 1] : 0;
  }
  __syncthreads();
  *ea = ba + ia - a;
  *eb = bb + ib - b;
}

template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* tmp, Op op) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  constexpr int NW = NT / kWave;
  v = wave_allreduce(v, op);
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
// NV/2 + NV/4 + ... exchanges instead of NV*log2(LT). The step for bit W
// pairs each lane with a partner that differs from it in bit W (partner<W>);
// the partner masks of the steps (lane^15, ^7, ^2, ^1 or lane^W) span all
// log2(LT) lane bits, so every lane of a group ends with the full sum.
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
          v[i] = keep + partner<W>(send);
        }
        step<T, W / 2, H>(v, lane);
      } else {
        v[0] += partner<W>(v[0]);
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

// Lanes below `lane` as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int clamp_len(int L, int max_tokens) {
  return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

}  // namespace ekv
