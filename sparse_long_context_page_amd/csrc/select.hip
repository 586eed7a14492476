// Page bounds and fixed-budget top-k page selection.
// EntmaxKV summary page (gist.science paper 2605.21649): section 2.A (the
// box metadata gives a deterministic upper bound on a page's best q.k) and
// section 2.B policy 1 (keep the k pages with the highest bounds).
//
// bounds_mfma_kernel (bf16 boxes): the bound as a dot product on the matrix
//   cores (described at the kernel); float32 sums of exact products, so a
//   bound can differ from the exactly rounded one by float32 accumulation
//   error (far inside the 1e-5 near-tie band of the selection).
// bounds_kernel (float32 boxes): one workgroup per (chunk of pages,
//   sequence, KV head). The G query heads that share the KV head are bounded
//   together, so each page's box is read once. Each page's (k_min, k_max) row
//   pair is split over D/4 lanes (four coordinates of each per lane); a
//   workgroup covers 32 pages and issues all of its box loads before using
//   the first. Per coordinate the lane takes k_max where q_d >= 0 and k_min
//   otherwise (the box maximum of q_d k_d), forms the products in float64
//   (exact: 24-bit x 24-bit significands) and sums in float64; a multi-value
//   butterfly finishes the G sums across the LP lanes. Result rounded once
//   to float32 (+0 for a zero).
// select_kernel: one workgroup per (sequence, query head). Radix select on
//   the order-preserving 32-bit image of the float32 bound, starting at the
//   highest bit where the bounds differ (so the first histogram is spread),
//   8 bits per pass, stopping as soon as the boundary digit is taken whole.
//   Ties on the full 32 bits go to the lower page index. The kept pages are
//   written in ascending order with two block scans.
#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"

namespace ekv {

// Threads of the select kernel: 512 when there are few heads (fewer keys
// per thread shorten each pass), 256 from kSelWideFrom heads on (the grid
// then fills the chip and smaller workgroups pack better).
constexpr int kSelWideFrom = 256;
constexpr int kSelLds = 16384;  // bounds staged in LDS when the sequence has at most this many pages
constexpr int kBoundPages = 32;  // pages per workgroup of the bounds kernel

template <typename KV, int D, int G>
__global__ void __launch_bounds__(256)
bounds_kernel(const float* __restrict__ q, const KV* __restrict__ meta,
              const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
              float* __restrict__ ub, int H, int Hkv, int ps, int max_pages, int num_phys, int U,
              int ldu) {
  constexpr int VPC = 4;                  // box coordinates per lane (per bound side)
  constexpr int LP = D / VPC;             // lanes per page
  constexpr int PPB = 256 / LP;           // pages per block step
  constexpr int STEPS = kBoundPages / PPB;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  using Chunk = typename std::conditional<sizeof(KV) == 2, u32x2, u32x4>::type;
  using BF = Butterfly<G, LP>;
  static_assert(BF::CNT == 1, "group size must not exceed lanes per page");
  static_assert(kBoundPages % PPB == 0, "whole block steps");
  __shared__ int sphys[kBoundPages];

  const int u = blockIdx.x % U;
  const int chunk = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int j0 = chunk * kBoundPages;
  // the chunk's block-table entries are read together with the length (not
  // after it); entries past the sequence are dropped below
  const int jt = j0 + (int)threadIdx.x;
  const int bt_entry = threadIdx.x < kBoundPages && jt < max_pages
                           ? block_table[(size_t)b * max_pages + jt] : -1;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  if (j0 >= P) return;
  const int n = min(kBoundPages, P - j0);

  // physical pages of the chunk, in LDS
  if (threadIdx.x < kBoundPages) sphys[threadIdx.x] = (int)threadIdx.x < n ? bt_entry : -1;

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

  // every box load of the workgroup is in flight before the first is used;
  // boxes are read once per call, so the loads are marked streaming
  Chunk xlo[STEPS], xhi[STEPS];
  bool ok[STEPS];
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    const int phys = sphys[t * PPB + threadIdx.x / LP];
    ok[t] = phys >= 0 && phys < num_phys;
    // page 0 stands in for an empty slot; its result is dropped
    const KV* row = meta + ((size_t)(ok[t] ? phys : 0) * Hkv + g) * 2 * D + c * VPC;
    xlo[t] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(row));
    xhi[t] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(row + D));
  }
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    float lo[VPC], hi[VPC];
    if constexpr (sizeof(KV) == 2) {
      lo[0] = bf16_lo(xlo[t].x); lo[1] = bf16_hi(xlo[t].x);
      lo[2] = bf16_lo(xlo[t].y); lo[3] = bf16_hi(xlo[t].y);
      hi[0] = bf16_lo(xhi[t].x); hi[1] = bf16_hi(xhi[t].x);
      hi[2] = bf16_lo(xhi[t].y); hi[3] = bf16_hi(xhi[t].y);
    } else {
      lo[0] = __uint_as_float(xlo[t].x); lo[1] = __uint_as_float(xlo[t].y);
      lo[2] = __uint_as_float(xlo[t].z); lo[3] = __uint_as_float(xlo[t].w);
      hi[0] = __uint_as_float(xhi[t].x); hi[1] = __uint_as_float(xhi[t].y);
      hi[2] = __uint_as_float(xhi[t].z); hi[3] = __uint_as_float(xhi[t].w);
    }
    double acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < VPC; ++e) {
        const float k = qf[h][e] >= 0.0f ? hi[e] : lo[e];
        a = fma((double)qf[h][e], (double)k, a);
      }
      acc[h] = a;
    }
    BF::reduce(acc, lane);
    const int jj = t * PPB + threadIdx.x / LP;
    if (ok[t] && owner) ub[(size_t)(h0 + my_head) * ldu + j0 + jj] = (float)acc[0] + 0.0f;
  }
}

// Matrix-core bounds for bf16 boxes. Coordinate-wise,
// max(q_d kmin_d, q_d kmax_d) = min(q_d, 0) kmin_d + max(q_d, 0) kmax_d, and a
// box record is [kmin | kmax] (2D values), so a page's bound is the dot
// product of c = [min(q, 0) | max(q, 0)] with its record: bounds of 16 pages
// x 4 heads are a chain of v_mfma_f32_16x16x32_bf16 over the 2D record
// values, the same operand scheme as the score kernel (c split exactly into
// three bf16 parts, one (head, part) per A row; records as B columns, so
// every product is exact and the sums are float32). Each wave streams tiles
// of 16 records into two LDS buffers with direct-to-LDS 16-byte loads (one
// instruction reads 1 KiB: two or four whole records, chunk c of record r
// stored at slot c ^ (r & 15) so the operand reads hit distinct banks) and
// scores one tile while the next is in flight. A workgroup covers
// 64 * nt pages of one (sequence, KV head), the physical ids staged in LDS.
//
// Workgroups of the matrix-core bounds kernel: about 256 in all (one per CU,
// a single round; on the 32K-512K workloads this beat 512-4096 shorter ones),
// each wave taking `nt` tiles of 16 pages.
constexpr long long kBoundsGrid = 256;
constexpr int kBoundsMaxTiles = 16;
constexpr int kBoundsBufs = 2;  // tile buffers per wave

// LDS of the matrix-core bounds kernel: kBoundsBufs 16-record tiles per wave, the
// chunk's physical page ids, then the split q table.
__host__ __device__ constexpr size_t bounds_lds_bytes(int D, int G, int cp) {
  return (size_t)kNW * kBoundsBufs * 16 * 4 * D + (size_t)cp * 4 + (size_t)G * 3 * (2 * D + 8) * 2;
}

template <int D, int G>
__global__ void __launch_bounds__(256)
bounds_mfma_kernel(const float* __restrict__ q, const bf16_t* __restrict__ meta,
                   const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                   float* __restrict__ ub, int H, int Hkv, int ps, int max_pages, int num_phys,
                   int U, int ldu, int nt) {
  constexpr int K2 = 2 * D;        // values per record
  constexpr int RB = K2 * 2;       // bytes per record
  constexpr int TP = 16;           // records (pages) per tile
  constexpr int PB = TP * RB;      // bytes per tile
  constexpr int NI = PB / 1024;    // 1 KiB load instructions per tile
  constexpr int RPI = 1024 / RB;   // records per load instruction
  constexpr int CPR = RB / 16;     // 16-byte chunks per record
  constexpr int KS = K2 / 32;      // k-steps of 32 values
  constexpr int NMB = (G + 3) / 4; // blocks of 4 heads
  static_assert(NI * 1024 == PB && RPI * RB == 1024 && D % 32 == 0, "tiling");
  extern __shared__ __align__(16) unsigned char smem[];
  int* sphys = reinterpret_cast<int*>(smem + kNW * kBoundsBufs * PB);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int u = blockIdx.x % U, chunk = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int cp = kNW * TP * nt;
  const int j0 = chunk * cp;
  // the chunk's block-table entries (up to kBoundsMaxTiles * 64, four per
  // thread) are read together with the length, not after it
  constexpr int BPT = kBoundsMaxTiles * kNW * TP / 256;
  int bt_entry[BPT];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int i = k * 256 + tid;
    bt_entry[k] = i < cp && j0 + i < max_pages ? block_table[(size_t)b * max_pages + j0 + i] : -1;
  }
  // and so are this thread's q values of the group
  const int h0 = b * H + g * G;
  constexpr int QPT = (G * D + 255) / 256;
  float qx[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = k * 256 + tid;
    qx[k] = i < G * D ? q[(size_t)h0 * D + i] : 0.0f;
  }
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  if (j0 >= P) return;
  const int n = min(cp, P - j0);
  const int ntl = (n + TP - 1) / TP;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int i = k * 256 + tid;
    if (i < ntl * TP) sphys[i] = i < n ? bt_entry[k] : -1;
  }

  const int kgrp = lane >> 4, col = lane & 15;
  // c = [min(q, 0) | max(q, 0)] of the group's heads, split exactly into
  // three bf16 parts, staged in LDS as rows (head, part) of 2D values (rows
  // padded by 16 bytes against bank conflicts): each thread splits two or
  // more q values, each lane then reads its A fragments with 16-byte loads.
  bf16x8 qa[NMB][KS];
  constexpr int QP = K2 + 8;  // row pitch in bf16 values
  uint16_t* qtab = reinterpret_cast<uint16_t*>(smem + kNW * kBoundsBufs * PB + (size_t)cp * 4);
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = k * 256 + tid;
    if (i >= G * D) break;
    const int h = i / D, d = i % D;
    const float x = qx[k];
    const uint32_t p0 = bf16_rne_bits(x);
    const float r1 = x - __uint_as_float(p0 << 16);
    const uint32_t p1 = bf16_rne_bits(r1);
    const uint32_t p2 = bf16_rne_bits(r1 - __uint_as_float(p1 << 16));
    const uint32_t pp[3] = {p0, p1, p2};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      uint16_t* row = qtab + (size_t)(h * 3 + part) * QP;
      row[d] = x < 0.0f ? (uint16_t)pp[part] : (uint16_t)0;
      row[D + d] = x > 0.0f ? (uint16_t)pp[part] : (uint16_t)0;
    }
  }
  // Source byte offset, within a record, of the chunk this lane stores in
  // load instruction i (record i * RPI + lane / CPR of the tile).
  int src_off[NI], rec_of[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = i * RPI + lane / CPR;
    rec_of[i] = r;
    src_off[i] = (((lane % CPR) ^ (r & 15)) * 16);
  }
  __syncthreads();

  unsigned char* kbuf = smem + (size_t)wave * kBoundsBufs * PB;
  // Tile t into buffer bsel; records past the chunk, or with an invalid
  // physical id, read page 0's record (its bound is not stored). Loads are
  // issued on every path so that the waits count them exactly.
  auto issue = [&](int t, int bsel) {
    unsigned char* dst = kbuf + bsel * PB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int p = t * TP + rec_of[i];
      const int ph = p < ntl * TP ? sphys[p] : -1;
      const bool ok = ph >= 0 && ph < num_phys;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(
          meta + ((size_t)(ok ? ph : 0) * Hkv + g) * K2);
      lds_load16(src + src_off[i], dst + i * 1024);
    }
  };
  auto bound_tile = [&](int t, int bsel) {
    const unsigned char* src = kbuf + bsel * PB;
    bf16x8 kv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kv[ks] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(
                      src + col * RB + (((ks * 4 + kgrp) ^ (col & 15)) * 16)));
    const int p = t * TP + col;
    const int ph = sphys[p];
    const bool ok = ph >= 0 && ph < num_phys;
#pragma unroll
    for (int blk = 0; blk < NMB; ++blk) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[blk][ks], kv[ks], acc, 0, 0, 0);
      const int h = blk * 4 + kgrp;
      if (h < G && p < n)
        ub[(size_t)(h0 + h) * ldu + j0 + p] =
            ok ? ((acc[0] + acc[1]) + acc[2]) + 0.0f : -__builtin_inff();
    }
  };
  // A operand, read before any load into LDS is in flight: lane l holds row
  // l % 16 = (head, part) and record values ks * 32 + (l / 16) * 8 .. +8 of
  // c; rows past the group are zero.
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

  // kBoundsBufs buffers form a ring, each refilled as soon as its tile is
  // bounded: before a buffer is read only the other buffers' loads may be
  // outstanding.
#pragma unroll
  for (int k = 0; k < kBoundsBufs; ++k) issue(wave + k * kNW, k);
  for (int t = wave, k = 0; t < ntl; t += kNW) {
    wait_vmcnt<(kBoundsBufs - 1) * NI>();
    bound_tile(t, k);
    issue(t + kBoundsBufs * kNW, k);
    k = k + 1 == kBoundsBufs ? 0 : k + 1;
  }
  wait_vmcnt<0>();  // no load into LDS is left in flight
}

// --------------------------------------------------------------------------

// kDrop: keys at or below the order value of -inf are not candidates (the
// Gaussian selection marks the pages that fail its rule that way); when no
// more than `budget` candidates remain all are kept and the row is -1 padded.
template <int kSelNT, bool kDrop>
__global__ void __launch_bounds__(kSelNT)
select_kernel(const float* __restrict__ ub, const int32_t* __restrict__ seq_lens, int H, int G,
              int Hkv, int U, int ps, int max_pages, int ldu, int budget,
              int32_t* __restrict__ sel, float* __restrict__ sel_ub) {
  constexpr uint32_t drop_below = 0x007fffffu;  // float_order(-inf)
  constexpr int NW = kSelNT / kWave;
  constexpr int UNR = 4;  // 16-byte loads in flight per thread
  __shared__ __align__(16) uint32_t sord[kSelLds];
  __shared__ __align__(16) int hist[2][256];
  __shared__ unsigned int ured[NW][2];
  __shared__ int wcnt[NW][2];
  __shared__ int vcnt[NW];
  __shared__ int bc[3];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int u = blockIdx.x % U, hh = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int bh = b * H + g * G + hh;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  const float* row = ub + (size_t)bh * ldu;
  int32_t* out = sel + (size_t)bh * budget;
  float* out_ub = sel_ub ? sel_ub + (size_t)bh * budget : nullptr;

  if (!kDrop && P <= budget) {
    for (int i = tid; i < budget; i += kSelNT) {
      out[i] = i < P ? i : -1;
      if (out_ub) out_ub[i] = i < P ? row[i] + 0.0f : -__builtin_inff();
    }
    return;
  }

  // Order-preserving 32-bit keys, handled four at a time (rows are padded to
  // a multiple of 4 floats; a quad's entries at or past P are masked). They
  // are staged in LDS when they fit, else re-read from the bounds row.
  const bool staged = P <= kSelLds;
  const int n4 = (P + 3) >> 2;
  const float4* row4 = reinterpret_cast<const float4*>(row);
  auto from_global = [&](int i4) -> uint4 {
    const float4 f = row4[i4];
    return make_uint4(float_order(f.x + 0.0f), float_order(f.y + 0.0f), float_order(f.z + 0.0f),
                      float_order(f.w + 0.0f));
  };
  auto quad = [&](int i4) -> uint4 {
    return staged ? *reinterpret_cast<const uint4*>(&sord[4 * i4]) : from_global(i4);
  };
  auto at = [](const uint4& v, int e) -> uint32_t {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
  };

  // A key counts when its page is below P (and, with kDrop, it is above -inf).
  auto valid = [&](int j, uint32_t o) { return j < P && (!kDrop || o > drop_below); };
  uint32_t mn = 0xffffffffu, mx = 0u;
  int nvalid = 0;
  for (int base = 0; base < n4; base += UNR * kSelNT) {
    uint4 v[UNR] = {};
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int i4 = base + r * kSelNT + tid;
      if (i4 < n4) v[r] = from_global(i4);
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int i4 = base + r * kSelNT + tid;
      if (i4 < n4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (valid(4 * i4 + e, at(v[r], e))) {
            mn = min(mn, at(v[r], e));
            mx = max(mx, at(v[r], e));
            if constexpr (kDrop) ++nvalid;
          }
        }
        if (staged) *reinterpret_cast<uint4*>(&sord[4 * i4]) = v[r];
      }
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if constexpr (kDrop) nvalid = wave_sum(nvalid);
  if (lane == 0) {
    ured[wave][0] = mn;
    ured[wave][1] = mx;
    if constexpr (kDrop) vcnt[wave] = nvalid;
  }
  if (tid < 256) hist[0][tid] = 0;
  __syncthreads();
  nvalid = kDrop ? 0 : P;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, ured[w][0]);
    mx = max(mx, ured[w][1]);
    if constexpr (kDrop) nvalid += vcnt[w];
  }

  // Radix select of the budget-th largest key, 8 bits per pass from the
  // highest bit where keys differ; stop once the boundary digit is taken
  // whole. Two histograms alternate so that a pass needs two barriers.
  uint32_t prefix, pmask;
  int k = budget;  // rank still to place among keys matching the prefix
  if (kDrop && nvalid <= budget) {
    // every counted key is kept: all of them "equal" an empty prefix
    prefix = 0u;
    pmask = 0u;
    k = nvalid;
    for (int i = nvalid + tid; i < budget; i += kSelNT) {
      out[i] = -1;
      if (out_ub) out_ub[i] = -__builtin_inff();
    }
  } else if (mn == mx) {
    prefix = mx;
    pmask = 0xffffffffu;
  } else {
    int hb = 31 - __clz(mn ^ mx);
    pmask = ~((2u << hb) - 1u);
    prefix = mx & pmask;
    int cur = 0;
    while (true) {
      const int lo = hb >= 7 ? hb - 7 : 0;
      const int width = hb - lo + 1;
      const uint32_t dmask = (1u << width) - 1u;
      if (tid < 256) hist[cur ^ 1][tid] = 0;
      for (int base = 0; base < n4; base += UNR * kSelNT) {
        uint4 v[UNR] = {};
#pragma unroll
        for (int r = 0; r < UNR; ++r) {
          const int i4 = base + r * kSelNT + tid;
          if (i4 < n4) v[r] = quad(i4);
        }
#pragma unroll
        for (int r = 0; r < UNR; ++r) {
          const int i4 = base + r * kSelNT + tid;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t o = at(v[r], e);
            if (i4 < n4 && valid(4 * i4 + e, o) && (o & pmask) == prefix)
              atomicAdd(&hist[cur][(o >> lo) & dmask], 1);
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        int c4[4];
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c4[i] = hist[cur][4 * lane + i];
          s += c4[i];
        }
        // keys in this lane's bins and above: the total less the keys in
        // lower lanes' bins
        const int incl = wave_incl_scan(s, lane);
        const int suf = lane_value(incl, kWave - 1) - incl + s;
        int above = suf - s;
        if (above < k && k <= suf) {
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if (above < k && k <= above + c4[i]) {
              bc[0] = 4 * lane + i;
              bc[1] = above;
              bc[2] = c4[i];
            }
            above += c4[i];
          }
        }
      }
      __syncthreads();
      const int d = bc[0];
      const int cnt_d = bc[2];
      k -= bc[1];
      prefix |= ((uint32_t)d) << lo;
      pmask |= dmask << lo;
      if (cnt_d == k || lo == 0) break;
      hb = lo - 1;
      cur ^= 1;
    }
  }

  // Keep keys above the prefix and the first k (by page index) equal to it,
  // written in ascending page order: thread t owns a contiguous run of quads,
  // one block scan of the runs' (above, equal) counts places each run, and
  // the thread writes its kept pages in order.
  const int qpt = (n4 + kSelNT - 1) / kSelNT;
  const int q0 = min(n4, tid * qpt), q1 = min(n4, q0 + qpt);
  int n_gt = 0, n_eq = 0;
  for (int i4 = q0; i4 < q1; ++i4) {
    const uint4 v = quad(i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = valid(4 * i4 + e, at(v, e));
      const uint32_t m = at(v, e) & pmask;
      n_eq += (ok && m == prefix) ? 1 : 0;
      n_gt += (ok && m > prefix) ? 1 : 0;
    }
  }
  int gt_base, eq_base;
  block_excl_scan2<kSelNT>(n_gt, n_eq, &wcnt[0][0], &gt_base, &eq_base);
  int pos = gt_base + min(eq_base, k);
  int eqc = eq_base;  // equal keys on lower pages
  for (int i4 = q0; i4 < q1 && pos < budget; ++i4) {
    const uint4 v = quad(i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = valid(4 * i4 + e, at(v, e));
      const uint32_t m = at(v, e) & pmask;
      const bool eq = ok && m == prefix;
      const bool take = (ok && m > prefix) || (eq && eqc < k);
      eqc += eq ? 1 : 0;
      if (take) {
        if (pos < budget) {
          out[pos] = 4 * i4 + e;
          if (out_ub) out_ub[pos] = order_float(at(v, e));
        }
        ++pos;
      }
    }
  }
}

template <int D, int G>
static hipError_t launch_bounds_mfma(const LaunchShape& s, const float* q, const void* meta,
                                     const int32_t* bt, const int32_t* lens, float* ub,
                                     hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  const long long tiles = (long long)U * ((s.max_pages + 15) / 16);
  long long nt = (tiles + kBoundsGrid * kNW - 1) / (kBoundsGrid * kNW);
  nt = nt < 1 ? 1 : (nt > kBoundsMaxTiles ? kBoundsMaxTiles : nt);
  const int cp = kNW * 16 * (int)nt;
  const long long chunks = (s.max_pages + cp - 1) / cp;
  const size_t lds = bounds_lds_bytes(D, G, cp);
  auto kern = bounds_mfma_kernel<D, G>;
  // The LDS limit is a kernel attribute: raised once, to the most any plan
  // asks for (a function-local static is initialised exactly once, also when
  // several host threads launch).
  static const hipError_t lds_raised = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)bounds_lds_bytes(D, 8, kNW * 16 * kBoundsMaxTiles));
  if (lds_raised != hipSuccess) return lds_raised;
  hipLaunchKernelGGL(kern, dim3((unsigned)(U * chunks)), dim3(256), lds, st, q,
                     static_cast<const bf16_t*>(meta), bt, lens, ub, s.num_q_heads,
                     s.num_kv_heads, s.page_size, s.max_pages, s.num_phys, U,
                     ub_ld(s.max_pages), (int)nt);
  return hipGetLastError();
}

template <typename KV, int D, int G>
static hipError_t launch_bounds_t(const LaunchShape& s, const float* q, const void* meta,
                                  const int32_t* bt, const int32_t* lens, float* ub,
                                  hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  const int chunks = (s.max_pages + kBoundPages - 1) / kBoundPages;
  hipLaunchKernelGGL((bounds_kernel<KV, D, G>), dim3(U * chunks), dim3(256), 0, st, q,
                     static_cast<const KV*>(meta), bt, lens, ub, s.num_q_heads, s.num_kv_heads,
                     s.page_size, s.max_pages, s.num_phys, U, ub_ld(s.max_pages));
  return hipGetLastError();
}

template <typename KV, int D>
static hipError_t launch_bounds_d(const LaunchShape& s, const float* q, const void* meta,
                                  const int32_t* bt, const int32_t* lens, float* ub,
                                  hipStream_t st) {
  if constexpr (sizeof(KV) == 2) {
    switch (s.group) {
      case 1: return launch_bounds_mfma<D, 1>(s, q, meta, bt, lens, ub, st);
      case 2: return launch_bounds_mfma<D, 2>(s, q, meta, bt, lens, ub, st);
      case 4: return launch_bounds_mfma<D, 4>(s, q, meta, bt, lens, ub, st);
      default: return launch_bounds_mfma<D, 8>(s, q, meta, bt, lens, ub, st);
    }
  } else {
    switch (s.group) {
      case 1: return launch_bounds_t<KV, D, 1>(s, q, meta, bt, lens, ub, st);
      case 2: return launch_bounds_t<KV, D, 2>(s, q, meta, bt, lens, ub, st);
      case 4: return launch_bounds_t<KV, D, 4>(s, q, meta, bt, lens, ub, st);
      default: return launch_bounds_t<KV, D, 8>(s, q, meta, bt, lens, ub, st);
    }
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
                         int32_t* sel, float* sel_ub, bool drop_neg_inf, hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  const bool wide = U * s.group >= kSelWideFrom;
  const dim3 grid(U * s.group), block(wide ? 256 : 512);
  auto kern = wide ? (drop_neg_inf ? select_kernel<256, true> : select_kernel<256, false>)
                   : (drop_neg_inf ? select_kernel<512, true> : select_kernel<512, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, st, ub, lens, s.num_q_heads, s.group, s.num_kv_heads,
                     U, s.page_size, s.max_pages, ub_ld(s.max_pages), budget, sel, sel_ub);
  return hipGetLastError();
}

size_t select_ws_bytes(const LaunchShape& s) {
  return (size_t)s.batch * s.num_q_heads * ub_ld(s.max_pages) * sizeof(float);
}

}  // namespace ekv
