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
// Chunked selection (bf16 boxes, budget at most half a bounds chunk): each
//   bounds workgroup keeps, per head, the top min(budget, chunk) pages of its
//   chunk (a wave-level radix select on the same keys, ties to the lower
//   page) and writes them in page order in place of its bound rows; the
//   select kernel then takes the budget largest of those candidates. The
//   result is the same selection: every page of the global top-k is in its
//   chunk's top-k, and the candidates stay in ascending page order, so ties
//   still go to the lower page.
#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"
#include "select_impl.hpp"

namespace ekv {

// Threads of the select kernel: 512 when there are few heads (fewer keys
// per thread shorten each pass), 256 from kSelWideFrom heads on (the grid
// then fills the chip and smaller workgroups pack better).
constexpr int kSelWideFrom = 256;
constexpr int kBoundPages = 32;  // pages per workgroup of the bounds kernel

// The k largest of n 32-bit keys, ties to the lower index, by one wave
// (k < n <= 64 * KPL): lane l holds keys l, l + 64, ... in kr[0..KPL). Radix
// select, 8 bits per pass from the highest bit where the keys differ, until
// the boundary digit is taken whole; the keys stay in registers. The
// histogram has kHistCopies interleaved copies (bin b, copy c at word
// b * kHistCopies + c, lane l adding to copy l % kHistCopies), so keys that
// share a digit, common in the first pass, spread their LDS atomics over
// that many banks. hist: 256 * kHistCopies ints of LDS owned by the wave.
// On return key i is kept iff (key & pmask) > prefix, or it equals prefix
// and fewer than keq equal keys precede it.
constexpr int kHistCopies = 4;
template <int KPL>
__device__ void wave_topk(const uint32_t (&kr)[KPL], int n, int k, int* hist, int lane,
                          uint32_t& prefix, uint32_t& pmask, int& keq) {
  static_assert(kHistCopies == 4, "one 16-byte access per bin");
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    if (r * kWave + lane < n) {
      mn = min(mn, kr[r]);
      mx = max(mx, kr[r]);
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (mn == mx) {
    prefix = mx;
    pmask = 0xffffffffu;
    keq = k;
    return;
  }
  int hb = 31 - __clz(mn ^ mx);
  pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  prefix = mx & pmask;
  int kk = k;
  uint4* mine = reinterpret_cast<uint4*>(hist) + 4 * lane;  // bins 4 lane .. 4 lane + 3
  int* slot = hist + (lane & (kHistCopies - 1));
  for (int pass = 0; pass < 8; ++pass) {
    const int lo = hb >= 7 ? hb - 7 : 0;
    const uint32_t dmask = (1u << (hb - lo + 1)) - 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[i] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const uint32_t o = kr[r];
      if (r * kWave + lane < n && (o & pmask) == prefix)
        atomicAdd(slot + ((o >> lo) & dmask) * kHistCopies, 1);
    }
    __builtin_amdgcn_wave_barrier();
    int c4[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = mine[i];
      c4[i] = (int)(v.x + v.y + v.z + v.w);
      sum += c4[i];
    }
    const int incl = wave_incl_scan(sum, lane);
    int above = lane_value(incl, kWave - 1) - incl;  // keys in higher lanes' bins
    int d = -1, ab = 0, cd = 0;
    if (above < kk && kk <= above + sum) {
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < kk && kk <= above + c4[i]) {
          d = 4 * lane + i;
          ab = above;
          cd = c4[i];
        }
        above += c4[i];
      }
    }
    const uint64_t bal = __ballot(d >= 0);
    __builtin_amdgcn_wave_barrier();
    if (bal == 0ull) break;  // (cannot happen: kk <= keys matching the prefix)
    const int src = __ffsll((unsigned long long)bal) - 1;
    d = __builtin_amdgcn_readlane(d, src);
    ab = __builtin_amdgcn_readlane(ab, src);
    cd = __builtin_amdgcn_readlane(cd, src);
    kk -= ab;
    prefix |= ((uint32_t)d) << lo;
    pmask |= dmask << lo;
    if (cd == kk || lo == 0) break;
    hb = lo - 1;
  }
  keq = kk;
}

// Calls emit(i, key, pos) for every kept key i (held as in wave_topk) in
// ascending i, pos = its rank among the kept. One wave.
template <int KPL, typename Emit>
__device__ void wave_emit_kept(const uint32_t (&kr)[KPL], int n, uint32_t prefix, uint32_t pmask,
                               int keq, int lane, Emit emit) {
  const uint64_t ltm = lanemask_below(lane);
  int eq_before = 0, pos0 = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    if (r * kWave >= n) break;
    const int i = r * kWave + lane;
    const uint32_t m = kr[r] & pmask;
    const bool gt = i < n && m > prefix;
    const bool eq = i < n && m == prefix;
    const uint64_t beq = __ballot(eq);
    const bool take = gt || (eq && eq_before + __popcll(beq & ltm) < keq);
    const uint64_t btk = __ballot(take);
    if (take) emit(i, kr[r], pos0 + __popcll(btk & ltm));
    eq_before += __popcll(beq);
    pos0 += __popcll(btk);
  }
}

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
    // a page whose block-table entry is out of range gets -inf (never kept
    // ahead of a valid page), so no bound of the row is left unwritten
    if (jj < n && owner)
      ub[(size_t)(h0 + my_head) * ldu + j0 + jj] = ok[t] ? (float)acc[0] + 0.0f : -__builtin_inff();
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
constexpr long long kBoundsGrid = kNumCUs;
constexpr int kBoundsMaxTiles = 16;
constexpr int kBoundsBufs = 2;  // tile buffers per wave

// LDS of the matrix-core bounds kernel: kBoundsBufs 16-record tiles per wave, the
// chunk's physical page ids, then the split q table; chunked (LOCAL) runs
// add the chunk's bounds [G][cp].
__host__ __device__ constexpr size_t bounds_lds_bytes(int D, int G, int cp, bool local = false) {
  return (size_t)kNW * kBoundsBufs * 16 * 4 * D + (size_t)cp * 4 + (size_t)G * 3 * (2 * D + 8) * 2 +
         (local ? (size_t)G * cp * 4 : 0);
}

// LOCAL: instead of the bound rows, each head's top keepc pages of the chunk
// go to cand[(head * nchunks + chunk) * keepc + ...] as (order key | page << 32).
template <int D, int G, bool LOCAL>
__global__ void __launch_bounds__(256)
bounds_mfma_kernel(const float* __restrict__ q, const bf16_t* __restrict__ meta,
                   const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                   float* __restrict__ ub, int H, int Hkv, int ps, int max_pages, int num_phys,
                   int U, int ldu, int nt, int keepc, int nchunks) {
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
  static_assert(!LOCAL || kBoundsBufs * PB >= 256 * kHistCopies * 4, "histogram fits a wave's tiles");
  extern __shared__ __align__(16) unsigned char smem[];
  int* sphys = reinterpret_cast<int*>(smem + kNW * kBoundsBufs * PB);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int u = blockIdx.x % U, chunk = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int cp = kNW * TP * nt;
  // LOCAL: the chunk's bounds, past the split q table
  float* lub = reinterpret_cast<float*>(smem + kNW * kBoundsBufs * PB + (size_t)cp * 4 +
                                        (size_t)G * 3 * (K2 + 8) * 2);
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
      const float bound = ok ? ((acc[0] + acc[1]) + acc[2]) + 0.0f : -__builtin_inff();
      if (h < G && p < n) {
        if constexpr (LOCAL) lub[h * cp + p] = bound;
        else ub[(size_t)(h0 + h) * ldu + j0 + p] = bound;
      }
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
  if constexpr (LOCAL) {
    // each head's top keepc pages of the chunk, in page order
    __syncthreads();
    constexpr int KPL = kNW * 16 * kBoundsMaxTiles / kWave;  // keys per lane, cp <= 64 KPL
    for (int h = wave; h < G; h += kNW) {
      const float* row = lub + h * cp;
      uint32_t kr[KPL];
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const int i = r * kWave + lane;
        kr[r] = i < n ? float_order(row[i]) : 0u;
      }
      uint32_t prefix = 0u, pmask = 0u;
      int keq = n;
      // the histogram lives in the wave's own tile buffers, idle now
      if (n > keepc)
        wave_topk<KPL>(kr, n, keepc, reinterpret_cast<int*>(kbuf), lane, prefix, pmask, keq);
      uint64_t* dst = reinterpret_cast<uint64_t*>(ub) + ((size_t)(h0 + h) * nchunks + chunk) * keepc;
      wave_emit_kept<KPL>(kr, n, prefix, pmask, keq, lane, [&](int i, uint32_t key, int pos) {
        dst[pos] = (uint64_t)key | ((uint64_t)(uint32_t)(j0 + i) << 32);
      });
    }
  }
}

// --------------------------------------------------------------------------

// kCand: the keys are the chunked candidates of bounds_mfma_kernel<..., true>
// (order key | page << 32, keepc per chunk of cp pages, nchunks per head),
// at most kSelCand of them per head; the kept candidates' pages are written.
constexpr long long kSelChunkedMinPages = 8192;
template <int kSelNT, bool kCand>
__global__ void __launch_bounds__(kSelNT)
select_kernel(const float* __restrict__ ub, const int32_t* __restrict__ seq_lens, int H, int G,
              int Hkv, int U, int ps, int max_pages, int ldu, int budget,
              int32_t* __restrict__ sel, float* __restrict__ sel_ub, int cp, int keepc,
              int nchunks) {
  __shared__ __align__(16) uint32_t sord[kSelLds];
  __shared__ SelectScratch<kSelNT> sh;
  const int tid = threadIdx.x;
  const int u = blockIdx.x % U, hh = blockIdx.x / U;
  const int b = u / Hkv, g = u % Hkv;
  const int bh = b * H + g * G + hh;
  const int L = clamp_len(seq_lens[b], max_pages * ps);
  const int P = (L + ps - 1) / ps;
  int32_t* out = sel + (size_t)bh * budget;
  float* out_ub = sel_ub ? sel_ub + (size_t)bh * budget : nullptr;
  const int kept = select_row<kSelNT, false, kCand>(
      ub + (size_t)bh * ldu, reinterpret_cast<const uint64_t*>(ub) + (size_t)bh * nchunks * keepc,
      P, budget, cp, keepc, kCand ? nchunks * keepc : ldu, sord, sh,
      [&](int pos, int page, uint32_t key) {
        out[pos] = page;
        if (out_ub) out_ub[pos] = order_float(key);
      });
  for (int i = kept + tid; i < budget; i += kSelNT) {
    out[i] = -1;
    if (out_ub) out_ub[i] = -__builtin_inff();
  }
}

SelectPlan plan_select(const LaunchShape& s, int budget) {
  SelectPlan p;
  const int U = s.batch * s.num_kv_heads;
  const long long tiles = (long long)U * ((s.max_pages + 15) / 16);
  long long nt = (tiles + kBoundsGrid * kNW - 1) / (kBoundsGrid * kNW);
  nt = nt < 1 ? 1 : (nt > kBoundsMaxTiles ? kBoundsMaxTiles : nt);
  p.nt = (int)nt;
  p.cp = kNW * 16 * p.nt;
  p.nchunks = (s.max_pages + p.cp - 1) / p.cp;
  p.keepc = budget < p.cp ? budget : p.cp;
  // Chunked when it leaves at most half the keys, they fit the select's LDS
  // staging (bf16 boxes, where the bounds kernel covers cp-page chunks), and
  // the one-workgroup-per-row select would scan at least kSelChunkedMinPages
  // pages per CU: the chunk-local top-k adds about 3.5 us to the bounds kernel
  // (its tail runs with one wave per SIMD), which the shorter select repays
  // only there (measured: 32K x 256 rows and 128K x 128 rows lose 2 us,
  // 64K x 512 rows, 512K and 1M x 32 rows gain 2-8 us).
  const long long rows = (long long)s.batch * s.num_q_heads;
  const long long per_cu = (rows + kNumCUs - 1) / kNumCUs * s.max_pages;
  p.chunked = s.bf16 && budget > 0 && 2 * (long long)p.keepc <= p.cp &&
              (long long)p.nchunks * p.keepc <= kSelCand && per_cu >= kSelChunkedMinPages;
  return p;
}

template <int D, int G, bool LOCAL>
static hipError_t launch_bounds_mfma(const LaunchShape& s, const SelectPlan& p, const float* q,
                                     const void* meta, const int32_t* bt, const int32_t* lens,
                                     float* ub, hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  const size_t lds = bounds_lds_bytes(D, G, p.cp, LOCAL);
  auto kern = bounds_mfma_kernel<D, G, LOCAL>;
  // The LDS limit is a kernel attribute: raised once, to the most any plan
  // asks for (a function-local static is initialised exactly once, also when
  // several host threads launch).
  static const hipError_t lds_raised = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)bounds_lds_bytes(D, 8, kNW * 16 * kBoundsMaxTiles, LOCAL));
  if (lds_raised != hipSuccess) return lds_raised;
  hipLaunchKernelGGL(kern, dim3((unsigned)(U * p.nchunks)), dim3(256), lds, st, q,
                     static_cast<const bf16_t*>(meta), bt, lens, ub, s.num_q_heads,
                     s.num_kv_heads, s.page_size, s.max_pages, s.num_phys, U,
                     ub_ld(s.max_pages), p.nt, p.keepc, p.nchunks);
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

template <int D, int G>
static hipError_t launch_bounds_mfma_any(const LaunchShape& s, const SelectPlan& p,
                                         const float* q, const void* meta, const int32_t* bt,
                                         const int32_t* lens, float* ub, hipStream_t st) {
  return p.chunked ? launch_bounds_mfma<D, G, true>(s, p, q, meta, bt, lens, ub, st)
                   : launch_bounds_mfma<D, G, false>(s, p, q, meta, bt, lens, ub, st);
}

template <typename KV, int D>
static hipError_t launch_bounds_d(const LaunchShape& s, const SelectPlan& p, const float* q,
                                  const void* meta, const int32_t* bt, const int32_t* lens,
                                  float* ub, hipStream_t st) {
  if constexpr (sizeof(KV) == 2) {
    switch (s.group) {
      case 1: return launch_bounds_mfma_any<D, 1>(s, p, q, meta, bt, lens, ub, st);
      case 2: return launch_bounds_mfma_any<D, 2>(s, p, q, meta, bt, lens, ub, st);
      case 4: return launch_bounds_mfma_any<D, 4>(s, p, q, meta, bt, lens, ub, st);
      default: return launch_bounds_mfma_any<D, 8>(s, p, q, meta, bt, lens, ub, st);
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

hipError_t launch_bounds(const LaunchShape& s, const SelectPlan& p, const float* q,
                         const void* meta, const int32_t* bt, const int32_t* lens, float* ub,
                         hipStream_t st) {
  if (s.bf16) {
    if (s.head_dim == 64) return launch_bounds_d<bf16_t, 64>(s, p, q, meta, bt, lens, ub, st);
    return launch_bounds_d<bf16_t, 128>(s, p, q, meta, bt, lens, ub, st);
  }
  if (s.head_dim == 64) return launch_bounds_d<float, 64>(s, p, q, meta, bt, lens, ub, st);
  return launch_bounds_d<float, 128>(s, p, q, meta, bt, lens, ub, st);
}

hipError_t launch_select(const LaunchShape& s, const SelectPlan& p, const float* ub,
                         const int32_t* lens, int budget, int32_t* sel, float* sel_ub,
                         hipStream_t st) {
  const int U = s.batch * s.num_kv_heads;
  const bool wide = U * s.group >= kSelWideFrom;
  const dim3 grid(U * s.group), block(wide ? 256 : 512);
  auto kern = wide ? (p.chunked ? select_kernel<256, true> : select_kernel<256, false>)
                   : (p.chunked ? select_kernel<512, true> : select_kernel<512, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, st, ub, lens, s.num_q_heads, s.group, s.num_kv_heads,
                     U, s.page_size, s.max_pages, ub_ld(s.max_pages), budget, sel, sel_ub, p.cp,
                     p.keepc, p.nchunks);
  return hipGetLastError();
}

size_t select_ws_bytes(const LaunchShape& s, int budget) {
  const size_t rows = (size_t)s.batch * s.num_q_heads * ub_ld(s.max_pages) * sizeof(float);
  const SelectPlan p = plan_select(s, budget);
  const size_t cand = p.chunked ? (size_t)s.batch * s.num_q_heads * p.nchunks * p.keepc * 8 : 0;
  return rows > cand ? rows : cand;
}

}  // namespace ekv
