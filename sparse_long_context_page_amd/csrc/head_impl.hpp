// Per-head select-and-decode kernel: the top-k page selection, the gather
// and score of the selected pages, the threshold and P.V of one query head
// in one workgroup.
// EntmaxKV summary page (gist.science paper 2605.21649): section 2.B policy 1
// (keep the budget pages with the highest box bounds, ties to the lower
// page), section 2.C (read only those pages' K/V and solve alpha-entmax on
// them). alpha-entmax: p_i = [(alpha-1) z_i - tau]_+^(1/(alpha-1)), sum p = 1
// (Peters, Niculae & Martins 2019).
//
// One workgroup of 512 threads per (sequence, query head), after the bounds
// kernel:
//   1. the head's block-table row is staged in LDS while the workgroup
//      radix-selects the budget largest bounds (or chunk candidates) of its
//      row (select_row); the selection goes to LDS and to `sel`;
//   2. each of the 8 waves streams its share of the selected pages (page s
//      to wave s % 8) through a ring of LDS page buffers with direct-to-LDS
//      16-byte loads, scores them on the matrix cores (the same operands and
//      order of operations as the score kernel, so every score is the same
//      float32 value) and keeps the tokens inside the window of the running
//      maximum (shared across the waves through LDS) in a per-wave list;
//   3. the lists, filtered against the workgroup's maximum (and, with many
//      candidates, a lower bound on tau from the page maxima), are gathered
//      into one window list in LDS, in (wave, page, row) order;
//   4. tau, the support and o = sum p v / sum p as in the threshold kernel
//      (tau_solve_pv), V rows read only where p > 0.
// No candidate crosses a workgroup, so the step needs no split combine and
// no launch between gather and threshold. Pages shared by the query heads
// of one KV head are read once per head (the other heads' reads are mostly
// served by the caches); the score kernel's union path remains for
// decode_sparse with a caller's selection and for shapes this kernel does
// not take (few heads, large budgets, float32 caches).
#pragma once

#include "decode_impl.hpp"
#include "select_impl.hpp"

namespace ekv {

constexpr int kHNT = 512;                  // threads of the per-head kernel
constexpr int kHNW = kHNT / kWave;         // its waves
constexpr int kHeadKbufWave = 16384;       // bytes of K page buffers per wave
constexpr int kHeadRegionA = kHNW * kHeadKbufWave;  // page buffers / select staging / window list
constexpr int kHeadSlots = 64;             // LDS candidate slots per wave
constexpr int kHeadMaxBudget = 1024;       // most pages one head's workgroup selects
constexpr int kHeadMaxBt = (kHeadRegionA - kSelLds * 4) / 4;  // block-table entries staged in LDS
constexpr int kHeadLcap = 8192;            // window-list entries held in LDS

__host__ __device__ constexpr int head_kbufs(int ps, int d) {
  return kHeadKbufWave / (ps * d * 2) < 1 ? 1 : kHeadKbufWave / (ps * d * 2);
}

// LDS of the per-head kernel (bytes): region A holds, in turn, the select's
// staged keys (and the block-table row past them), the waves' page buffers,
// then the window list and the P.V partial rows; region B the selection,
// the physical pages, the page maxima, the split q table and the per-wave
// candidate lists.
struct HeadLds {
  size_t bt, lz, li, sp, pv, sel, phys, pmax, qtab, rz, ri, total;
};
__host__ __device__ inline HeadLds head_lds_layout(int budget, int D) {
  HeadLds l;
  constexpr int NG = kHNT / 16;  // P.V rows in flight (16 lanes per bf16 V row at D = 128)
  l.bt = (size_t)kSelLds * 4;
  l.lz = 0;
  l.li = l.lz + (size_t)kHeadLcap * 4;
  l.sp = l.li + (size_t)kHeadLcap * 4;
  l.pv = l.sp + (size_t)kHeadLcap * 4;
  size_t o = kHeadRegionA;
  l.sel = o; o = align16(o + (size_t)budget * 4);
  l.phys = o; o = align16(o + (size_t)budget * 4);
  l.pmax = o; o = align16(o + (size_t)budget * 4);
  l.qtab = o; o = align16(o + (size_t)3 * qtab_pitch(D) * 2);
  l.rz = o; o = align16(o + (size_t)kHNW * kHeadSlots * 4);
  l.ri = o; o = align16(o + (size_t)kHNW * kHeadSlots * 4);
  l.total = o;
  (void)NG;
  return l;
}

struct HeadArgs {
  const float* q;
  const bf16_t* k_pool;
  const bf16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* ub;  // bounds rows [B*H, ldu], or the chunk candidates
  int32_t* sel;     // out: [B*H, budget]
  float* sel_ub;    // out (nullable)
  int H, Hkv, G, U, max_pages, num_phys, budget, ldu, cp, keepc, nchunks;
  int bt_lds;  // block_table rows may be staged with 16-byte loads
  float alpha;
  double window_d;
  Cand<float>* spill;  // per head and wave: wcap entries
  int wcap;
  float* list_z;  // per head: list_cap window members beyond the LDS list
  int* list_i;
  int list_cap;
  float* out;
  float* tau_out;
  int32_t* sup_out;
  // split form: workgroup (head, split) takes selection slots [split * pps,
  // (split + 1) * pps) and writes its candidate region (window members of
  // its own maximum; count and maximum) for the threshold kernel
  int splits, pps, rcap;
  Cand<float>* cand;
  int* counts;
  float* maxima;
};

template <int D, int PS, bool CAND, bool SPLIT>
__global__ void __launch_bounds__(kHNT)
head_decode_kernel(HeadArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SelectScratch<kHNT> ssh;
  __shared__ TauShared<kHNT> tsh;
  __shared__ float wmax[kHNW];
  __shared__ int wcnt[kHNW];
  __shared__ int woff[kHNW + 1];
  __shared__ float sbound;
  constexpr int RB = D * 2;         // bytes per K row
  constexpr int PB = PS * RB;       // bytes per page
  constexpr int NI = PB / 1024;     // 1 KiB load instructions per page
  constexpr int RPI = 1024 / RB;    // rows per load instruction
  constexpr int CPR = RB / 16;      // 16-byte chunks per row
  constexpr int KS = D / 32;        // k-steps of 32 dims
  constexpr int TILES = PS / 16;    // 16-token tiles per page
  constexpr int NBUF = head_kbufs(PS, D);
  static_assert(NI >= 1 && NI * 1024 == PB && CPR * 16 == RB, "page tiling");
  static_assert(NBUF * PB <= kHeadKbufWave, "page buffers fit the wave's share");
  static_assert(kHNT / (D / 8) * D * 4 + (size_t)kHeadLcap * 12 <= (size_t)kHeadRegionA,
                "window list and P.V rows fit region A");
  const HeadLds lay = head_lds_layout(a.budget, D);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nheads = a.U * a.G;
  const int hid = SPLIT ? (int)(blockIdx.x % nheads) : (int)blockIdx.x;
  const int split = SPLIT ? (int)(blockIdx.x / nheads) : 0;
  const int u = hid % a.U, hh = hid / a.U;
  const int b = u / a.Hkv, g = u % a.Hkv;
  const int bh = b * a.H + g * a.G + hh;
  const int budget = a.budget, max_pages = a.max_pages, num_phys = a.num_phys;
  // this thread's q value (threads below D), read first so that its latency
  // overlaps the select
  const float qv = tid < D ? a.q[(size_t)bh * D + tid] : 0.0f;
  const int L = clamp_len(a.seq_lens[b], max_pages * PS);
  const int P = (L + PS - 1) / PS;
  int32_t* sel_l = reinterpret_cast<int32_t*>(smem + lay.sel);
  int32_t* phys_l = reinterpret_cast<int32_t*>(smem + lay.phys);
  float* pmax = reinterpret_cast<float*>(smem + lay.pmax);
  const int32_t* bt_row = a.block_table + (size_t)b * max_pages;

  // 1. The block-table row into LDS past the select's keys, with
  // direct-to-LDS loads in flight during the select (issued before the
  // sequence length is known: the whole row when it fits); entries are read
  // once the select's barriers have passed.
  int32_t* bt_l = reinterpret_cast<int32_t*>(smem + lay.bt);
  const bool bt_staged = a.bt_lds && max_pages <= kHeadMaxBt;
  if (bt_staged) {
    // wave w loads 1 KiB pieces w, w + 8, ... (256 entries each); lanes past
    // the row's end re-read its last four entries (max_pages is a multiple
    // of 4, so every other lane reads whole entries of the row)
    const int npc = (max_pages + 255) / 256;
    for (int pc = wave; pc < npc; pc += kHNW) {
      const int e0 = pc * 256 + lane * 4;
      const int es = e0 + 4 <= max_pages ? e0 : max_pages - 4;
      lds_load16(bt_row + es, bt_l + pc * 256);
    }
  }
  const int n_sel = select_row<kHNT, false, CAND>(
      a.ub + (size_t)bh * a.ldu,
      reinterpret_cast<const uint64_t*>(a.ub) + (size_t)bh * a.nchunks * a.keepc, P, budget,
      a.cp, a.keepc, CAND ? a.nchunks * a.keepc : a.ldu, reinterpret_cast<uint32_t*>(smem), ssh,
      [&](int pos, int page, uint32_t key) {
        sel_l[pos] = page;
        if (split == 0) {  // (every split selects; the first writes the selection)
          a.sel[(size_t)bh * budget + pos] = page;
          if (a.sel_ub) a.sel_ub[(size_t)bh * budget + pos] = order_float(key);
        }
      });
  for (int i = n_sel + tid; i < budget && split == 0; i += kHNT) {
    a.sel[(size_t)bh * budget + i] = -1;
    if (a.sel_ub) a.sel_ub[(size_t)bh * budget + i] = -__builtin_inff();
  }
  wait_vmcnt<0>();  // the block-table pieces are in LDS
  __syncthreads();
  for (int s = tid; s < n_sel; s += kHNT) {
    const int j = sel_l[s];
    phys_l[s] = bt_staged ? bt_l[j] : bt_row[j];
  }
  // q split exactly into three bf16 parts, one LDS row per part
  constexpr int QP = qtab_pitch(D);
  uint16_t* qtab = reinterpret_cast<uint16_t*>(smem + lay.qtab);
  if (tid < D) {
    const uint32_t p0 = bf16_rne_bits(qv);
    const float r1 = qv - __uint_as_float(p0 << 16);
    const uint32_t p1 = bf16_rne_bits(r1);
    const uint32_t p2 = bf16_rne_bits(r1 - __uint_as_float(p1 << 16));
    qtab[tid] = (uint16_t)p0;
    qtab[QP + tid] = (uint16_t)p1;
    qtab[2 * QP + tid] = (uint16_t)p2;
  }
  if (tid < kHNW) wmax[tid] = -__builtin_inff();
  __syncthreads();

  // 2. Gather and score. A operand: row l % 16 = part (rows 3..15 zero) of
  // q, dims ks * 32 + (l / 16) * 8 .. + 8; lanes 0..15 end with the three
  // part sums of token l % 16 of a 16-token tile.
  const int kgrp = lane >> 4, tok = lane & 15;
  bf16x8 qa[KS];
  {
    const int part = lane & 15;
    const bool live = part < 3;
    const uint16_t* row = qtab + (size_t)(live ? part : 0) * QP + kgrp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + ks * 32);
      qa[ks] = __builtin_bit_cast(bf16x8, live ? v : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  auto swz = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & (CPR - 1)); };
  int src_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = i * RPI + lane / CPR;
    src_off[i] = r * RB + (((lane % CPR) ^ swz(r)) * 16);
  }
  unsigned char* kbuf = smem + (size_t)wave * kHeadKbufWave;
  float* rz = reinterpret_cast<float*>(smem + lay.rz) + wave * kHeadSlots;
  int* ri = reinterpret_cast<int*>(smem + lay.ri) + wave * kHeadSlots;
  Cand<float>* wspill = a.spill + (((size_t)bh * a.splits + split) * kHNW + wave) * a.wcap;
  // this workgroup's selection slots (all of them unless split)
  const int s_lo = SPLIT ? split * a.pps : 0;
  const int s_hi = SPLIT ? min(n_sel, s_lo + a.pps) : n_sel;
  const float window = (float)a.window_d;
  const uint64_t ltm = lanemask_below(lane);
  // Slot s (page sel_l[s]) into buffer k; a slot past the selection or an
  // invalid physical page reads page 0 of the pool (its scores are dropped).
  // The loads are issued on every path, so the waits count them exactly.
  auto issue = [&](int s, int k) {
    const int ph = s < s_hi ? phys_l[s] : 0;
    const bool okp = ph >= 0 && ph < num_phys;
    const unsigned char* base = reinterpret_cast<const unsigned char*>(
        a.k_pool + ((size_t)(okp ? ph : 0) * a.Hkv + g) * (size_t)PS * D);
    unsigned char* dst = kbuf + k * PB;
#pragma unroll
    for (int i = 0; i < NI; ++i) lds_load16(base + src_off[i], dst + i * 1024);
  };
  float M = -__builtin_inff();
  int cnt = 0;
  // Scores slot s from buffer k; returns the store instructions it issued
  // (spilled candidates), which the waits must allow in flight.
  auto score_page = [&](int s, int k) -> int {
    int nst = 0;
    const int j = sel_l[s];
    const int phys = phys_l[s];
    const int nvalid = (phys >= 0 && phys < num_phys) ? min(PS, L - j * PS) : 0;
    // the other waves' running maxima (plain LDS reads: some earlier value,
    // each a maximum of some of the head's scores)
    float om = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kHNW; ++w) om = max(om, wmax[w]);
    const unsigned char* src = kbuf + k * PB;
    float zz[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int row = t * 16 + tok;
      bf16x8 kv[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kv[ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(src + row * RB +
                                                    (((ks * 4 + kgrp) ^ swz(row)) * 16)));
      f32x4 cacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kv[ks], cacc, 0, 0, 0);
      zz[t] = (kgrp == 0 && row < nvalid) ? (cacc[0] + cacc[1]) + cacc[2] : -__builtin_inff();
    }
    float pm = zz[0];
#pragma unroll
    for (int t = 1; t < TILES; ++t) pm = max(pm, zz[t]);
    pm = max(pm, partner<1>(pm));
    pm = max(pm, partner<2>(pm));
    pm = max(pm, partner<4>(pm));
    pm = max(pm, partner<8>(pm));
    pm = lane_value(pm, 0);  // the page's maximum (lanes 0..15 hold it)
    M = max(M, pm);
    if (lane == 0) {
      wmax[wave] = M;
      pmax[s] = pm;
    }
    const float thr = max(M, om) - window;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const float z = zz[t];
      const bool f = z > -__builtin_inff() && z >= thr;
      const uint64_t bal = __ballot(f);
      const int pos = cnt + __popcll(bal & ltm);
      const int ix = phys * PS + t * 16 + tok;
      if (f && pos < kHeadSlots) {
        rz[pos] = z;
        ri[pos] = ix;
      }
      if (__ballot(f && pos >= kHeadSlots) != 0ull) {
        ++nst;
        if (f && pos >= kHeadSlots) {
          Cand<float> cv;
          cv.z = z;
          cv.idx = ix;
          wspill[pos - kHeadSlots] = cv;
        }
      }
      cnt += __popcll(bal);
    }
    return nst;
  };
  // A ring of NBUF buffers: buffer k holds slots wave + (r * NBUF + k) * 8.
  // Before buffer k is read, only the other buffers' loads and the stores
  // issued since buffer k's loads may be outstanding (vmcnt completes in
  // issue order); `since` counts those stores per buffer.
  int since[NBUF];
#pragma unroll
  for (int k = 0; k < NBUF; ++k) {
    issue(s_lo + wave + k * kHNW, k);
    since[k] = 0;
  }
  for (int s0 = s_lo + wave; s0 < s_hi; s0 += NBUF * kHNW) {
#pragma unroll
    for (int k = 0; k < NBUF; ++k) {
      const int s = s0 + k * kHNW;
      if (s < s_hi) {
        wait_vmcnt_plus<(NBUF - 1) * NI>(since[k]);
        const int nst = score_page(s, k);
#pragma unroll
        for (int kk = 0; kk < NBUF; ++kk) since[kk] += nst;
        issue(s + NBUF * kHNW, k);
        since[k] = 0;
      }
    }
  }
  wait_vmcnt<0>();  // no load into LDS is left in flight
  if (lane == 0) {
    wmax[wave] = M;
    wcnt[wave] = cnt;
  }
  __syncthreads();

  // 3. Window list: the workgroup maximum, the window below it (tightened by
  // a lower bound on tau when there are many candidates), each wave's
  // survivors in order at its offset.
  const double am1 = (double)a.alpha - 1.0;
  const double m = 1.0 / am1;
  const int mcode = (m == 1.0) ? 1 : (m == 2.0) ? 2 : (m == 3.0) ? 3 : (m == 4.0) ? 4 : 0;
  float Mg = -__builtin_inff();
  int n_cand = 0;
#pragma unroll
  for (int w = 0; w < kHNW; ++w) {
    Mg = max(Mg, wmax[w]);
    n_cand += wcnt[w];
  }
  float* out_row = a.out + (size_t)bh * D;
  const size_t reg = (size_t)bh * a.splits + split;  // split form: this region
  if (SPLIT && Mg == -__builtin_inff()) {
    if (tid == 0) {
      a.counts[reg] = 0;
      a.maxima[reg] = -__builtin_inff();
    }
    return;
  }
  if (Mg == -__builtin_inff()) {
    for (int d = tid; d < D; d += kHNT) out_row[d] = 0.0f;
    if (tid == 0) {
      if (a.tau_out) a.tau_out[bh] = __builtin_nanf("");
      if (a.sup_out) a.sup_out[bh] = 0;
    }
    return;
  }
  const double amax = am1 * (double)Mg;
  float thr = Mg - window;
  if (n_cand > kTauBoundFrom) {
    // The threshold t_S of any set S of the head's tokens is at most tau;
    // S = the largest page maxima seen by the first 256 threads (each the
    // score of a distinct token), solved by wave 0 in registers. Every
    // support token has a > t_S.
    if (tid < kRegList * kWave) {
      float v = -__builtin_inff();
      for (int s = s_lo + tid; s < s_hi; s += kRegList * kWave) v = max(v, pmax[s]);
      reinterpret_cast<float*>(smem + lay.lz)[tid] = v;  // region A is idle here
    }
    __syncthreads();
    if (wave == 0) {
      const float* pv = reinterpret_cast<const float*>(smem + lay.lz);
      double av[kRegList];
#pragma unroll
      for (int k = 0; k < kRegList; ++k) {
        const float v = pv[k * kWave + lane];
        av[k] = v == -__builtin_inff() ? -DBL_MAX : am1 * (double)v;
      }
      const double ts = with_mcode(mcode, [&](auto mc) {
        return solve_tau_regs<kRegList, decltype(mc)::value>(av, kRegList * kWave, am1, m, mcode,
                                                             amax);
      });
      if (lane == 0) sbound = (float)((ts - 1e-6 * fmax(1.0, fabs(ts))) / am1);
    }
    __syncthreads();
    thr = max(thr, sbound);
  }
  // each wave counts its survivors, then writes them at its offset
  auto entry = [&](int pos, float& z, int& ix) {
    if (pos < kHeadSlots) {
      z = rz[pos];
      ix = ri[pos];
    } else {
      const Cand<float> cv = wspill[pos - kHeadSlots];
      z = cv.z;
      ix = cv.idx;
    }
  };
  int keep = 0;
  for (int base = 0; base < cnt; base += kWave) {
    float z = -__builtin_inff();
    int ix = 0;
    if (base + lane < cnt) entry(base + lane, z, ix);
    keep += __popcll(__ballot(base + lane < cnt && z >= thr));
  }
  if (lane == 0) wcnt[wave] = keep;
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int w = 0; w < kHNW; ++w) {
      woff[w] = o;
      o += wcnt[w];
    }
    woff[kHNW] = o;
  }
  __syncthreads();
  float* lz = reinterpret_cast<float*>(smem + lay.lz);
  int* li = reinterpret_cast<int*>(smem + lay.li);
  float* gz = a.list_z + (size_t)bh * a.list_cap;
  int* gi = a.list_i + (size_t)bh * a.list_cap;
  const int n_list = woff[kHNW];
  {
    int o = woff[wave];
    for (int base = 0; base < cnt; base += kWave) {
      float z = -__builtin_inff();
      int ix = 0;
      if (base + lane < cnt) entry(base + lane, z, ix);
      const bool f = base + lane < cnt && z >= thr;
      const uint64_t bal = __ballot(f);
      const int pos = o + __popcll(bal & ltm);
      if (f) {
        if (pos < kHeadLcap) {
          lz[pos] = z;
          li[pos] = ix;
        } else {
          gz[pos] = z;
          gi[pos] = ix;
        }
      }
      o += __popcll(bal);
    }
  }
  __syncthreads();

  if constexpr (SPLIT) {
    // the region for the threshold kernel: the window list in order, its
    // length and this split's maximum (at most rcap <= LCAP entries)
    Cand<float>* dst = a.cand + reg * a.rcap;
    for (int i = tid; i < n_list; i += kHNT) {
      Cand<float> cv;
      cv.z = lz[i];
      cv.idx = li[i];
      dst[i] = cv;
    }
    if (tid == 0) {
      a.counts[reg] = n_list;
      a.maxima[reg] = Mg;
    }
    return;
  }
  // 4. Threshold, support and output.
  tau_solve_pv<bf16_t, D, kHNT>(a.v_pool, a.Hkv, g, PS, lz, li,
                                reinterpret_cast<float*>(smem + lay.sp),
                                reinterpret_cast<float*>(smem + lay.pv), n_list, kHeadLcap, gz,
                                gi, am1, m, mcode, amax, tsh, out_row,
                                a.tau_out ? a.tau_out + bh : nullptr,
                                a.sup_out ? a.sup_out + bh : nullptr, am1 * (double)thr);
}

}  // namespace ekv
