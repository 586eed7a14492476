// Host plan and instantiations of the per-head select-and-decode kernel
// (bf16 caches; its own translation unit so it compiles in parallel).
#include "head_impl.hpp"

namespace ekv {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

HeadPlan plan_head(const LaunchShape& s, int budget, size_t select_bytes) {
  HeadPlan p;
  const long long heads = (long long)s.batch * s.num_q_heads;
  const int keep = budget < s.max_pages ? budget : s.max_pages;
  const long long head_bytes = (long long)keep * s.page_size * s.head_dim * 2;
  const long long max_bytes = heads > kNumCUs ? kHeadMaxBytesRounds : kHeadMaxBytes;
  const bool fits = s.bf16 && kMfmaScores && budget <= kHeadMaxBudget &&
                    head_lds_layout(budget, s.head_dim).total <= kHeadMaxLds;
  if (fits && heads >= kHeadMinHeads && head_bytes <= max_bytes) {
    p.use = true;
  } else if (fits && heads < kHeadMinHeads) {
    // split form: about kHeadSplitTarget workgroups in all
    long long sp = (kHeadSplitTarget + heads - 1) / heads;
    if (sp > keep) sp = keep;
    if (sp < 1) sp = 1;
    p.pps = (int)((keep + sp - 1) / sp);
    p.splits = (keep + p.pps - 1) / p.pps;
    p.use = (long long)p.pps * s.page_size <= kHeadLcap;
  }
  p.list_cap = keep * s.page_size;
  p.spill = align256(select_bytes);
  if (p.splits > 1) {
    p.wcap = ((p.pps + kHNW - 1) / kHNW) * s.page_size;
    p.tp.pages_per_split = p.pps;
    p.tp.splits = p.splits;
    p.tp.cap = p.pps * s.page_size;
    p.tp.regions = p.splits;
    p.tp.rcap = p.tp.cap;
    p.tp.list_cap = p.list_cap;
    p.tws = decode_ws_layout(s, p.tp);
    p.dec = align256(p.spill + (size_t)heads * p.splits * kHNW * p.wcap * sizeof(Cand<float>));
    p.list = p.dec;
    p.total = align256(p.dec + p.tws.total);
  } else {
    p.pps = keep;
    p.wcap = ((keep + kHNW - 1) / kHNW) * s.page_size;
    p.list = align256(p.spill + (size_t)heads * kHNW * p.wcap * sizeof(Cand<float>));
    p.total = align256(p.list + (size_t)heads * p.list_cap * 8);
  }
  return p;
}

template <int D, int PS, bool CAND, bool SPLIT>
static hipError_t launch_head_t(const LaunchShape& s, const SelectPlan& sp, const HeadPlan& hp,
                                const HeadArgs& a, hipStream_t st) {
  auto kern = head_decode_kernel<D, PS, CAND, SPLIT>;
  // The LDS limit is a kernel attribute: raised once, to the most any plan
  // asks for (a function-local static is initialised exactly once, also when
  // several host threads launch).
  static const hipError_t lds_raised =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHeadMaxLds);
  if (lds_raised != hipSuccess) return lds_raised;
  (void)sp;
  (void)hp;
  const size_t lds = head_lds_layout(a.budget, D).total;
  hipLaunchKernelGGL(kern, dim3((unsigned)(s.batch * s.num_q_heads * hp.splits)), dim3(kHNT), lds,
                     st, a);
  return hipGetLastError();
}

template <int D, bool CAND, bool SPLIT>
static hipError_t launch_head_ps(const LaunchShape& s, const SelectPlan& sp, const HeadPlan& hp,
                                 const HeadArgs& a, hipStream_t st) {
  switch (s.page_size) {
    case 16: return launch_head_t<D, 16, CAND, SPLIT>(s, sp, hp, a, st);
    case 32: return launch_head_t<D, 32, CAND, SPLIT>(s, sp, hp, a, st);
    default: return launch_head_t<D, 64, CAND, SPLIT>(s, sp, hp, a, st);
  }
}

template <int D, bool CAND>
static hipError_t launch_head_sp(const LaunchShape& s, const SelectPlan& sp, const HeadPlan& hp,
                                 const HeadArgs& a, hipStream_t st) {
  return hp.splits > 1 ? launch_head_ps<D, CAND, true>(s, sp, hp, a, st)
                       : launch_head_ps<D, CAND, false>(s, sp, hp, a, st);
}

hipError_t launch_head_decode(const LaunchShape& s, const SelectPlan& sp, const HeadPlan& hp,
                              const float* q, const void* k_pool, const void* v_pool,
                              const int32_t* bt, const int32_t* lens, int budget, float alpha,
                              float window, int32_t* sel, float* sel_ub, float* out, float* tau,
                              int32_t* support, void* ws, bool bt_lds, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  HeadArgs a;
  a.q = q;
  a.k_pool = static_cast<const bf16_t*>(k_pool);
  a.v_pool = static_cast<const bf16_t*>(v_pool);
  a.block_table = bt;
  a.seq_lens = lens;
  a.ub = reinterpret_cast<const float*>(w);
  a.sel = sel;
  a.sel_ub = sel_ub;
  a.H = s.num_q_heads;
  a.Hkv = s.num_kv_heads;
  a.G = s.group;
  a.U = s.batch * s.num_kv_heads;
  a.max_pages = s.max_pages;
  a.num_phys = s.num_phys;
  a.budget = budget;
  a.ldu = ub_ld(s.max_pages);
  a.cp = sp.cp;
  a.keepc = sp.keepc;
  a.nchunks = sp.nchunks;
  a.bt_lds = bt_lds ? 1 : 0;
  a.alpha = alpha;
  a.window_d = (double)window;
  a.spill = reinterpret_cast<Cand<float>*>(w + hp.spill);
  a.wcap = hp.wcap;
  a.list_z = reinterpret_cast<float*>(w + hp.list);
  a.list_i = reinterpret_cast<int*>(a.list_z + (size_t)s.batch * s.num_q_heads * hp.list_cap);
  a.list_cap = hp.list_cap;
  a.out = out;
  a.tau_out = tau;
  a.sup_out = support;
  a.splits = hp.splits;
  a.pps = hp.pps;
  a.rcap = hp.tp.rcap;
  a.cand = hp.splits > 1 ? reinterpret_cast<Cand<float>*>(w + hp.dec + hp.tws.cand) : nullptr;
  a.counts = hp.splits > 1 ? reinterpret_cast<int*>(w + hp.dec + hp.tws.counts) : nullptr;
  a.maxima = hp.splits > 1 ? reinterpret_cast<float*>(w + hp.dec + hp.tws.maxima) : nullptr;
  if (s.head_dim == 64)
    return sp.chunked ? launch_head_sp<64, true>(s, sp, hp, a, st)
                      : launch_head_sp<64, false>(s, sp, hp, a, st);
  return sp.chunked ? launch_head_sp<128, true>(s, sp, hp, a, st)
                    : launch_head_sp<128, false>(s, sp, hp, a, st);
}

}  // namespace ekv
