// Instantiations of the decode kernels for f32 caches (one translation unit
// per cache dtype so the two compile in parallel).
#include "decode_impl.hpp"

namespace ekv {

hipError_t launch_score_f32(const LaunchShape& s, const SplitPlan& p, const float* q,
                          const void* k_pool, const int32_t* bt, const int32_t* lens,
                          const int32_t* sel, int budget, float alpha, float window, void* ws,
                          const DecodeWs& L, hipStream_t st) {
  return launch_score_kv<float>(s, p, q, k_pool, bt, lens, sel, budget, alpha, window, ws, L, st);
}

hipError_t launch_tau_pv_f32(const LaunchShape& s, const SplitPlan& p, const void* v_pool,
                           const int32_t* bt, const int32_t* lens, const int32_t* sel,
                           int budget, float alpha, float window, float* out, float* tau,
                           int32_t* support, void* ws, const DecodeWs& L, hipStream_t st) {
  return launch_tau_pv_kv<float>(s, p, v_pool, bt, lens, sel, budget, alpha, window, out, tau,
                              support, ws, L, st);
}

}  // namespace ekv
