// Host-only exercise of the C ABI's validation and planning code, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
// Every call here either fails validation or only plans workspaces, so no
// HIP call is reached and no GPU is needed. Exits non-zero on the first
// return code that differs from the documented one.
#include <math.h>
#include <stdio.h>

#include "entmaxkv.h"

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static entmaxkv_shape make(int B, int H, int Hkv, int D, int ps, int mp, int nphys, int dt) {
  entmaxkv_shape s;
  s.batch = B;
  s.num_q_heads = H;
  s.num_kv_heads = Hkv;
  s.head_dim = D;
  s.page_size = ps;
  s.max_pages_per_seq = mp;
  s.num_phys_pages = nphys;
  s.kv_dtype = dt;
  return s;
}

int main() {
  // fake, suitably aligned addresses: never dereferenced on the host, and
  // every call below is rejected before anything is launched
  void* d = reinterpret_cast<void*>(uintptr_t(1) << 20);
  void* mis8 = reinterpret_cast<void*>((uintptr_t(1) << 20) + 8);
  void* mis16 = reinterpret_cast<void*>((uintptr_t(1) << 20) + 16);
  const float* q = static_cast<const float*>(d);
  const int32_t* ci = static_cast<const int32_t*>(d);
  int32_t* oi = static_cast<int32_t*>(d);
  float* of = static_cast<float*>(d);
  const size_t big = size_t(1) << 40;

  if (entmaxkv_version() < 100) ++failures;
  for (int c = -12; c <= 12; ++c)
    if (!entmaxkv_strerror(c) || !entmaxkv_strerror(c)[0]) ++failures;

  // workspace planning over the supported set, up to the largest sizes the
  // ABI accepts (sizes computed in 64 bits: UBSan flags any signed overflow)
  const int Ds[] = {64, 128}, pss[] = {16, 32, 64}, Gs[] = {1, 2, 4, 8};
  const int mps[] = {1, 7, 4096, 262144};
  const int budgets[] = {1, 82, 1024, 1025, 1 << 22};
  for (int D : Ds)
    for (int ps : pss)
      for (int G : Gs)
        for (int mp : mps)
          for (int dt = 0; dt < 2; ++dt)
            for (int B : {1, 16, (1 << 24) / 64}) {
              const int Hkv = 8, H = Hkv * G;
              if ((long long)B * H > (1LL << 24)) continue;
              const int nphys = 0x7fffffff / ps;
              entmaxkv_shape s = make(B, H, Hkv, D, ps, mp, nphys, dt);
              size_t n = 0;
              int rc = entmaxkv_workspace_bytes(&s, 0, ENTMAXKV_WS_FULL, &n);
              if (rc != ENTMAXKV_OK && rc != ENTMAXKV_ERR_UNSUPPORTED) ++failures;
              for (int budget : budgets) {
                for (int which = 0; which <= 4; ++which) {
                  rc = entmaxkv_workspace_bytes(&s, budget, which, &n);
                  if (rc != ENTMAXKV_OK && rc != ENTMAXKV_ERR_UNSUPPORTED) {
                    fprintf(stderr, "workspace_bytes rc %d (which %d)\n", rc, which);
                    ++failures;
                  }
                }
                int32_t k = 0;
                rc = entmaxkv_topk_kernels(&s, budget, &k);
                if (rc == ENTMAXKV_OK && (k < 2 || k > 4)) ++failures;
              }
            }

  entmaxkv_shape s = make(4, 32, 8, 128, 32, 4096, 16384, ENTMAXKV_BF16);
  size_t n = 0;
  EXPECT(entmaxkv_workspace_bytes(nullptr, 82, ENTMAXKV_WS_SELECT, &n), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_workspace_bytes(&s, 82, ENTMAXKV_WS_SELECT, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_workspace_bytes(&s, 82, 5, &n), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_workspace_bytes(&s, 82, -1, &n), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_workspace_bytes(&s, 0, ENTMAXKV_WS_TOPK, &n), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_topk_kernels(&s, 82, nullptr), ENTMAXKV_ERR_INVALID);

  // shapes outside the supported set or with non-positive sizes
  const entmaxkv_shape bad[] = {
      make(0, 32, 8, 128, 32, 4096, 16384, 1),   make(4, 6, 4, 128, 32, 4096, 16384, 1),
      make(4, 32, 8, 96, 32, 4096, 16384, 1),    make(4, 32, 8, 128, 8, 4096, 16384, 1),
      make(4, 48, 3, 128, 32, 4096, 16384, 1),   make(4, 32, 8, 128, 32, 4096, 16384, 7),
      make(4, 32, 8, 128, 32, 262145, 16384, 1), make(4, 32, 8, 128, 32, 4096, 0, 1),
      make(4, 32, 8, 128, 64, 4096, 0x7fffffff / 32, 1),
      make(1 << 20, 32, 8, 128, 32, 4096, 16384, 1), make(-1, -1, -1, -1, -1, -1, -1, -1)};
  for (const entmaxkv_shape& b : bad) {
    if (entmaxkv_workspace_bytes(&b, 82, ENTMAXKV_WS_FULL, &n) == ENTMAXKV_OK) ++failures;
    if (entmaxkv_build_page_meta(&b, d, ci, ci, d, nullptr, nullptr) == ENTMAXKV_OK) ++failures;
    if (entmaxkv_decode_full(&b, q, d, d, ci, ci, 1.5f, of, nullptr, nullptr, d, big, nullptr,
                             nullptr) == ENTMAXKV_OK)
      ++failures;
  }

  // null and misaligned pointers, bad budgets and alphas, short workspaces
  EXPECT(entmaxkv_build_page_meta(nullptr, d, ci, ci, d, nullptr, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_build_page_meta(&s, nullptr, ci, ci, d, nullptr, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_build_page_meta(&s, mis8, ci, ci, d, nullptr, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_build_page_meta(&s, d, ci, ci, mis8, nullptr, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_append_page_meta(&s, d, ci, ci, ci, 0, d, nullptr, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_append_page_meta(&s, d, ci, ci, nullptr, 1, d, nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_build_page_moments(&s, d, ci, ci, mis8, nullptr, nullptr), ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_append_page_moments(&s, d, ci, ci, ci, -1, d, nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);

  EXPECT(entmaxkv_score_select(&s, q, d, ci, ci, 0, oi, nullptr, d, big, nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_score_select(&s, q, d, ci, ci, (1 << 22) + 1, oi, nullptr, d, big, nullptr,
                               nullptr),
         ENTMAXKV_ERR_UNSUPPORTED);
  EXPECT(entmaxkv_score_select(&s, q, d, ci, ci, 82, oi, nullptr, d, 16, nullptr, nullptr),
         ENTMAXKV_ERR_WORKSPACE);
  EXPECT(entmaxkv_score_select(&s, q, d, ci, ci, 82, oi, nullptr, nullptr, big, nullptr, nullptr),
         ENTMAXKV_ERR_WORKSPACE);
  EXPECT(entmaxkv_score_select(&s, q, d, ci, ci, 82, oi, nullptr, mis16, big, nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_score_select_noalloc(&s, q, d, ci, ci, 82, nullptr, nullptr, nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);
  {
    entmaxkv_shape huge = make(4, 32, 8, 128, 16, 32772, 1 << 20, 1);
    EXPECT(entmaxkv_score_select_noalloc(&huge, q, d, ci, ci, 82, oi, nullptr, nullptr, nullptr),
           ENTMAXKV_ERR_WORKSPACE);
  }

  const float alphas[] = {1.0f, 0.5f, -2.0f, NAN, INFINITY};
  for (float a : alphas) {
    EXPECT(entmaxkv_decode_full(&s, q, d, d, ci, ci, a, of, nullptr, nullptr, d, big, nullptr,
                                nullptr),
           ENTMAXKV_ERR_INVALID);
    EXPECT(entmaxkv_decode_sparse(&s, q, d, d, ci, ci, ci, 82, a, of, nullptr, nullptr, d, big,
                                  nullptr, nullptr),
           ENTMAXKV_ERR_INVALID);
    EXPECT(entmaxkv_decode_topk(&s, q, d, d, d, ci, ci, 82, a, oi, nullptr, of, nullptr, nullptr,
                                d, big, nullptr, nullptr),
           ENTMAXKV_ERR_INVALID);
    EXPECT(entmaxkv_gauss_select(&s, q, d, ci, ci, a, 0.0f, 64, oi, nullptr, d, big, nullptr,
                                 nullptr),
           ENTMAXKV_ERR_INVALID);
  }
  EXPECT(entmaxkv_gauss_select(&s, q, d, ci, ci, 1.4f, 0.0f, 64, oi, nullptr, d, big, nullptr,
                               nullptr),
         ENTMAXKV_ERR_UNSUPPORTED);
  EXPECT(entmaxkv_gauss_select(&s, q, d, ci, ci, 1.5f, -1.0f, 64, oi, nullptr, d, big, nullptr,
                               nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_gauss_select(&s, q, d, ci, ci, 1.5f, 0.0f, 0, oi, nullptr, d, big, nullptr,
                               nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_gauss_select(&s, q, d, ci, ci, 1.5f, 0.0f, 64, oi, nullptr, d, 1, nullptr,
                               nullptr),
         ENTMAXKV_ERR_WORKSPACE);

  for (int w = 0; w <= 2; ++w) {
    const size_t need = [&] {
      size_t x = 0;
      entmaxkv_workspace_bytes(&s, 82, w == 0 ? ENTMAXKV_WS_SPARSE
                                             : (w == 1 ? ENTMAXKV_WS_FULL : ENTMAXKV_WS_TOPK),
                               &x);
      return x;
    }();
    if (need == 0) ++failures;
    if (w == 0)
      EXPECT(entmaxkv_decode_sparse(&s, q, d, d, ci, ci, ci, 82, 1.5f, of, nullptr, nullptr, d,
                                    need - 1, nullptr, nullptr),
             ENTMAXKV_ERR_WORKSPACE);
    if (w == 1)
      EXPECT(entmaxkv_decode_full(&s, q, d, d, ci, ci, 1.5f, of, nullptr, nullptr, d, need - 1,
                                  nullptr, nullptr),
             ENTMAXKV_ERR_WORKSPACE);
    if (w == 2)
      EXPECT(entmaxkv_decode_topk(&s, q, d, d, d, ci, ci, 82, 1.5f, oi, nullptr, of, nullptr,
                                  nullptr, d, need - 1, nullptr, nullptr),
             ENTMAXKV_ERR_WORKSPACE);
  }
  EXPECT(entmaxkv_decode_sparse(&s, q, mis8, d, ci, ci, ci, 82, 1.5f, of, nullptr, nullptr, d, big,
                                nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_decode_sparse(&s, q, d, d, ci, ci, ci, -3, 1.5f, of, nullptr, nullptr, d, big,
                                nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);
  EXPECT(entmaxkv_decode_topk(&s, q, d, d, d, ci, ci, 82, 1.5f, nullptr, nullptr, of, nullptr,
                              nullptr, d, big, nullptr, nullptr),
         ENTMAXKV_ERR_INVALID);

  if (failures) {
    fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  printf("abi driver ok\n");
  return 0;
}
