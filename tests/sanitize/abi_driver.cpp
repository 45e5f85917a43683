// Host-side check of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_abi_sanitize.py with the host code of every library source
// instrumented (device code is not).  Every call below either fails validation or is a
// workspace-size query, so nothing is launched and no pointer is dereferenced: the fake
// pointer P is never read.  The parameter sweep covers the shapes the library serves
// (decode, prefill, the split and chunk limits) and extreme sizes whose arithmetic
// would overflow if it were done in the wrong type.  Exit status 0: every status was one
// of the expected ones; sanitizer reports abort the run.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "dsv4attn.h"

static int failures = 0;
static long answered = 0;   // size queries answered with DSV4_OK
static void* const P = (void*)(uintptr_t)16;

static void expect(const char* what, int st, std::initializer_list<int> ok) {
  bool hit = false;
  for (int o : ok) hit = hit || st == o;
  if (!hit) {
    ++failures;
    printf("FAIL %s: status %d (%s), last error: %s\n", what, st, dsv4_status_string(st), dsv4_last_error());
  }
}

// A size query must answer OK (or reject the shape) and answer the same twice.
static void query(const char* what, int st1, size_t n1, int st2, size_t n2) {
  expect(what, st1, {DSV4_OK, DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED});
  answered += st1 == DSV4_OK;
  if (st1 != st2 || (st1 == DSV4_OK && n1 != n2)) {
    ++failures;
    printf("FAIL %s: two size queries disagree (%d %zu, %d %zu)\n", what, st1, n1, st2, n2);
  }
}

int main() {
  // Some calls below pass validation with sizes a launch would use: they may run only
  // where no GPU is visible (then the launch fails cleanly).
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    printf("skipped: a GPU is visible (this check runs on hosts without one)\n");
    return 77;
  }
  const int F32 = DSV4_F32, BF16 = DSV4_BF16, E4M3 = DSV4_FP8_E4M3, MX = DSV4_MXFP4;
  expect("version", dsv4_version() >= 100 ? 0 : 1, {0});
  for (int s = -1; s < 8; ++s) expect("status string", dsv4_status_string(s) ? 0 : 1, {0});
  expect("time_next_kernel one event", dsv4_time_next_kernel((hipEvent_t)P, nullptr), {DSV4_ERR_INVALID_ARG});

  const int64_t big[] = {0, 1, 7, 4096, 65536, 262144, (int64_t)1 << 21, (int64_t)1 << 31, (int64_t)1 << 40,
                         INT64_MAX / 2, INT64_MAX, -1, INT64_MIN};

  // ---- pooling: invalid arguments only
  expect("compress m=0", csa_compress(P, BF16, (float*)P, (float*)P, 1, 16, 64, 0, 0, P, nullptr, BF16, 0, nullptr),
         {DSV4_ERR_INVALID_ARG});
  expect("compress null x", csa_compress(nullptr, BF16, (float*)P, (float*)P, 1, 16, 64, 4, 0, P, nullptr, BF16, 0, nullptr),
         {DSV4_ERR_INVALID_ARG});
  for (int64_t v : big) {
    expect("compress B", csa_compress(P, BF16, (float*)P, (float*)P, v, 16, 64, 4, 0, P, nullptr, BF16, 0, nullptr),
           {DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED, DSV4_OK, DSV4_ERR_LAUNCH});
    expect("compress T", csa_compress(P, BF16, (float*)P, (float*)P, 1, v, 64, 4, 0, nullptr, nullptr, BF16, 0, nullptr),
           {DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED, DSV4_OK, DSV4_ERR_LAUNCH});
    expect("compress2 C2", csa_compress2(P, P, BF16, (float*)P, (float*)P, 1, 4, 4, 64, 0, P, nullptr, BF16, 0, v, 0,
                                         nullptr, nullptr, MX, 0, nullptr),
           {DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED, DSV4_OK, DSV4_ERR_LAUNCH});
    expect("append L", kv_cache_append(P, BF16, (float*)P, (int32_t*)P, 1, 64, P, (float*)P, v, (float*)P, 4,
                                       nullptr, nullptr, BF16, 16, 0, nullptr),
           {DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED, DSV4_OK, DSV4_ERR_LAUNCH});
  }

  // ---- indexer + top-k: size queries over a sweep, then invalid arguments
  const int kinds[][2] = {{BF16, BF16}, {BF16, MX}, {E4M3, E4M3}, {MX, MX}, {F32, F32}, {BF16, E4M3}};
  const int64_t Bs[] = {1, 8, 64, 65535, 65536, (int64_t)1 << 31};
  const int64_t Qs[] = {1, 3, 8, 4096, (int64_t)1 << 20};
  const int64_t Ns[] = {0, 1, 100, 4096, 65536, 262144, ((int64_t)1 << 21) + 5, (int64_t)1 << 31, (int64_t)1 << 40};
  const int32_t Ks[] = {1, 64, 1024, 2048, 1 << 20};
  const int32_t HIs[] = {4, 8, 16, 3};
  const int32_t DIs[] = {64, 128, 256, 96};
  for (auto& kd : kinds)
    for (int64_t B : Bs)
      for (int64_t Q : Qs)
        for (int64_t N : Ns)
          for (int32_t k : Ks)
            for (int hi = 0; hi < 4; ++hi) {
              const int32_t HI = HIs[hi], DI = DIs[(hi + (int)(N & 3)) % 4];
              size_t n1 = 0, n2 = 0;
              const uint8_t* ks = kd[1] == MX ? (const uint8_t*)P : nullptr;
              int s1 = csa_index_topk(P, kd[0], (float*)P, P, ks, kd[1], (int32_t*)P, B, Q, HI, DI, N, 0, 4, k,
                                      (int32_t*)P, nullptr, nullptr, &n1, nullptr);
              int s2 = csa_index_topk(P, kd[0], (float*)P, P, ks, kd[1], (int32_t*)P, B, Q, HI, DI, N, 0, 4, k,
                                      (int32_t*)P, nullptr, nullptr, &n2, nullptr);
              query("index_topk query", s1, n1, s2, n2);
            }
  for (int64_t v : big) {
    size_t n = 0;
    expect("index_topk ki_bstride", csa_index_topk(P, BF16, (float*)P, P, nullptr, BF16, (int32_t*)P, 2, 1, 8, 128, 4096,
                                                   v, 4, 64, (int32_t*)P, nullptr, nullptr, &n, nullptr),
           {DSV4_OK, DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED});
  }
  expect("index_topk k=0", csa_index_topk(P, BF16, (float*)P, P, nullptr, BF16, (int32_t*)P, 1, 1, 8, 128, 4096, 0, 4, 0,
                                          (int32_t*)P, nullptr, nullptr, nullptr, nullptr),
         {DSV4_ERR_INVALID_ARG});
  expect("index_topk small workspace", csa_index_topk(P, BF16, (float*)P, P, nullptr, BF16, (int32_t*)P, 1, 1, 8, 128,
                                                      4096, 0, 4, 64, (int32_t*)P, nullptr, P, nullptr, nullptr),
         {DSV4_ERR_INVALID_ARG, DSV4_ERR_WORKSPACE});
  {
    size_t tiny = 1;
    expect("index_topk too small", csa_index_topk(P, BF16, (float*)P, P, nullptr, BF16, (int32_t*)P, 1, 1, 8, 128, 4096, 0,
                                                  4, 64, (int32_t*)P, nullptr, P, &tiny, nullptr),
           {DSV4_ERR_WORKSPACE});
  }
  expect("noalloc too large", csa_index_topk_noalloc(P, BF16, (float*)P, P, nullptr, BF16, (int32_t*)P, 64, 4096, 8, 128,
                                                     65536, 0, 4, 2048, (int32_t*)P, nullptr, nullptr),
         {DSV4_ERR_UNSUPPORTED, DSV4_ERR_LAUNCH, DSV4_ERR_INVALID_ARG});

  // ---- pooling + indexer in one launch: size queries and invalid pools
  {
    dsv4_block_pool pl = {P, P, (float*)P, (float*)P, 1024, 128, 128, P, nullptr, BF16, 0, 0};
    for (int64_t N : Ns)
      for (int64_t row : {(int64_t)0, N - 1, N, (int64_t)-1})
        for (int32_t DI : {64, 128, 256}) {
          pl.row = row;
          size_t n1 = 0, n2 = 0;
          int s1 = csa_pool_index_topk(&pl, P, BF16, (float*)P, P, (uint8_t*)P, MX, (int32_t*)P, 8, 1, 8, DI, N, 0, 4, 1024,
                                       (int32_t*)P, nullptr, nullptr, &n1, nullptr);
          int s2 = csa_pool_index_topk(&pl, P, BF16, (float*)P, P, (uint8_t*)P, MX, (int32_t*)P, 8, 1, 8, DI, N, 0, 4, 1024,
                                       (int32_t*)P, nullptr, nullptr, &n2, nullptr);
          query("pool_index_topk query", s1, n1, s2, n2);
          if (row < 0 || row >= N) expect("pool row outside [0, N)", s1, {DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED});
        }
    expect("pool NULL", csa_pool_index_topk(nullptr, P, BF16, (float*)P, P, (uint8_t*)P, MX, (int32_t*)P, 8, 1, 8, 128,
                                            4096, 0, 4, 64, (int32_t*)P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_INVALID_ARG});
    pl.row = 5;
    pl.y_dt = E4M3;
    expect("pool y_dt", csa_pool_index_topk(&pl, P, BF16, (float*)P, P, (uint8_t*)P, MX, (int32_t*)P, 8, 1, 8, 128, 4096,
                                            0, 4, 64, (int32_t*)P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_UNSUPPORTED});
    pl.y_dt = BF16;
    expect("pool bf16 keys", csa_pool_index_topk(&pl, P, BF16, (float*)P, P, nullptr, BF16, (int32_t*)P, 8, 1, 8, 128,
                                                 4096, 0, 4, 64, (int32_t*)P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_UNSUPPORTED});
    expect("pool m*DI", csa_pool_index_topk(&pl, P, BF16, (float*)P, P, (uint8_t*)P, MX, (int32_t*)P, 8, 1, 8, 256, 4096,
                                            0, 4, 64, (int32_t*)P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_UNSUPPORTED});
    expect("pool m not a power of two", csa_pool_index_topk(&pl, P, BF16, (float*)P, P, (uint8_t*)P, MX, (int32_t*)P, 8,
                                                            1, 8, 128, 4096, 0, 3, 64, (int32_t*)P, nullptr, nullptr,
                                                            nullptr, nullptr),
           {DSV4_ERR_UNSUPPORTED});
  }

  // ---- attention: size queries over a sweep (bf16, f32, FP8 rows), then invalid arguments
  const int32_t Hs[] = {16, 64, 48, 17};
  const int32_t Ds[] = {128, 512, 256, 100};
  const int64_t Ls[] = {0, 128, 4096};
  const int32_t Ws[] = {0, 128, 4096};
  for (int dt : {BF16, F32})
    for (int64_t B : Bs)
      for (int64_t Q : Qs)
        for (int64_t N : Ns)
          for (int32_t k : Ks)
            for (int i = 0; i < 4; ++i)
              for (int w = 0; w < 3; ++w) {
                const int32_t H = Hs[i], D = Ds[(i + w) % 4], W = Ws[w];
                const int64_t L = Ls[(w + 1) % 3];
                size_t n1 = 0, n2 = 0;
                int s1 = csa_attend(P, P, P, dt, (int32_t*)P, k, P, P, (int32_t*)P, L, W, (int32_t*)P, B, Q, H, D, N, 0, 0,
                                    0, 0.1f, P, nullptr, nullptr, &n1, nullptr);
                int s2 = csa_attend(P, P, P, dt, (int32_t*)P, k, P, P, (int32_t*)P, L, W, (int32_t*)P, B, Q, H, D, N, 0, 0,
                                    0, 0.1f, P, nullptr, nullptr, &n2, nullptr);
                query("csa_attend query", s1, n1, s2, n2);
                s1 = hca_attend(P, P, P, dt, 128, P, P, nullptr, L, W, (int32_t*)P, B, Q, H, D, N, 0, 0, 0, 0.1f, P,
                                nullptr, nullptr, &n1, nullptr);
                s2 = hca_attend(P, P, P, dt, 128, P, P, nullptr, L, W, (int32_t*)P, B, Q, H, D, N, 0, 0, 0, 0.1f, P,
                                nullptr, nullptr, &n2, nullptr);
                query("hca_attend query", s1, n1, s2, n2);
                if (dt == BF16) {
                  s1 = csa_attend_fp8kv(P, P, P, (int32_t*)P, k, P, P, (int32_t*)P, L, W, (int32_t*)P, B, Q, H, D, 64, N,
                                        0, 0, 0, 1.f, 1.f, 0.1f, P, nullptr, nullptr, &n1, nullptr);
                  s2 = csa_attend_fp8kv(P, P, P, (int32_t*)P, k, P, P, (int32_t*)P, L, W, (int32_t*)P, B, Q, H, D, 64, N,
                                        0, 0, 0, 1.f, 1.f, 0.1f, P, nullptr, nullptr, &n2, nullptr);
                  query("csa_attend_fp8kv query", s1, n1, s2, n2);
                  s1 = hca_attend_fp8kv(P, P, P, 128, P, P, nullptr, L, W, (int32_t*)P, B, Q, H, D, 64, N, 0, 0, 0, 1.f,
                                        1.f, 0.1f, P, nullptr, nullptr, &n1, nullptr);
                  s2 = hca_attend_fp8kv(P, P, P, 128, P, P, nullptr, L, W, (int32_t*)P, B, Q, H, D, 64, N, 0, 0, 0, 1.f,
                                        1.f, 0.1f, P, nullptr, nullptr, &n2, nullptr);
                  query("hca_attend_fp8kv query", s1, n1, s2, n2);
                }
              }
  for (int64_t v : big) {
    size_t n = 0;
    expect("csa_attend strides", csa_attend(P, P, P, BF16, (int32_t*)P, 64, P, P, (int32_t*)P, 128, 128, (int32_t*)P, 2,
                                            1, 64, 512, 4096, v, v, v, 0.1f, P, nullptr, nullptr, &n, nullptr),
           {DSV4_OK, DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED});
  }
  expect("csa_attend null q", csa_attend(nullptr, P, P, BF16, (int32_t*)P, 64, P, P, (int32_t*)P, 128, 128, (int32_t*)P, 2,
                                         1, 64, 512, 4096, 0, 0, 0, 0.1f, P, nullptr, nullptr, nullptr, nullptr),
         {DSV4_ERR_INVALID_ARG});
  expect("hca_attend m=0", hca_attend(P, P, P, BF16, 0, P, P, nullptr, 128, 128, (int32_t*)P, 2, 1, 64, 512, 4096, 0, 0,
                                      0, 0.1f, P, nullptr, nullptr, nullptr, nullptr),
         {DSV4_ERR_INVALID_ARG});

  // ---- HCA pooling + attention in one launch: size queries and invalid arguments
  {
    const int32_t QP[] = {1, 2, 15, 16};
    for (int64_t N : Ns)
      for (int32_t Q : QP)
        for (int32_t H : {16, 64}) {
          size_t n1 = 0, n2 = 0;
          uint16_t* kc = (uint16_t*)P;
          int s1 = hca_pool_attend(P, (float*)P, (float*)P, 0, P, kc, kc + 512, BF16, 128, P, P, (int32_t*)P, 128, 128,
                                   (int32_t*)P, 8, Q, H, 512, N, 0, 1024, 0, 0.1f, P, nullptr, nullptr, &n1, nullptr);
          int s2 = hca_pool_attend(P, (float*)P, (float*)P, 0, P, kc, kc + 512, BF16, 128, P, P, (int32_t*)P, 128, 128,
                                   (int32_t*)P, 8, Q, H, 512, N, 0, 1024, 0, 0.1f, P, nullptr, nullptr, &n2, nullptr);
          query("hca_pool_attend query", s1, n1, s2, n2);
        }
    uint16_t* kc = (uint16_t*)P;
    expect("hca_pool_attend split K/V", hca_pool_attend(P, (float*)P, (float*)P, 0, P, kc, kc + 4096, BF16, 128, P, P,
                                                        (int32_t*)P, 128, 128, (int32_t*)P, 8, 1, 64, 512, 1000, 0, 1024,
                                                        0, 0.1f, P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_INVALID_ARG});
    expect("hca_pool_attend D", hca_pool_attend(P, (float*)P, (float*)P, 0, P, kc, kc + 256, BF16, 128, P, P,
                                                (int32_t*)P, 128, 128, (int32_t*)P, 8, 1, 64, 256, 1000, 0, 512, 0,
                                                0.1f, P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_UNSUPPORTED});
    expect("hca_pool_attend N=0", hca_pool_attend(P, (float*)P, (float*)P, 0, P, kc, kc + 512, BF16, 128, P, P,
                                                  (int32_t*)P, 128, 128, (int32_t*)P, 8, 1, 64, 512, 0, 0, 1024, 0,
                                                  0.1f, P, nullptr, nullptr, nullptr, nullptr),
           {DSV4_ERR_INVALID_ARG});
  }

  // ---- merge: invalid arguments only
  for (int64_t v : big) {
    expect("lse_merge R", lse_merge((float*)P, (float*)P, 2, v, 64, P, F32, nullptr, nullptr),
           {DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED, DSV4_OK, DSV4_ERR_LAUNCH});
  }
  expect("lse_merge P=0", lse_merge((float*)P, (float*)P, 0, 4, 64, P, F32, nullptr, nullptr), {DSV4_ERR_INVALID_ARG});

  printf("%s: %d failures; %ld size queries answered\n", failures ? "FAILED" : "ok", failures, answered);
  return failures ? 1 : 0;
}
