// Host-side argument checks of the C ABI, for a build of the host code with
// AddressSanitizer and UndefinedBehaviorSanitizer: every call below must be
// rejected on the host, before any HIP call, with the status and a message
// naming the problem.  Needs no GPU.  Exit status 0 iff every check holds;
// a sanitizer report aborts the process.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "sekv.h"

static int g_fail = 0;

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

static sekv_config base_config() {
  sekv_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = 2;
  c.n_q_heads = 8;
  c.n_kv_heads = 2;
  c.head_dim = 128;
  c.route_dim = 32;
  c.window = 512;
  c.max_rank = 32;
  c.min_span_len = 4;
  c.alpha = 1.0;
  c.gamma = 0.0;
  c.kv_dtype = SEKV_BF16;
  c.factor_tier = SEKV_TIER_DEVICE;
  c.svd_mode = SEKV_SVD_EXACT;
  return c;
}

// a non-NULL pointer that is never dereferenced (the checks fail first)
static void* const P = reinterpret_cast<void*>(8);

static void expect_bad_config(void (*edit)(sekv_config&), const char* word) {
  sekv_config c = base_config();
  edit(c);
  sekv_cache* out = reinterpret_cast<sekv_cache*>(P);
  const sekv_status st = sekv_build_spans(&c, 100, static_cast<const float*>(P), P, P,
                                          static_cast<const float*>(P), nullptr, nullptr, &out);
  CHECK(st == SEKV_ERR_INVALID);
  CHECK(std::strstr(sekv_last_error(), word) != nullptr);
  CHECK(out == nullptr);
}

int main() {
  expect_bad_config([](sekv_config& c) { c.head_dim = 64; }, "head_dim");
  expect_bad_config([](sekv_config& c) { c.n_q_heads = 7; }, "multiple");
  expect_bad_config([](sekv_config& c) { c.n_kv_heads = 0; }, "multiple");
  expect_bad_config([](sekv_config& c) { c.route_dim = 65; }, "route_dim");
  expect_bad_config([](sekv_config& c) { c.max_rank = 129; }, "max_rank");
  expect_bad_config([](sekv_config& c) { c.min_span_len = 0; }, "min_span_len");
  expect_bad_config([](sekv_config& c) { c.window = -1; }, "window");
  expect_bad_config([](sekv_config& c) { c.n_layers = 0; }, "n_layers");
  expect_bad_config([](sekv_config& c) { c.kv_dtype = 7; }, "kv_dtype");
  expect_bad_config([](sekv_config& c) { c.factor_tier = 3; }, "factor_tier");
  expect_bad_config([](sekv_config& c) { c.alpha = NAN; }, "finite");
  expect_bad_config([](sekv_config& c) { c.gamma = INFINITY; }, "finite");
  expect_bad_config([](sekv_config& c) { c.svd_mode = 2; }, "svd_mode");
  expect_bad_config([](sekv_config& c) { c.append_capacity = -1; }, "append_capacity");
  expect_bad_config([](sekv_config& c) { c.n_q_heads = 1 << 20; c.n_kv_heads = 1 << 17; },
                    "");

  // NULL inputs, sizes and outputs of the build and the segmentation
  sekv_config c = base_config();
  sekv_cache* out = nullptr;
  const float* F = static_cast<const float*>(P);
  CHECK(sekv_build_spans(&c, 100, nullptr, P, P, F, nullptr, nullptr, &out) == SEKV_ERR_INVALID);
  CHECK(sekv_build_spans(&c, 0, F, P, P, F, nullptr, nullptr, &out) == SEKV_ERR_INVALID);
  CHECK(sekv_build_spans(&c, -5, F, P, P, F, nullptr, nullptr, &out) == SEKV_ERR_INVALID);
  CHECK(sekv_build_spans(&c, 10, F, P, P, F, nullptr, nullptr, nullptr) == SEKV_ERR_INVALID);
  CHECK(sekv_build_spans(nullptr, 10, F, P, P, F, nullptr, nullptr, &out) == SEKV_ERR_INVALID);
  CHECK(sekv_segment(nullptr, 10, F, nullptr, nullptr, nullptr, nullptr) == SEKV_ERR_INVALID);
  CHECK(sekv_segment(&c, 10, nullptr, nullptr, nullptr, nullptr, nullptr) == SEKV_ERR_INVALID);

  // every call on a NULL cache
  sekv_route_out ro;
  std::memset(&ro, 0, sizeof ro);
  CHECK(sekv_route(nullptr, 0, F, F, F, &ro, nullptr) == SEKV_ERR_INVALID);
  CHECK(sekv_decode_attn(nullptr, 0, F, &ro, nullptr, nullptr, 0, nullptr, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_route_attn(nullptr, 0, F, F, F, &ro, nullptr, nullptr, 0, nullptr, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_route_attn_noalloc(nullptr, 0, F, F, F, &ro, nullptr, nullptr, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_cap_budget(nullptr, &ro, 0, nullptr) == SEKV_ERR_INVALID);
  CHECK(sekv_cap_budget_layer(nullptr, &ro, 0, nullptr) == SEKV_ERR_INVALID);
  CHECK(sekv_set_residency(nullptr, 1 << 20, 1 << 16) == SEKV_ERR_INVALID);
  CHECK(sekv_set_fetch_mode(nullptr, SEKV_FETCH_MEMCPY) == SEKV_ERR_INVALID);
  CHECK(sekv_apply_gates(nullptr, F, F, 0.5f, nullptr) == SEKV_ERR_INVALID);
  CHECK(sekv_append_tokens(nullptr, 1, F, P, P, F, nullptr, nullptr) == SEKV_ERR_INVALID);
  uint64_t stats[6];
  CHECK(sekv_residency_stats(nullptr, stats, 0) == SEKV_ERR_INVALID);
  CHECK(sekv_decode_workspace_bytes(nullptr) == 0);
  sekv_cache_info info;
  CHECK(sekv_cache_info_get(nullptr, &info) == SEKV_ERR_INVALID);
  CHECK(sekv_cache_copy_spans(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_cache_copy_group(nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_cache_copy_factors(nullptr, 0, 0, 0, 0, nullptr, nullptr, nullptr) ==
        SEKV_ERR_INVALID);
  sekv_cache_destroy(nullptr);

  // batch calls: no array, batch sizes out of range, NULL caches in the array
  const sekv_cache* caches[2] = {nullptr, nullptr};
  const float* qs[2] = {F, F};
  sekv_route_out ros[2];
  std::memset(ros, 0, sizeof ros);
  float* os[2] = {nullptr, nullptr};
  void* wss[2] = {nullptr, nullptr};
  size_t sizes[2] = {0, 0};
  for (int b : {0, -1, SEKV_MAX_BATCH + 1}) {
    CHECK(sekv_route_attn_batch(caches, b, 0, qs, F, F, ros, os, wss, sizes, nullptr) ==
          SEKV_ERR_INVALID);
    CHECK(std::strstr(sekv_last_error(), "batch") != nullptr);
    CHECK(sekv_decode_attn_batch(caches, b, 0, qs, ros, os, wss, sizes, nullptr) ==
          SEKV_ERR_INVALID);
  }
  CHECK(sekv_route_attn_batch(nullptr, 2, 0, qs, F, F, ros, os, wss, sizes, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_route_attn_batch(caches, 2, 0, qs, F, F, ros, os, wss, sizes, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_route_attn_batch(caches, 2, 0, qs, nullptr, nullptr, ros, os, wss, sizes, nullptr) ==
        SEKV_ERR_INVALID);
  CHECK(sekv_decode_attn_batch(caches, 2, 0, qs, ros, os, wss, sizes, nullptr) ==
        SEKV_ERR_INVALID);

  // the fetch-failure test hook: arguments only (nothing fetches here)
  CHECK(sekv_test_fail_fetch(-1) == SEKV_ERR_INVALID);
  CHECK(sekv_test_fail_fetch(2) == SEKV_OK);
  CHECK(sekv_test_fail_fetch(0) == SEKV_OK);

  // a long message is truncated, never overrun
  CHECK(std::strlen(sekv_last_error()) < 4096);
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi host checks: all passed\n");
  return 0;
}
