// Host-only checks of liblla's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer over every host path of the library (argument
// validation, workspace and split planning, the token-eviction page rule,
// eq. (4) scalars, status strings).  No call here reaches a kernel launch: the
// pointers are never dereferenced because every call either plans only or
// fails validation first.  Exit status 0 and "host check OK" on success.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <set>
#include <string>
#include <thread>
#include <vector>

#include "lla.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static lla_dims dims(int T, int D, int H, int d, int rk, int rv, int variant = LLA_PER_HEAD,
                     int dtype = LLA_BF16) {
  lla_dims m;
  m.T = T; m.D = D; m.H = H; m.d_head = d; m.r_k = rk; m.r_v = rv;
  m.variant = variant; m.dtype = dtype; m.page_size = 16; m.rope_base = 10000.f;
  return m;
}

static void *const FAKE = (void *)0x1000;

static void check_planning() {
  const lla_dims shapes[] = {dims(4, 24, 16, 128, 16, 32), dims(4, 24, 16, 128, 96, 160),
                             dims(4, 1, 2, 64, 16, 32, LLA_PER_HEAD, LLA_F32),
                             dims(8, 4, 32, 128, 256, 256, LLA_2D), dims(4, 2, 8, 128, 32, 64)};
  const int ops[] = {LLA_OP_DECODE, LLA_OP_PREFILL, LLA_OP_WINDOW_DECODE, LLA_OP_DECOUPLED_DECODE,
                     LLA_OP_FULL_DECODE, LLA_OP_ENCODE, LLA_OP_RECONSTRUCT, LLA_OP_ROPE_KEY_APPEND, 99};
  const int batches[] = {0, 1, 3, 32, 768, 100000};
  const int ctxs[] = {-1, 0, 1, 15, 16, 17, 4096, 262144, 1 << 24};
  const int ns[] = {-1, 0, 1, 64, 260, 512};
  for (const lla_dims &m : shapes)
    for (int op : ops)
      for (int b : batches)
        for (int c : ctxs)
          for (int n : ns) {
            const size_t bytes = lla_workspace_bytes(&m, op, b, c, n);
            int32_t splits = -7, pps = -7;
            const int32_t rc = lla_attn_plan(&m, op, b, c, n, &splits, &pps);
            if (rc == LLA_OK) {
              CHECK(splits >= 1 && pps >= 1);
              CHECK(bytes >= 256);
              if (splits == 1) CHECK(bytes == 256);
              // every page of the longest context lies in some split
              if (op == LLA_OP_DECODE || op == LLA_OP_FULL_DECODE)
                CHECK((long long)splits * pps >= (c + 15) / 16);
            } else {
              CHECK(rc == LLA_ERR_UNSUPPORTED || rc == LLA_ERR_INVALID_ARG);
              CHECK(strlen(lla_last_error()) > 0);
            }
            lla_supported(&m, op);
          }
  CHECK(lla_workspace_bytes(nullptr, LLA_OP_DECODE, 1, 16, 0) == 0);
  int32_t s, p;
  CHECK(lla_attn_plan(nullptr, LLA_OP_DECODE, 1, 16, 0, &s, &p) == LLA_ERR_INVALID_ARG);
  const lla_dims m = dims(4, 24, 16, 128, 16, 32);
  CHECK(lla_attn_plan(&m, LLA_OP_DECODE, 1, 16, 0, nullptr, &p) == LLA_ERR_INVALID_ARG);
}

// The windowed decode reads exactly the pages that hold a retained token.
static void check_window_pages() {
  const int sinks[] = {0, 1, 4, 16, 17, 225, 1000};
  const int windows[] = {0, 1, 15, 16, 256, 4000};
  for (int ctx = 0; ctx <= 1200; ctx += (ctx < 80 ? 1 : 37))
    for (int sk : sinks)
      for (int wi : windows) {
        int32_t na = -1, pb = -1;
        const int32_t rc = lla_window_pages(ctx, sk, wi, &na, &pb);
        if (sk + wi < 1) {
          CHECK(rc == LLA_ERR_INVALID_ARG);
          continue;
        }
        CHECK(rc == LLA_OK);
        std::set<int> want;
        for (int j = 0; j < ctx; ++j)
          if (j < sk || j >= ctx - wi) want.insert(j / 16);
        std::set<int> got;
        for (int v = 0; v < na; ++v) got.insert(v);
        for (int v = pb; v < (ctx + 15) / 16; ++v) got.insert(v);
        CHECK(got == want);
        CHECK((int)got.size() == na + (ctx + 15) / 16 - pb);  // no page twice
      }
  int32_t a, b;
  CHECK(lla_window_pages(-1, 4, 4, &a, &b) == LLA_ERR_INVALID_ARG);
  CHECK(lla_window_pages(10, 4, 4, nullptr, &b) == LLA_ERR_INVALID_ARG);
}

static void check_validation() {
  const lla_dims m = dims(4, 24, 16, 128, 16, 32);
  lla_dims bad = m;
  bad.page_size = 8;
  const lla_codec codec = {FAKE, FAKE, FAKE, FAKE, FAKE, FAKE};
  const lla_codec nocodec = {FAKE, nullptr, FAKE, FAKE, FAKE, FAKE};
  const lla_cache cache = {FAKE, FAKE, (const int32_t *)FAKE, 32, 256, 8192};
  const lla_cache nocache = {FAKE, FAKE, nullptr, 32, 256, 8192};
  const float *rope = (const float *)FAKE;
  const int32_t *ip = (const int32_t *)FAKE;
  int32_t *err = (int32_t *)FAKE;
  // each call fails on the host before anything is enqueued
  CHECK(lla_decode_attn(&bad, &codec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 4096, 0.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &nocodec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 4096, 0.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &codec, &nocache, rope, 4096, 0, 0, FAKE, ip, ip, 4096, 0.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &codec, &cache, rope, 4096, 24, 0, FAKE, ip, ip, 4096, 0.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &codec, &cache, rope, 4096, 0, 4, FAKE, ip, ip, 4096, 0.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &codec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 4097, 0.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &codec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 4096, -1.f, FAKE, FAKE, 1 << 30,
                        nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_decode_attn(&m, &codec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 4096, 0.f, FAKE, FAKE, 16,
                        nullptr) == LLA_ERR_WORKSPACE);
  CHECK(lla_decode_attn_noalloc(&m, &codec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 4096, 0.f, FAKE, nullptr,
                                nullptr) == LLA_ERR_INVALID_ARG);
  const lla_cache huge = {FAKE, FAKE, (const int32_t *)FAKE, 768, 1 << 16, 1 << 24};
  CHECK(lla_decode_attn_noalloc(&m, &codec, &huge, rope, 1 << 20, 0, 0, FAKE, ip, ip, 1 << 20, 0.f, FAKE, err,
                                nullptr) == LLA_ERR_WORKSPACE);
  CHECK(lla_decode_window_attn(&m, &codec, &cache, rope, 4096, 0, 0, FAKE, ip, ip, 0, 0, 4096, 0.f, FAKE, FAKE,
                               1 << 30, nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_prefill_attn(&m, &codec, &cache, rope, 4096, 0, 0, -1, FAKE, ip, 4096, 0.f, FAKE, FAKE, 1 << 30,
                         nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_encode_append(&m, &codec, &cache, FAKE, FAKE, ip, 1, 20, 5, FAKE, 1 << 30, nullptr) ==
        LLA_ERR_INVALID_ARG);
  CHECK(lla_encode_append(&m, &codec, &cache, FAKE, FAKE, ip, 1, 0, 1, FAKE, 16, nullptr) == LLA_ERR_WORKSPACE);
  CHECK(lla_reconstruct_kv(&m, &codec, &cache, rope, 4096, 0, 0, ip, 4096, nullptr, FAKE, FAKE, 1 << 30,
                           nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_full_decode_attn(&m, &cache, FAKE, FAKE, rope, 4096, FAKE, ip, ip, 0, 0.f, FAKE, FAKE, 1 << 30,
                             nullptr) == LLA_ERR_INVALID_ARG);
  CHECK(lla_rope_key_append(&m, &cache, 3, FAKE, rope, 4096, FAKE, ip, 1, 0, 1, FAKE, 1 << 30, nullptr) ==
        LLA_ERR_INVALID_ARG);
  CHECK(lla_decoupled_decode_attn(&m, &codec, &cache, 64, FAKE, rope, 4096, 0, 0, FAKE, ip, ip, 4096, 0.f,
                                  FAKE, FAKE, 16, nullptr) == LLA_ERR_WORKSPACE);
  CHECK(lla_rope_table(&bad, 16, (float *)FAKE, nullptr) == LLA_ERR_INVALID_ARG);
  int64_t t = 0, l = 0;
  CHECK(lla_cache_scalars(&m, &t, &l) == LLA_OK && t == 2LL * 4 * 16 * 128 && l == 48LL * 16);
  CHECK(lla_cache_scalars(&m, nullptr, &l) == LLA_ERR_INVALID_ARG);
  for (int st = -5; st <= 1; ++st) CHECK(lla_status_string(st) != nullptr);
}

// The last-error message is thread-local: concurrent failing calls each see
// their own message.
static void check_threads() {
  std::vector<std::thread> pool;
  std::vector<int> ok(8, 0);
  for (int i = 0; i < 8; ++i)
    pool.emplace_back([i, &ok] {
      const lla_dims m = dims(4, 24, 16, 128, 16, 32);
      const lla_codec codec = {FAKE, FAKE, FAKE, FAKE, FAKE, FAKE};
      const lla_cache cache = {FAKE, FAKE, (const int32_t *)FAKE, 32, 256, 8192};
      int good = 1;
      for (int k = 0; k < 2000; ++k) {
        const bool ws = (i + k) % 2 == 0;
        const int32_t rc =
            lla_decode_attn(&m, &codec, &cache, (const float *)FAKE, 4096, ws ? 0 : 99, 0, FAKE,
                            (const int32_t *)FAKE, (const int32_t *)FAKE, 4096, 0.f, FAKE, FAKE, 16, nullptr);
        const std::string msg = lla_last_error();
        good &= ws ? (rc == LLA_ERR_WORKSPACE && msg.find("workspace") != std::string::npos)
                   : (rc == LLA_ERR_INVALID_ARG && msg.find("layer") != std::string::npos);
      }
      ok[i] = good;
    });
  for (auto &th : pool) th.join();
  for (int v : ok) CHECK(v == 1);
}

int main() {
  check_planning();
  check_window_pages();
  check_validation();
  check_threads();
  if (failures) {
    fprintf(stderr, "host check: %d failures\n", failures);
    return 1;
  }
  printf("host check OK\n");
  return 0;
}
