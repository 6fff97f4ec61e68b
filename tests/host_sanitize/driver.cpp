// Host-only exercise of the C ABI (mx_api.cpp) against recording launcher
// stubs: every entry point's accepted calls reach the right launcher with
// the right item count, dtype, mode and pointers; rejected calls reach none;
// a failing launch turns into MX_ERR_HIP with a per-thread detail string.
// Built and run under sanitizers by tests/test_host_sanitizers.py.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <thread>

#include "mx.h"
#include "stubs.h"

static int g_fail = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #c); \
      g_fail++;                                                     \
    }                                                               \
  } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }
static const uintptr_t X = 1ull << 32, Cd = 2ull << 32, Sc = 3ull << 32, Y = 4ull << 32,
                       Ws = 5ull << 32, Ts = 6ull << 32;

// an accepted call: exactly one launch, of `name`, with `nitems`
static void expect_launch(mx_status_t st, const char *name, int64_t nitems, int before) {
  CHECK(st == MX_OK);
  CHECK(g_calls == before + 1);
  CHECK(g_last.name && strcmp(g_last.name, name) == 0);
  CHECK(g_last.nitems == nitems);
}

static void mxfp4() {
  int n0 = g_calls;
  expect_launch(mx_quantize(P(X), MX_BF16, 64, 4096, MX_SCALE_OAS_NF, (uint8_t *)P(Cd),
                            (uint8_t *)P(Sc), nullptr),
                "quantize", 64 * 4096 / 8, n0);
  CHECK(g_last.bf16 == 1 && g_last.mode == MX_SCALE_OAS_NF && g_last.p[0] == P(X) &&
        g_last.p[1] == P(Cd) && g_last.p[2] == P(Sc));
  n0 = g_calls;
  expect_launch(mx_dequantize((uint8_t *)P(Cd), (uint8_t *)P(Sc), 3, 96, MX_F32, P(Y), nullptr),
                "dequantize", 3 * 96 / 8, n0);
  CHECK(g_last.bf16 == 0 && g_last.p[2] == P(Y));
  n0 = g_calls;
  expect_launch(mx_fakequant(P(X), MX_F32, 5, 32, MX_SCALE_OCP, P(X), nullptr), "fakequant",
                5 * 32 / 8, n0);  // in place is allowed
  n0 = g_calls;
  const size_t wsb = mx_block_mse_workspace_size(1000, 4096);
  CHECK(wsb >= 16 && wsb % 8 == 0);
  expect_launch(mx_block_mse(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 1000, 4096,
                             (float *)P(Y), (double *)P(Ts), P(Ws), wsb, nullptr),
                "block_mse", 1000 * 4096 / 8, n0);
  CHECK(g_last.p[4] == P(Ts) && g_last.p[5] == P(Ws) && g_last.space == (int64_t)(wsb / 8));
  // the call without a workspace: its partial sums go to the fixed scratch
  // of the stream's device (the current device for the null stream)
  n0 = g_calls;
  expect_launch(mx_block_mse_noalloc(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 1000,
                                     4096, (float *)P(Y), (double *)P(Ts), nullptr),
                "block_mse", 1000 * 4096 / 8, n0);
  CHECK(g_last.p[4] == P(Ts) && g_last.p[5] == stub_scratch(0) && g_last.space == 4096);
  n0 = g_calls;
  expect_launch(mx_block_mse_noalloc(P(X), MX_F32, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 8, 64,
                                     nullptr, (double *)P(Ts), P(Ws)),
                "block_mse", 8 * 64 / 8, n0);
  CHECK(g_last.p[5] == stub_scratch(1) && g_last.bf16 == 0);
  n0 = g_calls;
  expect_launch(mx_block_mse_noalloc(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 8, 64,
                                     (float *)P(Y), nullptr, nullptr),
                "block_mse", 8 * 64 / 8, n0);
  CHECK(g_last.p[4] == nullptr && g_last.p[5] == nullptr);
  n0 = g_calls;
  expect_launch(mx_block_mse_noalloc(nullptr, MX_BF16, nullptr, nullptr, 0, 32, nullptr,
                                     (double *)P(Ts), nullptr),
                "block_mse", 0, n0);
  n0 = g_calls;
  CHECK(mx_block_mse_noalloc(nullptr, MX_BF16, nullptr, nullptr, 0, 32, (float *)P(Y), nullptr,
                             nullptr) == MX_OK);
  CHECK(mx_block_mse_noalloc(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 1, 48, nullptr,
                             (double *)P(Ts), nullptr) == MX_ERR_SHAPE);
  CHECK(mx_block_mse_noalloc(P(X + 4), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 1, 32, nullptr,
                             (double *)P(Ts), nullptr) == MX_ERR_ALIGN);
  CHECK(mx_block_mse_noalloc(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 4, 64, nullptr,
                             (double *)P(Cd + 8), nullptr) == MX_ERR_ALIAS);
  CHECK(g_calls == n0);
  n0 = g_calls;
  expect_launch(mx_quantize_fused(P(X), MX_BF16, 1000, 4096, MX_SCALE_OAS, (uint8_t *)P(Cd),
                                  (uint8_t *)P(Sc), P(Y), (float *)P(Ws + (1u << 24)),
                                  (double *)P(Ts), P(Ws), wsb, nullptr),
                "quantize_fused_y", 1000 * 4096 / 8, n0);
  CHECK(g_last.mode == MX_SCALE_OAS && g_last.p[4] == P(Ts) && g_last.p[5] == P(Ws));
  n0 = g_calls;
  expect_launch(mx_quantize_fused(P(X), MX_F32, 4, 64, MX_SCALE_OCP, (uint8_t *)P(Cd),
                                  (uint8_t *)P(Sc), nullptr, nullptr, nullptr, nullptr, 0, nullptr),
                "quantize_fused", 32, n0);
  CHECK(g_last.p[5] == nullptr);
  n0 = g_calls;
  CHECK(mx_quantize_fused(P(X), MX_BF16, 4, 64, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc),
                          P(Cd + 64), nullptr, nullptr, nullptr, 0, nullptr) == MX_ERR_ALIAS);
  CHECK(mx_quantize_fused(P(X), MX_BF16, 4, 64, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc),
                          P(Y), nullptr, (double *)P(Ts), P(Ws), 8, nullptr) == MX_ERR_WORKSPACE);
  CHECK(mx_quantize_fused(P(X), MX_BF16, 4, 64, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc),
                          P(Y), (float *)P(Y + 32), nullptr, nullptr, 0, nullptr) == MX_ERR_ALIAS);
  CHECK(mx_quantize_fused(P(X), MX_BF16, 4, 64, (mx_scale_mode_t)9, (uint8_t *)P(Cd),
                          (uint8_t *)P(Sc), nullptr, nullptr, nullptr, nullptr, 0, nullptr) == MX_ERR_MODE);
  CHECK(g_calls == n0);
  // rows == 0: nothing launched, except block_mse's zero write of the sums
  n0 = g_calls;
  CHECK(mx_quantize(nullptr, MX_BF16, 0, 32, MX_SCALE_OCP, nullptr, nullptr, nullptr) == MX_OK);
  CHECK(mx_dequantize(nullptr, nullptr, 0, 32, MX_F32, nullptr, nullptr) == MX_OK);
  CHECK(g_calls == n0);
  expect_launch(mx_block_mse(nullptr, MX_BF16, nullptr, nullptr, 0, 32, nullptr, (double *)P(Ts),
                             P(Ws), 16, nullptr),
                "block_mse", 0, n0);
  // rejected calls launch nothing
  n0 = g_calls;
  CHECK(mx_quantize(P(X), MX_BF16, 1, 48, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_SHAPE);
  CHECK(mx_quantize(P(X), MX_BF16, INT64_MAX, 32, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_SHAPE);
  CHECK(mx_quantize(P(X), MX_BF16, INT64_MAX / 2, INT64_MAX / 64 * 32, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_SHAPE);
  CHECK(mx_quantize(P(X), (mx_dtype_t)7, 1, 32, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_DTYPE);
  CHECK(mx_quantize(P(X), MX_BF16, 1, 32, (mx_scale_mode_t)4, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_MODE);
  CHECK(mx_quantize(P(X), MX_BF16, 1, 32, (mx_scale_mode_t)-1, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_MODE);
  CHECK(mx_quantize(P(X + 2), MX_BF16, 1, 32, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_ALIGN);
  CHECK(mx_quantize(P(X), MX_BF16, 4, 64, MX_SCALE_OCP, (uint8_t *)P(X + 64), (uint8_t *)P(Sc), nullptr) == MX_ERR_ALIAS);
  CHECK(mx_fakequant(P(X), MX_BF16, 4, 64, MX_SCALE_OCP, P(X + 16), nullptr) == MX_ERR_ALIAS);
  CHECK(mx_block_mse(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 1, 32, nullptr, nullptr, nullptr, 0, nullptr) == MX_ERR_NULL);
  CHECK(mx_block_mse(P(X), MX_BF16, (uint8_t *)P(Cd), (uint8_t *)P(Sc), 1, 32, nullptr, (double *)P(Ts), P(Ws), 8, nullptr) == MX_ERR_WORKSPACE);
  CHECK(g_calls == n0);
}

static void mxfp8_nvfp4_mbs() {
  int n0 = g_calls;
  expect_launch(mx_quantize_mxfp8(P(X), MX_F32, 7, 64, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr),
                "quantize8", 7 * 64 / 8, n0);
  n0 = g_calls;
  expect_launch(mx_dequantize_mxfp8((uint8_t *)P(Cd), (uint8_t *)P(Sc), 7, 64, MX_BF16, P(Y), nullptr),
                "dequantize8", 7 * 64 / 8, n0);
  n0 = g_calls;
  expect_launch(mx_fakequant_mxfp8(P(X), MX_BF16, 2, 32, P(Y), nullptr), "fakequant8", 8, n0);
  n0 = g_calls;
  const size_t nvb = mx_nvfp4_workspace_size(9, 48);
  CHECK(nvb >= 4 && nvb % 4 == 0);
  expect_launch(mx_quantize_nvfp4(P(X), MX_BF16, 9, 48, (uint8_t *)P(Cd), (uint8_t *)P(Sc),
                                  (uint8_t *)P(Ts), P(Ws), nvb, nullptr),
                "quantize_nv", 9 * 48 / 8, n0);
  CHECK(g_last.p[4] == P(Ts) && g_last.p[5] == P(Ws));
  n0 = g_calls;
  expect_launch(mx_dequantize_nvfp4((uint8_t *)P(Cd), (uint8_t *)P(Sc), (uint8_t *)P(Ts), 9, 48,
                                    MX_F32, P(Y), nullptr),
                "dequantize_nv", 9 * 48 / 8, n0);
  n0 = g_calls;
  expect_launch(mx_quantize_mbs(P(X), MX_F32, 3, 384, (uint8_t *)P(Cd), (uint8_t *)P(Sc),
                                (uint8_t *)P(Ts), nullptr),
                "quantize_mbs", 3 * 384 / 8, n0);
  CHECK(g_last.p[3] == P(Ts) && g_last.bf16 == 0);
  n0 = g_calls;
  expect_launch(mx_dequantize_mbs((uint8_t *)P(Cd), (uint8_t *)P(Sc), (uint8_t *)P(Ts), 3, 384,
                                  MX_BF16, P(Y), nullptr),
                "dequantize_mbs", 3 * 384 / 8, n0);
  n0 = g_calls;
  expect_launch(mx_fakequant_nvfp4(P(X), MX_BF16, 9, 48, P(Y), P(Ws), nvb, nullptr),
                "fakequant_nv", 9 * 48 / 8, n0);
  CHECK(g_last.p[1] == P(Y) && g_last.p[5] == P(Ws));
  n0 = g_calls;
  expect_launch(mx_fakequant_nvfp4(P(X), MX_F32, 9, 48, P(X), P(Ws), nvb, nullptr),
                "fakequant_nv", 9 * 48 / 8, n0);  // in place
  n0 = g_calls;
  expect_launch(mx_fakequant_mbs(P(X), MX_BF16, 2, 256, P(Y), nullptr), "fakequant_mbs", 64, n0);
  n0 = g_calls;
  CHECK(mx_fakequant_nvfp4(P(X), MX_BF16, 9, 48, P(X + 16), P(Ws), nvb, nullptr) == MX_ERR_ALIAS);
  CHECK(mx_fakequant_nvfp4(P(X), MX_BF16, 9, 48, P(Y), P(Y + 32), nvb, nullptr) == MX_ERR_ALIAS);
  CHECK(mx_fakequant_nvfp4(P(X), MX_BF16, 9, 48, P(Y), nullptr, 0, nullptr) == MX_ERR_WORKSPACE);
  CHECK(mx_fakequant_mbs(P(X), MX_BF16, 2, 192, P(Y), nullptr) == MX_ERR_SHAPE);
  CHECK(mx_fakequant_mbs(P(X), MX_BF16, 2, 256, P(X + 32), nullptr) == MX_ERR_ALIAS);
  CHECK(g_calls == n0);
  CHECK(mx_quantize_mbs(P(X), MX_F32, 3, 320, (uint8_t *)P(Cd), (uint8_t *)P(Sc), (uint8_t *)P(Ts), nullptr) == MX_ERR_SHAPE);
  CHECK(mx_quantize_nvfp4(P(X), MX_BF16, 9, 40, (uint8_t *)P(Cd), (uint8_t *)P(Sc), (uint8_t *)P(Ts), P(Ws), nvb, nullptr) == MX_ERR_SHAPE);
  CHECK(mx_quantize_nvfp4(P(X), MX_BF16, 9, 48, (uint8_t *)P(Cd), (uint8_t *)P(Sc), (uint8_t *)P(Ts), P(Ws + 2), nvb, nullptr) == MX_ERR_WORKSPACE);
  CHECK(g_calls == n0);
}

// many tensors in one call: empty ones are dropped, the rest reach the
// launcher in order; a bad tensor or a cross-tensor overlap launches nothing
static void multi() {
  mx_tensor_t t[5] = {};
  for (int i = 0; i < 5; i++) {
    t[i].x = P(X + (uintptr_t)i * (1u << 24));
    t[i].codes = (uint8_t *)P(Cd + (uintptr_t)i * (1u << 24));
    t[i].scales = (uint8_t *)P(Sc + (uintptr_t)i * (1u << 24));
    t[i].y = P(Y + (uintptr_t)i * (1u << 24));
    t[i].rows = 3 + i;
    t[i].k = 64;
  }
  t[2].rows = 0;
  int n0 = g_calls;
  int64_t items = 0;
  for (int i = 0; i < 5; i++) items += t[i].rows * t[i].k / 8;
  expect_launch(mx_quantize_multi(t, 5, MX_BF16, MX_SCALE_OAS, nullptr), "quantize_multi", items, n0);
  CHECK(g_last.p[5] == P(4) && g_last.mode == MX_SCALE_OAS);
  n0 = g_calls;
  expect_launch(mx_fakequant_multi(t, 5, MX_F32, MX_SCALE_OCP, nullptr), "fakequant_multi", items, n0);
  CHECK(g_last.bf16 == 0);
  n0 = g_calls;
  t[3].k = 40;
  CHECK(mx_quantize_multi(t, 5, MX_BF16, MX_SCALE_OCP, nullptr) == MX_ERR_SHAPE);
  CHECK(strcmp(mx_last_error_detail(), "tensor 3: shape") == 0);
  t[3].k = 64;
  t[4].codes = t[1].codes;  // two tensors writing the same codes
  CHECK(mx_quantize_multi(t, 5, MX_BF16, MX_SCALE_OCP, nullptr) == MX_ERR_ALIAS);
  t[4].codes = (uint8_t *)P(Cd + 4u * (1u << 24));
  t[4].y = const_cast<void *>(t[0].x);  // fake-quant output over another tensor's input
  CHECK(mx_fakequant_multi(t, 5, MX_BF16, MX_SCALE_OCP, nullptr) == MX_ERR_ALIAS);
  CHECK(mx_quantize_multi(nullptr, 3, MX_BF16, MX_SCALE_OCP, nullptr) == MX_ERR_NULL);
  CHECK(mx_quantize_multi(t, -2, MX_BF16, MX_SCALE_OCP, nullptr) == MX_ERR_SHAPE);
  CHECK(g_calls == n0);
  t[4].y = const_cast<void *>(t[4].x);  // in place is fine
  expect_launch(mx_fakequant_multi(t, 5, MX_BF16, MX_SCALE_OCP, nullptr), "fakequant_multi", items, n0);
  n0 = g_calls;
  t[4].x = t[0].x;  // two tensors may read one input, but not write over it
  t[4].y = const_cast<void *>(t[0].x);
  CHECK(mx_fakequant_multi(t, 5, MX_BF16, MX_SCALE_OCP, nullptr) == MX_ERR_ALIAS);
  t[4].y = P(Y + 4u * (1u << 24));
  expect_launch(mx_fakequant_multi(t, 5, MX_BF16, MX_SCALE_OCP, nullptr), "fakequant_multi", items, n0);
}

// the overlap rule against a brute-force check on random layouts: tensors
// of 32 elements (bf16: x and y 64 B, codes 16 B, scales 1 B, all at 16-byte
// steps) scattered over a small window so that ranges often collide
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (uint32_t)(g_rng % n);
}
static bool ov(uintptr_t a, int64_t na, uintptr_t b, int64_t nb) {
  return a < b + (uintptr_t)nb && b < a + (uintptr_t)na;
}
static void multi_random() {
  for (int trial = 0; trial < 4000; trial++) {
    const bool fq = trial & 1;
    const int n = 1 + (int)rnd(7);
    mx_tensor_t t[8] = {};
    for (int i = 0; i < n; i++) {
      t[i].rows = 1;
      t[i].k = 32;
      t[i].x = P(X + 16 * rnd(40));
      t[i].codes = (uint8_t *)P(X + 16 * rnd(40));
      t[i].scales = (uint8_t *)P(X + 16 * rnd(40));
      t[i].y = rnd(4) == 0 ? const_cast<void *>(t[i].x) : P(X + 16 * rnd(40));
    }
    // brute force: own ranges first (as the single-tensor calls), then every
    // output against every other tensor's ranges
    mx_status_t want = MX_OK;
    struct R { uintptr_t p; int64_t n; int o; bool out; } r[24];
    int nr = 0;
    for (int i = 0; i < n && want == MX_OK; i++) {
      const uintptr_t x = (uintptr_t)t[i].x;
      if (fq) {
        const uintptr_t y = (uintptr_t)t[i].y;
        if (x != y && ov(x, 64, y, 64)) want = MX_ERR_ALIAS;
        r[nr++] = {x, 64, i, false};
        r[nr++] = {y, 64, i, true};
      } else {
        const uintptr_t c = (uintptr_t)t[i].codes, sc = (uintptr_t)t[i].scales;
        if (ov(x, 64, c, 16) || ov(x, 64, sc, 1) || ov(c, 16, sc, 1)) want = MX_ERR_ALIAS;
        r[nr++] = {x, 64, i, false};
        r[nr++] = {c, 16, i, true};
        r[nr++] = {sc, 1, i, true};
      }
    }
    for (int a = 0; a < nr && want == MX_OK; a++)
      for (int b = 0; b < nr; b++)
        if (r[a].out && r[a].o != r[b].o && ov(r[a].p, r[a].n, r[b].p, r[b].n)) {
          want = MX_ERR_ALIAS;
          break;
        }
    const mx_status_t got = fq ? mx_fakequant_multi(t, n, MX_BF16, MX_SCALE_OCP, nullptr)
                               : mx_quantize_multi(t, n, MX_BF16, MX_SCALE_OCP, nullptr);
    if (got != want) {
      fprintf(stderr, "random layout %d (%s, %d tensors): got %d, want %d\n", trial,
              fq ? "fakequant" : "quantize", n, (int)got, (int)want);
      g_fail++;
      return;
    }
  }
}

// a failing launch reports MX_ERR_HIP; the detail string is per thread
static void hip_errors() {
  const int64_t k = 8 * kFailItems;  // one row whose item count makes the stub fail
  CHECK(mx_quantize(P(X), MX_BF16, 1, k, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr) == MX_ERR_HIP);
  CHECK(strcmp(mx_last_error_detail(), "stubbed launch failure") == 0);
  CHECK(mx_quantize_mbs(P(X), MX_BF16, 1, k, (uint8_t *)P(Cd), (uint8_t *)P(Sc), (uint8_t *)P(Ts), nullptr) == MX_ERR_HIP);
  bool other_clean = false;
  std::thread t([&] { other_clean = mx_last_error_detail()[0] == '\0'; });
  t.join();
  CHECK(other_clean);
  for (int s = 0; s <= 8; s++) CHECK(strncmp(mx_status_string((mx_status_t)s), "MX_", 3) == 0);
  CHECK(strstr(mx_status_string((mx_status_t)99), "unknown") != nullptr);
}

// many threads validating and launching at once (shared state would race)
static void threads() {
  std::thread ts[8];
  int bad[8] = {};
  for (int i = 0; i < 8; i++) {
    ts[i] = std::thread([i, &bad] {
      for (int r = 0; r < 2000; r++) {
        const bool fail = (r + i) % 3 == 0;
        const int64_t k = fail ? 8 * kFailItems : 32 * (1 + r % 7);
        const mx_status_t st = mx_quantize(P(X), MX_BF16, 1, k, MX_SCALE_OCP, (uint8_t *)P(Cd), (uint8_t *)P(Sc), nullptr);
        if (st != (fail ? MX_ERR_HIP : MX_OK)) bad[i]++;
        if (g_last.nitems != k / 8) bad[i]++;
      }
    });
  }
  for (auto &t : ts) t.join();
  for (int i = 0; i < 8; i++) CHECK(bad[i] == 0);
}

int main() {
  mxfp4();
  mxfp8_nvfp4_mbs();
  multi();
  multi_random();
  hip_errors();
  threads();
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
