// Stand-ins for the kernel launchers and the one HIP runtime call the C ABI
// makes, so that mx_api.cpp can be built and exercised on the host alone
// (under AddressSanitizer, UndefinedBehaviorSanitizer or ThreadSanitizer).
// Every stub records its call; a launcher returns an error when the item
// count equals kFailItems, which drives the MX_ERR_HIP path.
#include <stdint.h>
#include <string.h>

#include "mx_internal.h"
#include "stubs.h"

thread_local StubCall g_last;
thread_local int g_calls = 0;

static hipError_t rec(const char *name, int64_t nitems, int bf16, int mode, const void *a,
                      const void *b, const void *c, const void *d) {
  g_last.name = name;
  g_last.nitems = nitems;
  g_last.bf16 = bf16;
  g_last.mode = mode;
  g_last.p[0] = a;
  g_last.p[1] = b;
  g_last.p[2] = c;
  g_last.p[3] = d;
  g_calls++;
  return nitems == kFailItems ? hipErrorInvalidValue : hipSuccess;
}

extern "C" const char *hipGetErrorString(hipError_t) { return "stubbed launch failure"; }

hipError_t mxi_launch_quantize(const void *x, int bf16, int mode, int64_t n, uint8_t *c,
                               uint8_t *s, hipStream_t) {
  return rec("quantize", n, bf16, mode, x, c, s, nullptr);
}
hipError_t mxi_launch_fakequant(const void *x, int bf16, int mode, int64_t n, void *y,
                                hipStream_t) {
  return rec("fakequant", n, bf16, mode, x, y, nullptr, nullptr);
}
hipError_t mxi_launch_dequantize(const uint8_t *c, const uint8_t *s, int bf16, int64_t n, void *y,
                                 hipStream_t) {
  return rec("dequantize", n, bf16, -1, c, s, y, nullptr);
}
size_t mxi_block_mse_partials(int64_t n) {  // one pair per 512 items, a second level past 8192
  int64_t g = n > 0 ? (n + 511) / 512 : 1;
  if (g > 8192LL * 8192) g = 8192LL * 8192;
  return 2 * (size_t)(g + (g > 8192 ? (g + 8191) / 8192 : 0));
}
hipError_t mxi_launch_block_mse(const void *x, int bf16, const uint8_t *c, const uint8_t *s,
                                int64_t n, float *bm, double *sums, double *part,
                                int64_t space, hipStream_t) {
  g_last.p[4] = sums;
  g_last.p[5] = part;
  g_last.space = space;
  return rec("block_mse", n, bf16, -1, x, c, s, bm);
}
hipError_t mxi_launch_quantize_fused(const void *x, int bf16, int mode, int64_t n, uint8_t *c,
                                     uint8_t *s, void *y, float *bm, double *sums, double *part,
                                     int64_t space, hipStream_t) {
  g_last.p[4] = sums;
  g_last.p[5] = part;
  g_last.space = space;
  return rec(y ? "quantize_fused_y" : "quantize_fused", n, bf16, mode, x, c, s, bm);
}
size_t mxi_scratch_partials() { return 4096; }
hipError_t mxi_scratch_address(int dev, double **out) {
  *out = static_cast<double *>(const_cast<void *>(stub_scratch(dev)));
  return hipSuccess;
}
// the device of a stream: device 1 for any non-null stream in these tests
extern "C" hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *d) {
  *d = 1;
  return hipSuccess;
}
hipError_t mxi_launch_quantize8(const void *x, int bf16, int64_t n, uint8_t *c, uint8_t *s,
                                hipStream_t) {
  return rec("quantize8", n, bf16, -1, x, c, s, nullptr);
}
hipError_t mxi_launch_dequantize8(const uint8_t *c, const uint8_t *s, int bf16, int64_t n, void *y,
                                  hipStream_t) {
  return rec("dequantize8", n, bf16, -1, c, s, y, nullptr);
}
hipError_t mxi_launch_fakequant8(const void *x, int bf16, int64_t n, void *y, hipStream_t) {
  return rec("fakequant8", n, bf16, -1, x, y, nullptr, nullptr);
}
size_t mxi_nvfp4_partials(int64_t n) { return n > 0 ? (size_t)((n + 1023) / 1024 > 2048 ? 2048 : (n + 1023) / 1024) : 1; }
hipError_t mxi_launch_quantize_nv(const void *x, int bf16, int64_t n, uint8_t *c, uint8_t *bs,
                                  uint8_t *ts, uint32_t *part, void *y, hipStream_t) {
  g_last.p[4] = ts;
  g_last.p[5] = part;
  return rec(y ? "fakequant_nv" : "quantize_nv", n, bf16, -1, x, y ? y : (const void *)c, bs,
             nullptr);
}
hipError_t mxi_launch_dequantize_nv(const uint8_t *c, const uint8_t *bs, const uint8_t *ts,
                                    int bf16, int64_t n, void *y, hipStream_t) {
  return rec("dequantize_nv", n, bf16, -1, c, bs, ts, y);
}
hipError_t mxi_launch_quantize_mbs(const void *x, int bf16, int64_t n, uint8_t *c, uint8_t *ss,
                                   uint8_t *mm, void *y, hipStream_t) {
  return rec(y ? "fakequant_mbs" : "quantize_mbs", n, bf16, -1, x, y ? y : (const void *)c, ss,
             mm);
}
hipError_t mxi_launch_dequantize_mbs(const uint8_t *c, const uint8_t *ss, const uint8_t *mm,
                                     int bf16, int64_t n, void *y, hipStream_t) {
  return rec("dequantize_mbs", n, bf16, -1, c, ss, mm, y);
}
hipError_t mxi_launch_multi(const MxiTensor *t, int count, int bf16, int mode, int fakequant,
                            hipStream_t) {
  int64_t total = 0;
  for (int i = 0; i < count; i++) total += t[i].nitems;  // reads every descriptor
  g_last.p[4] = t;
  g_last.p[5] = reinterpret_cast<const void *>(static_cast<intptr_t>(count));
  return rec(fakequant ? "fakequant_multi" : "quantize_multi", total, bf16, mode, t[0].x,
             t[0].out, t[0].scales, nullptr);
}
