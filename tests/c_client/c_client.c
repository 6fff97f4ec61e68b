/* c_client.c - a plain C99 caller of the MX library (test infrastructure).
 *
 * Uses only include/mx.h and the HIP runtime's C API: no Python, no torch.
 * It builds a ragged test tensor with special values, calls every entry
 * point on a stream of its own (error paths included), and writes the input
 * and every output to the file named by argv[1] as records
 *   name[32] (NUL-padded) | int64 byte count | bytes
 * for the test that checks them against the oracle. Exit status 0 only if
 * every call returned what it should.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mx.h"

#define ROWS 37
#define K 4224 /* a multiple of 128, so every format takes it */
#define N ((int64_t)ROWS * K)

static FILE *out;
static int failures;

#define HIPCHECK(call)                                                        \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,            \
              hipGetErrorString(e_));                                         \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

/* a call that must return `want` */
#define EXPECT(call, want)                                                    \
  do {                                                                        \
    mx_status_t s_ = (call);                                                  \
    if (s_ != (want)) {                                                       \
      fprintf(stderr, "%s:%d %s returned %s, expected %s (%s)\n", __FILE__,   \
              __LINE__, #call, mx_status_string(s_), mx_status_string(want),  \
              mx_last_error_detail());                                        \
      failures++;                                                             \
    }                                                                         \
  } while (0)
#define CHECK(call) EXPECT(call, MX_OK)

static void emit(const char *name, const void *host, int64_t nbytes) {
  char tag[32];
  memset(tag, 0, sizeof tag);
  strncpy(tag, name, sizeof tag - 1);
  fwrite(tag, 1, sizeof tag, out);
  fwrite(&nbytes, sizeof nbytes, 1, out);
  fwrite(host, 1, (size_t)nbytes, out);
}

/* copy a device buffer back and write it as one record */
static void emit_dev(const char *name, const void *dev, int64_t nbytes) {
  void *h = malloc((size_t)nbytes);
  HIPCHECK(hipMemcpy(h, dev, (size_t)nbytes, hipMemcpyDeviceToHost));
  emit(name, h, nbytes);
  free(h);
}

static void *dev_alloc(int64_t nbytes) {
  void *p = NULL;
  HIPCHECK(hipMalloc(&p, (size_t)nbytes));
  return p;
}

/* xorshift64* (Vigna), then uniform doubles in (0, 1) and Box-Muller normals */
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) {
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return ((double)((rng * 0x2545F4914F6CDD1Dull) >> 11) + 0.5) * 0x1.0p-53;
}
static double nrand(void) {
  return sqrt(-2.0 * log(urand())) * cos(6.283185307179586 * urand());
}

/* fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
    return 2;
  }
  out = fopen(argv[1], "wb");
  if (!out) {
    perror(argv[1]);
    return 2;
  }

  /* input: heavy-tailed values whose size varies per 32-element block, plus
   * special blocks in row 0 */
  float *x32 = malloc(N * sizeof(float));
  uint16_t *x16 = malloc(N * sizeof(uint16_t));
  for (int64_t b = 0; b < N / 32; b++) {
    const double size = exp(2.0 * nrand());
    for (int i = 0; i < 32; i++)
      x32[32 * b + i] = (float)(size * nrand() / sqrt(urand()));
  }
  x32[5] = NAN;                                    /* block 0: NaN */
  x32[40] = -INFINITY;                             /* block 1: -Inf */
  for (int i = 64; i < 96; i++) x32[i] = 0.0f;     /* block 2: zeros */
  x32[70] = -0.0f;
  for (int i = 96; i < 128; i++) x32[i] = (float)((i - 112) * 1e-41); /* block 3: subnormal */
  for (int i = 128; i < 160; i++) x32[i] = (i & 1 ? -3.0e38f : 1.0e38f); /* block 4: huge */
  for (int i = 160; i < 192; i++) x32[i] = 6.0f * (float)(i - 176) / 16.0f; /* block 5: on the grid */
  for (int64_t i = 0; i < N; i++) x16[i] = to_bf16(x32[i]);
  emit("x32", x32, N * 4);
  emit("x16", x16, N * 2);

  hipStream_t st;
  HIPCHECK(hipStreamCreate(&st));
  void *s = (void *)st;

  float *d_x32 = dev_alloc(N * 4);
  uint16_t *d_x16 = dev_alloc(N * 2);
  HIPCHECK(hipMemcpy(d_x32, x32, N * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_x16, x16, N * 2, hipMemcpyHostToDevice));
  uint8_t *d_codes = dev_alloc(N / 2), *d_scales = dev_alloc(N / 32);
  uint8_t *d_codes2 = dev_alloc(N / 2), *d_scales2 = dev_alloc(N / 32);
  uint16_t *d_y16 = dev_alloc(N * 2);
  float *d_y32 = dev_alloc(N * 4);
  float *d_bm = dev_alloc(N / 32 * 4);
  double *d_sums = dev_alloc(16);
  const size_t ws_bytes = mx_block_mse_workspace_size(ROWS, K);
  void *d_ws = dev_alloc((int64_t)ws_bytes);

  /* MXFP4 */
  CHECK(mx_quantize(d_x16, MX_BF16, ROWS, K, MX_SCALE_OCP, d_codes, d_scales, s));
  CHECK(mx_dequantize(d_codes, d_scales, ROWS, K, MX_BF16, d_y16, s));
  CHECK(mx_dequantize(d_codes, d_scales, ROWS, K, MX_F32, d_y32, s));
  CHECK(mx_block_mse(d_x16, MX_BF16, d_codes, d_scales, ROWS, K, d_bm, d_sums, d_ws, ws_bytes, s));
  HIPCHECK(hipStreamSynchronize(st));
  emit_dev("q_ocp_bf16.codes", d_codes, N / 2);
  emit_dev("q_ocp_bf16.scales", d_scales, N / 32);
  emit_dev("dq_ocp.bf16", d_y16, N * 2);
  emit_dev("dq_ocp.f32", d_y32, N * 4);
  emit_dev("mse_ocp_bf16.block", d_bm, N / 32 * 4);
  emit_dev("mse_ocp_bf16.sums", d_sums, 16);

  CHECK(mx_quantize(d_x16, MX_BF16, ROWS, K, MX_SCALE_OAS_NF, d_codes, d_scales, s));
  CHECK(mx_quantize(d_x32, MX_F32, ROWS, K, MX_SCALE_OAS, d_codes2, d_scales2, s));
  HIPCHECK(hipStreamSynchronize(st));
  emit_dev("q_oas_nf_bf16.codes", d_codes, N / 2);
  emit_dev("q_oas_nf_bf16.scales", d_scales, N / 32);
  emit_dev("q_oas_f32.codes", d_codes2, N / 2);
  emit_dev("q_oas_f32.scales", d_scales2, N / 32);

  /* fake-quant in place: y == x */
  HIPCHECK(hipMemcpyAsync(d_y16, d_x16, N * 2, hipMemcpyDeviceToDevice, st));
  CHECK(mx_fakequant(d_y16, MX_BF16, ROWS, K, MX_SCALE_OAS_BITS, d_y16, s));
  HIPCHECK(hipStreamSynchronize(st));
  emit_dev("fq_oas_bits_bf16", d_y16, N * 2);

  /* one pass, every output */
  CHECK(mx_quantize_fused(d_x32, MX_F32, ROWS, K, MX_SCALE_OCP, d_codes, d_scales, d_y32, d_bm,
                          d_sums, d_ws, ws_bytes, s));
  HIPCHECK(hipStreamSynchronize(st));
  emit_dev("fused_f32.codes", d_codes, N / 2);
  emit_dev("fused_f32.scales", d_scales, N / 32);
  emit_dev("fused_f32.y", d_y32, N * 4);
  emit_dev("fused_f32.block", d_bm, N / 32 * 4);
  emit_dev("fused_f32.sums", d_sums, 16);

  /* two row ranges as separate tensors in one call */
  {
    const int64_t r0 = 20;
    mx_tensor_t t[2];
    memset(t, 0, sizeof t);
    t[0].x = d_x16;
    t[0].codes = d_codes2;
    t[0].scales = d_scales2;
    t[0].rows = r0;
    t[0].k = K;
    t[1].x = d_x16 + r0 * K;
    t[1].codes = d_codes2 + r0 * K / 2;
    t[1].scales = d_scales2 + r0 * K / 32;
    t[1].rows = ROWS - r0;
    t[1].k = K;
    CHECK(mx_quantize_multi(t, 2, MX_BF16, MX_SCALE_OAS, s));
    HIPCHECK(hipStreamSynchronize(st));
    emit_dev("multi_oas_bf16.codes", d_codes2, N / 2);
    emit_dev("multi_oas_bf16.scales", d_scales2, N / 32);
  }

  /* MXFP8 */
  {
    uint8_t *d_c8 = dev_alloc(N);
    CHECK(mx_quantize_mxfp8(d_x16, MX_BF16, ROWS, K, d_c8, d_scales, s));
    HIPCHECK(hipStreamSynchronize(st));
    emit_dev("q8_bf16.codes", d_c8, N);
    emit_dev("q8_bf16.scales", d_scales, N / 32);
    HIPCHECK(hipFree(d_c8));
  }

  /* NVFP4 */
  {
    uint8_t *d_bs = dev_alloc(N / 16), *d_ts = dev_alloc(16);
    const size_t nv_bytes = mx_nvfp4_workspace_size(ROWS, K);
    void *d_wsn = dev_alloc((int64_t)nv_bytes);
    EXPECT(mx_quantize_nvfp4(d_x32, MX_F32, ROWS, K, d_codes, d_bs, d_ts, d_wsn, nv_bytes - 4, s),
           MX_ERR_WORKSPACE);
    CHECK(mx_quantize_nvfp4(d_x32, MX_F32, ROWS, K, d_codes, d_bs, d_ts, d_wsn, nv_bytes, s));
    HIPCHECK(hipStreamSynchronize(st));
    emit_dev("qnv_f32.codes", d_codes, N / 2);
    emit_dev("qnv_f32.block_scales", d_bs, N / 16);
    emit_dev("qnv_f32.tensor_scale", d_ts, 1);
    HIPCHECK(hipFree(d_bs));
    HIPCHECK(hipFree(d_ts));
    HIPCHECK(hipFree(d_wsn));
  }

  /* MBS-Static */
  {
    uint8_t *d_sub = dev_alloc(N / 16), *d_mac = dev_alloc(N / 128);
    CHECK(mx_quantize_mbs(d_x16, MX_BF16, ROWS, K, d_codes, d_sub, d_mac, s));
    CHECK(mx_fakequant_mbs(d_x32, MX_F32, ROWS, K, d_y32, s));
    HIPCHECK(hipStreamSynchronize(st));
    emit_dev("qmbs_bf16.codes", d_codes, N / 2);
    emit_dev("qmbs_bf16.sub_scales", d_sub, N / 16);
    emit_dev("qmbs_bf16.macro", d_mac, N / 128);
    emit_dev("fqmbs_f32", d_y32, N * 4);
    HIPCHECK(hipFree(d_sub));
    HIPCHECK(hipFree(d_mac));
  }

  /* error paths: each is refused on the host and launches nothing */
  EXPECT(mx_quantize(d_x16, MX_BF16, ROWS, 33, MX_SCALE_OCP, d_codes, d_scales, s), MX_ERR_SHAPE);
  EXPECT(mx_quantize(d_x16, MX_BF16, -1, K, MX_SCALE_OCP, d_codes, d_scales, s), MX_ERR_SHAPE);
  EXPECT(mx_quantize(d_x16, MX_BF16, ROWS, K, MX_SCALE_OCP, NULL, d_scales, s), MX_ERR_NULL);
  EXPECT(mx_quantize(d_x16 + 1, MX_BF16, ROWS, K, MX_SCALE_OCP, d_codes, d_scales, s),
         MX_ERR_ALIGN);
  EXPECT(mx_quantize(d_x16, (mx_dtype_t)7, ROWS, K, MX_SCALE_OCP, d_codes, d_scales, s),
         MX_ERR_DTYPE);
  EXPECT(mx_quantize(d_x16, MX_BF16, ROWS, K, (mx_scale_mode_t)9, d_codes, d_scales, s),
         MX_ERR_MODE);
  EXPECT(mx_fakequant(d_x16, MX_BF16, ROWS, K, MX_SCALE_OCP, d_x16 + 64, s), MX_ERR_ALIAS);
  EXPECT(mx_block_mse(d_x16, MX_BF16, d_codes, d_scales, ROWS, K, d_bm, d_sums, d_ws, 8, s),
         MX_ERR_WORKSPACE);
  EXPECT(mx_quantize(NULL, MX_BF16, 0, K, MX_SCALE_OCP, NULL, NULL, s), MX_OK);

  HIPCHECK(hipStreamSynchronize(st));
  HIPCHECK(hipStreamDestroy(st));
  void *bufs[] = {d_x32, d_x16, d_codes, d_scales, d_codes2, d_scales2, d_y16, d_y32, d_bm,
                  d_sums, d_ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++) HIPCHECK(hipFree(bufs[i]));
  free(x32);
  free(x16);
  fclose(out);
  printf("c client: %d failed call(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
