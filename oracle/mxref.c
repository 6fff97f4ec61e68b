/* mxref.c - CPU oracle for OCP MXFP4 block quantization.
 *
 * TEST INFRASTRUCTURE. The plain, slow, scalar reference the GPU library is
 * checked against; only tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code with the GPU library.
 *
 * What it computes, and where the pages state it:
 *  - An MX block is 32 contiguous elements of the last dimension sharing one
 *    scale (vLLM MXFP8/MXFP4 page, "MXFP8: Block-32 scaling" section and the
 *    MX format table; Axolotl MXFP4 PR page, section 2: block size must be 32).
 *  - The scale is E8M0: a bare power of two stored in one byte (vLLM page, MX
 *    format table; "Unveiling the Potential of Quantization with MXFP4",
 *    technical summary section 1). The byte's bias is 127 and 255 is NaN
 *    (reading taken where the pages are silent).
 *  - The element is E2M1: sign, 2 exponent bits, 1 mantissa bit, largest
 *    magnitude 6.0 (Axolotl page, section 2; "Unveiling..." section 2.A).
 *  - Two 4-bit codes per byte, so a row of k elements packs to k/2 bytes
 *    (vLLM page, "MXFP4: 4-bit MoE" section). Even element in the low nibble
 *    (reading; the pages do not fix the order).
 *  - Scale exponent: floor(log2(amax)) - 2, so the block maximum lands in
 *    [4, 8) (the OCP rule; the pages only say the scale is 2^k).
 *  - Elements round to the nearest E2M1 value, ties to the even code,
 *    saturating at 6 (reading; the pages are silent on rounding).
 *  - Overflow-aware scaling ("Unveiling..." section 2.A): a block may take a
 *    scale one step smaller, letting its top values saturate, when that
 *    lowers the block's squared error (MXREF_OAS: around the OCP byte). The
 *    page's own form starts from the scale that maps the block maximum to at
 *    most 6 and halves it when the maximum lands in (3, 3.5] under that
 *    scale, a test on the maximum's mantissa bits (MXREF_OAS_BITS); the
 *    error-driven choice around that no-overflow scale is MXREF_OAS_NF.
 *  - Signal-to-noise of the quantization error (QSNR, "Unveiling..."
 *    sections 3-4): 10 log10(sum x^2 / sum (x - x_hat)^2); the oracle
 *    returns both sums.
 *  - Error measure: mean of squared differences (MXFP4 wiki page, example 2)
 *    and per-block sum of squared errors ("Unveiling..." section 2.B).
 *
 * Arithmetic is C double throughout (exact for every quantity here: x/2^k,
 * grid midpoints, decoded values), except the overflow-aware decision, which
 * both this oracle and the device take in float in one fixed order, with
 * each error measured in units of the larger candidate scale.
 * Build with -O2 -ffp-contract=off, never -ffast-math.
 */
#include "mxref.h"

#include <math.h>
#include <pthread.h>
#include <string.h>
#include <xmmintrin.h>

#define BLOCK 32

/* E2M1 magnitudes in code order 0..7: exponent field e (2 bits, bias 1) and
 * mantissa bit m give m*0.5 when e == 0, else 2^(e-1) * (1 + m/2). */
static const double kGrid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Denormals must be honoured on the host as on the device. */
static unsigned int enter_ieee(void) {
  unsigned int old = _mm_getcsr();
  _mm_setcsr(old & ~(0x8000u | 0x0040u)); /* clear FTZ and DAZ */
  return old;
}
static void leave_ieee(unsigned int old) { _mm_setcsr(old); }

static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static uint16_t float_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return 0x7FC0;
  /* round to nearest, ties to even, on the dropped 16 bits */
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static double load_elem(const void *x, int dtype, int64_t i) {
  if (dtype == MXREF_F32) return (double)((const float *)x)[i];
  return bf16_bits_to_double(((const uint16_t *)x)[i]);
}

static void store_elem(void *y, int dtype, int64_t i, double v) {
  float f = (float)v; /* exact for every decoded value below 2^128 */
  if (isnan(v)) {
    uint32_t q = 0x7FC00000u; /* canonical quiet NaN */
    memcpy(&f, &q, 4);
  }
  if (dtype == MXREF_F32)
    ((float *)y)[i] = f;
  else
    ((uint16_t *)y)[i] = float_to_bf16_bits(f);
}

/* OCP shared exponent: floor(log2 amax) - 2, biased by 127, clamped to the
 * finite E8M0 range [0, 254]. amax == 0 gives byte 0. */
int mxref_ocp_scale(double amax) {
  if (amax == 0.0) return 0;
  int e2;
  (void)frexp(amax, &e2); /* amax = f * 2^e2, f in [0.5, 1) */
  int floor_log2 = e2 - 1;
  int s = floor_log2 - 2 + 127;
  if (s < 0) s = 0;
  if (s > 254) s = 254;
  return s;
}

/* Nearest E2M1 value to |x| / 2^(s-127), ties to the even code, saturating. */
int mxref_encode(double x, int s) {
  int sign = signbit(x) ? 8 : 0;
  if (s == 255) return sign;
  double v = fabs(x) / ldexp(1.0, s - 127); /* exact: power-of-two divisor */
  int idx;
  if (v >= 6.0) {
    idx = 7;
  } else {
    int lo = 0;
    while (lo < 6 && kGrid[lo + 1] <= v) lo++;
    int hi = lo + 1;
    double mid = 0.5 * (kGrid[lo] + kGrid[hi]); /* exact: quarter multiples */
    if (v < mid)
      idx = lo;
    else if (v > mid)
      idx = hi;
    else
      idx = (lo % 2 == 0) ? lo : hi;
  }
  return sign | idx;
}

/* Exact value of code c at scale byte s; byte 255 decodes to NaN. */
double mxref_decode(int c, int s) {
  if (s == 255) return NAN;
  double mag = kGrid[c & 7] * ldexp(1.0, s - 127);
  return (c & 8) ? -mag : mag;
}

/* Block squared error at candidate byte c, in float, measured in units of
 * the larger candidate's scale 2^(h-127) (h >= c): each element's error is
 * d = (x - x_hat) * 2^(127-h), exact in double and rounded once to float, so
 * the comparison between the two candidates does not depend on the block's
 * magnitude (no overflow of d*d for huge blocks, no underflow for tiny ones).
 * The terms are summed in a fixed order: four groups of eight consecutive
 * elements; inside a group one accumulator takes the even positions and one
 * the odd positions, each by fused multiply-add; then group = even + odd,
 * total = (g0 + g1) + (g2 + g3). */
float mxref_oas_sse32(const double *xb, int c, int h) {
  const double unit = ldexp(1.0, 127 - h); /* exact power of two */
  float grp[4];
  for (int g = 0; g < 4; g++) {
    float acc_even = 0.0f, acc_odd = 0.0f;
    for (int t = 0; t < 4; t++) {
      int i = 8 * g + 2 * t;
      float d0 = (float)((xb[i] - mxref_decode(mxref_encode(xb[i], c), c)) * unit);
      float d1 = (float)((xb[i + 1] - mxref_decode(mxref_encode(xb[i + 1], c), c)) * unit);
      acc_even = fmaf(d0, d0, acc_even);
      acc_odd = fmaf(d1, d1, acc_odd);
    }
    grp[g] = acc_even + acc_odd;
  }
  return (grp[0] + grp[1]) + (grp[2] + grp[3]);
}

/* No-overflow byte: the smallest byte s >= 0 with amax / 2^(s-127) <= 6,
 * so no element saturates. Clamped to 252, the largest byte whose every code
 * decodes to a finite fp32/bf16 value. */
static int no_overflow_scale(double amax) {
  int s = 0;
  while (s < 252 && amax / ldexp(1.0, s - 127) > 6.0) s++;
  return s;
}

/* Scale byte of one block (xb holds its 32 values). */
static int block_scale(const double *xb, int mode) {
  double amax = 0.0;
  for (int i = 0; i < BLOCK; i++) {
    if (isnan(xb[i]) || isinf(xb[i])) return 255;
    double a = fabs(xb[i]);
    if (a > amax) amax = a;
  }
  if (mode == MXREF_OCP || mode == MXREF_OAS) {
    int s0 = mxref_ocp_scale(amax);
    if (mode == MXREF_OAS && s0 >= 1) {
      float sse_ocp = mxref_oas_sse32(xb, s0, s0);
      float sse_low = mxref_oas_sse32(xb, s0 - 1, s0);
      if (sse_low < sse_ocp) return s0 - 1; /* strict: a tie keeps the OCP byte */
    }
    return s0;
  }
  int snf = no_overflow_scale(amax);
  if (mode == MXREF_OAS_BITS) {
    /* the block maximum under the no-overflow scale lies in (3, 6]; in
       (3, 3.5] the doubled value (6, 7] overflows 6 with no more relative
       error than rounding at the larger scale, so the scale is halved */
    double v = amax / ldexp(1.0, snf - 127);
    if (snf >= 1 && v > 3.0 && v <= 3.5) return snf - 1;
    return snf;
  }
  /* MXREF_OAS_NF: the smaller of the two errors, ties keep snf */
  if (snf >= 1) {
    float sse_nf = mxref_oas_sse32(xb, snf, snf);
    float sse_low = mxref_oas_sse32(xb, snf - 1, snf);
    if (sse_low < sse_nf) return snf - 1;
  }
  return snf;
}

/* ---- row-parallel drivers ---------------------------------------------- */

typedef struct {
  int op; /* 0 quantize, 1 dequantize, 2 fakequant, 3 block_mse */
  const void *x;
  int dtype;
  int mode;
  int64_t k;
  const uint8_t *codes_in;
  const uint8_t *scales_in;
  uint8_t *codes;
  uint8_t *scales;
  void *y;
  float *block_mse;
  int64_t r0, r1;
  long double sse; /* per-thread partial of the tensor SSE */
  long double ssq; /* per-thread partial of the tensor sum of x^2 */
} job_t;

static void run_rows(job_t *j) {
  unsigned int csr = enter_ieee();
  const int64_t nb = j->k / BLOCK;
  double xb[BLOCK];
  j->sse = 0.0L;
  j->ssq = 0.0L;
  for (int64_t r = j->r0; r < j->r1; r++) {
    for (int64_t b = 0; b < nb; b++) {
      const int64_t e0 = r * j->k + b * BLOCK; /* first element of the block */
      const int64_t bi = r * nb + b;           /* block index */
      if (j->op == 0 || j->op == 2) {
        for (int i = 0; i < BLOCK; i++) xb[i] = load_elem(j->x, j->dtype, e0 + i);
        int s = block_scale(xb, j->mode);
        int code[BLOCK];
        for (int i = 0; i < BLOCK; i++) code[i] = mxref_encode(xb[i], s);
        if (j->op == 0) {
          for (int t = 0; t < BLOCK / 2; t++)
            j->codes[e0 / 2 + t] = (uint8_t)(code[2 * t] | (code[2 * t + 1] << 4));
          j->scales[bi] = (uint8_t)s;
        } else {
          for (int i = 0; i < BLOCK; i++)
            store_elem(j->y, j->dtype, e0 + i, mxref_decode(code[i], s));
        }
      } else {
        const int s = j->scales_in[bi];
        double sse = 0.0, ssq = 0.0;
        for (int i = 0; i < BLOCK; i++) {
          uint8_t byte = j->codes_in[(e0 + i) / 2];
          int c = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
          double q = mxref_decode(c, s);
          if (j->op == 1) {
            store_elem(j->y, j->dtype, e0 + i, q);
          } else {
            /* the reconstruction is the value a dequantize in x's dtype
               would return: round the exact value to float */
            double qf = isnan(q) ? q : (double)(float)q;
            double xv = load_elem(j->x, j->dtype, e0 + i);
            double d = xv - qf;
            sse += d * d;
            ssq += xv * xv;
          }
        }
        if (j->op == 3) {
          if (j->block_mse) j->block_mse[bi] = (float)(sse / BLOCK);
          j->sse += (long double)sse;
          j->ssq += (long double)ssq;
        }
      }
    }
  }
  leave_ieee(csr);
}

static void *thread_main(void *arg) {
  run_rows((job_t *)arg);
  return NULL;
}

#define MAX_THREADS 256

static int run(job_t proto, int64_t rows, int threads, long double *sse_out,
               long double *ssq_out) {
  if (threads < 1) threads = 1;
  if (threads > MAX_THREADS) threads = MAX_THREADS;
  if (threads > rows) threads = rows > 0 ? (int)rows : 1;
  job_t jobs[MAX_THREADS];
  pthread_t tid[MAX_THREADS];
  for (int t = 0; t < threads; t++) {
    jobs[t] = proto;
    jobs[t].r0 = rows * t / threads;
    jobs[t].r1 = rows * (t + 1) / threads;
  }
  if (threads == 1) {
    run_rows(&jobs[0]);
  } else {
    for (int t = 0; t < threads; t++)
      if (pthread_create(&tid[t], NULL, thread_main, &jobs[t]) != 0) return -9;
    for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
  }
  if (sse_out) {
    long double s = 0.0L, q = 0.0L;
    for (int t = 0; t < threads; t++) {
      s += jobs[t].sse;
      q += jobs[t].ssq;
    }
    *sse_out = s;
    if (ssq_out) *ssq_out = q;
  }
  return 0;
}

static int check_shape(int64_t rows, int64_t k) {
  if (rows < 0 || k <= 0 || k % BLOCK != 0) return -2;
  return 0;
}

int mxref_quantize(const void *x, int dtype, int64_t rows, int64_t k, int mode,
                   uint8_t *codes, uint8_t *scales, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (mode < MXREF_OCP || mode > MXREF_OAS_NF) return -4;
  if (rows == 0) return 0;
  if (!x || !codes || !scales) return -1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.op = 0; j.x = x; j.dtype = dtype; j.mode = mode; j.k = k;
  j.codes = codes; j.scales = scales;
  return run(j, rows, threads, NULL, NULL);
}

int mxref_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                     int64_t k, int dtype, void *y, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!codes || !scales || !y) return -1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.op = 1; j.dtype = dtype; j.k = k;
  j.codes_in = codes; j.scales_in = scales; j.y = y;
  return run(j, rows, threads, NULL, NULL);
}

int mxref_fakequant(const void *x, int dtype, int64_t rows, int64_t k, int mode,
                    void *y, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (mode < MXREF_OCP || mode > MXREF_OAS_NF) return -4;
  if (rows == 0) return 0;
  if (!x || !y) return -1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.op = 2; j.x = x; j.dtype = dtype; j.mode = mode; j.k = k; j.y = y;
  return run(j, rows, threads, NULL, NULL);
}

int mxref_block_mse(const void *x, int dtype, const uint8_t *codes,
                    const uint8_t *scales, int64_t rows, int64_t k,
                    float *block_mse, double *tensor_sums, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) {
    if (tensor_sums) tensor_sums[0] = tensor_sums[1] = 0.0;
    return 0;
  }
  if (!x || !codes || !scales) return -1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.op = 3; j.x = x; j.dtype = dtype; j.k = k;
  j.codes_in = codes; j.scales_in = scales; j.block_mse = block_mse;
  long double sse = 0.0L, ssq = 0.0L;
  int rc = run(j, rows, threads, &sse, &ssq);
  if (tensor_sums) {
    tensor_sums[0] = (double)sse;
    tensor_sums[1] = (double)ssq;
  }
  return rc;
}

/* ======================================================================
 * MXFP8 (E4M3 elements) - vLLM MXFP8/MXFP4 page, "MXFP8: Block-32 scaling"
 * section (online MXFP8 quantization: FP8 values plus one uint8 scale per
 * 32 elements) and the MX format table (MXFP8: E4M3/E5M2, block 32, E8M0).
 *  - E4M3 ("fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 *    0 is subnormal (m/8 * 2^-6); no infinities; exponent 15 with mantissa 7
 *    is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 *  - Scale: floor(log2 amax) - 8 (8 = exponent of 448), biased by 127 and
 *    clamped to [0, 254]; NaN/Inf blocks get 255 (as for MXFP4). The block
 *    maximum lands in [256, 512) and values above 448 saturate (reading: the
 *    same saturation as the FP4 elements).
 *  - Elements: nearest E4M3 value, ties to the even code; the sign is kept.
 *    NaN/Inf blocks: codes hold the sign bit alone, decode to NaN.
 * ====================================================================== */

/* Magnitude of E4M3 code c (0..126) from its fields. */
static double e4m3_value(int c) {
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 0) return ldexp((double)m / 8.0, -6);
  return ldexp(1.0 + (double)m / 8.0, e - 7);
}

int mxref8_scale(double amax) {
  if (amax == 0.0) return 0;
  int e2;
  (void)frexp(amax, &e2);
  int s = (e2 - 1) - 8 + 127;
  if (s < 0) s = 0;
  if (s > 254) s = 254;
  return s;
}

int mxref8_encode(double x, int s) {
  int sign = signbit(x) ? 0x80 : 0;
  if (s == 255) return sign;
  double v = fabs(x) / ldexp(1.0, s - 127);
  if (v >= 448.0) return sign | 0x7E;
  int lo = 0; /* largest code with value <= v */
  while (lo < 126 && e4m3_value(lo + 1) <= v) lo++;
  int hi = lo + 1;
  double mid = 0.5 * (e4m3_value(lo) + e4m3_value(hi)); /* exact in double */
  int c;
  if (v < mid)
    c = lo;
  else if (v > mid)
    c = hi;
  else
    c = (lo % 2 == 0) ? lo : hi;
  return sign | c;
}

/* Exact value of E4M3 code c at scale byte s; NaN for byte 255 or a NaN code. */
double mxref8_decode(int c, int s) {
  if (s == 255 || (c & 0x7F) == 0x7F) return NAN;
  double mag = e4m3_value(c & 0x7F) * ldexp(1.0, s - 127);
  return (c & 0x80) ? -mag : mag;
}

typedef struct {
  int op; /* 0 quantize, 1 dequantize, 2 fakequant */
  const void *x;
  int dtype;
  int64_t k;
  const uint8_t *codes_in, *scales_in;
  uint8_t *codes, *scales;
  void *y;
  int64_t r0, r1;
} job8_t;

static void *run8_rows(void *arg) {
  job8_t *j = (job8_t *)arg;
  unsigned int csr = enter_ieee();
  const int64_t nb = j->k / BLOCK;
  for (int64_t r = j->r0; r < j->r1; r++) {
    for (int64_t b = 0; b < nb; b++) {
      const int64_t e0 = r * j->k + b * BLOCK, bi = r * nb + b;
      if (j->op == 1) {
        int s = j->scales_in[bi];
        for (int i = 0; i < BLOCK; i++)
          store_elem(j->y, j->dtype, e0 + i, mxref8_decode(j->codes_in[e0 + i], s));
        continue;
      }
      double xb[BLOCK], amax = 0.0;
      int nonfinite = 0;
      for (int i = 0; i < BLOCK; i++) {
        xb[i] = load_elem(j->x, j->dtype, e0 + i);
        if (isnan(xb[i]) || isinf(xb[i])) nonfinite = 1;
        else if (fabs(xb[i]) > amax) amax = fabs(xb[i]);
      }
      int s = nonfinite ? 255 : mxref8_scale(amax);
      for (int i = 0; i < BLOCK; i++) {
        int c = mxref8_encode(xb[i], s);
        if (j->op == 0)
          j->codes[e0 + i] = (uint8_t)c;
        else
          store_elem(j->y, j->dtype, e0 + i, mxref8_decode(c, s));
      }
      if (j->op == 0) j->scales[bi] = (uint8_t)s;
    }
  }
  leave_ieee(csr);
  return NULL;
}

static int run8(job8_t proto, int64_t rows, int threads) {
  if (threads < 1) threads = 1;
  if (threads > MAX_THREADS) threads = MAX_THREADS;
  if (threads > rows) threads = rows > 0 ? (int)rows : 1;
  job8_t jobs[MAX_THREADS];
  pthread_t tid[MAX_THREADS];
  for (int t = 0; t < threads; t++) {
    jobs[t] = proto;
    jobs[t].r0 = rows * t / threads;
    jobs[t].r1 = rows * (t + 1) / threads;
  }
  if (threads == 1) {
    run8_rows(&jobs[0]);
    return 0;
  }
  for (int t = 0; t < threads; t++)
    if (pthread_create(&tid[t], NULL, run8_rows, &jobs[t]) != 0) return -9;
  for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
  return 0;
}

int mxref8_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                    uint8_t *scales, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!x || !codes || !scales) return -1;
  job8_t j;
  memset(&j, 0, sizeof j);
  j.op = 0; j.x = x; j.dtype = dtype; j.k = k; j.codes = codes; j.scales = scales;
  return run8(j, rows, threads);
}

int mxref8_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t k,
                      int dtype, void *y, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!codes || !scales || !y) return -1;
  job8_t j;
  memset(&j, 0, sizeof j);
  j.op = 1; j.dtype = dtype; j.k = k; j.codes_in = codes; j.scales_in = scales; j.y = y;
  return run8(j, rows, threads);
}

int mxref8_fakequant(const void *x, int dtype, int64_t rows, int64_t k, void *y, int threads) {
  if (check_shape(rows, k)) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!x || !y) return -1;
  job8_t j;
  memset(&j, 0, sizeof j);
  j.op = 2; j.x = x; j.dtype = dtype; j.k = k; j.y = y;
  return run8(j, rows, threads);
}

/* ======================================================================
 * NVFP4 comparator ("Unveiling the Potential of Quantization with MXFP4",
 * technical summary section 1: NVFP4 shares one scale per 16 elements and
 * stores it as E4M3, i.e. with mantissa bits; Axolotl MXFP4 PR page: NVFP4
 * uses group size 16). Readings where the pages stop:
 *  - elements E2M1 as for MXFP4, two codes per byte, even element low;
 *  - a per-tensor power of two S = 2^t, the largest with S * amax <= 6 * 448,
 *    keeps the block scales inside E4M3's range; it is stored as the byte
 *    t + 127 (clamped to [0, 254]); amax over finite elements, S = 1 if 0;
 *  - block scale: E4M3 nearest-even of min((a_b / 6) * S, 448) in fp32 (the
 *    division by 6 rounded to fp32 first);
 *  - element code: nearest-even E2M1 (saturating) of x * r_b in fp32 with
 *    r_b = S / s_b rounded to fp32 (0 when s_b == 0);
 *  - decode: (E2M1 value * s_b) / S, exact before the output rounding;
 *  - a block holding NaN/Inf gets block scale 0x7F (E4M3 NaN) and sign-only
 *    codes, and decodes to NaN.
 * ====================================================================== */

#define NVB 16

/* t of the tensor factor S = 2^t: the largest t with 2^t * amax <= 2688. */
int mxrefnv_tensor_exp(double amax) {
  if (amax == 0.0) return 0;
  int t = 127;
  while (t > -127 && ldexp(amax, t) > 2688.0) t--;
  return t;
}

/* E2M1 code of float v (already divided by the block scale): nearest, ties
 * to the even code, saturating; computed with the MXFP4 encoder at scale 1. */
static int e2m1_code(float v) { return mxref_encode((double)v, 127); }

static int e4m3_code_nonneg(float t) {
  double v = t;
  if (v >= 448.0) return 0x7E;
  int lo = 0;
  while (lo < 126 && e4m3_value(lo + 1) <= v) lo++;
  int hi = lo + 1;
  double mid = 0.5 * (e4m3_value(lo) + e4m3_value(hi));
  if (v < mid) return lo;
  if (v > mid) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

int mxrefnv_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                     uint8_t *block_scales, uint8_t *tensor_scale) {
  if (rows < 0 || k <= 0 || k % NVB != 0) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) {
    if (tensor_scale) *tensor_scale = 127;
    return 0;
  }
  if (!x || !codes || !block_scales || !tensor_scale) return -1;
  unsigned int csr = enter_ieee();
  const int64_t n = rows * k;
  double amax = 0.0;
  for (int64_t i = 0; i < n; i++) {
    double v = load_elem(x, dtype, i);
    if (!isnan(v) && !isinf(v) && fabs(v) > amax) amax = fabs(v);
  }
  int t = mxrefnv_tensor_exp(amax);
  *tensor_scale = (uint8_t)(t + 127);
  const float S = (float)ldexp(1.0, t);
  for (int64_t b = 0; b < n / NVB; b++) {
    double xb[NVB], ab = 0.0;
    int nonfinite = 0;
    for (int i = 0; i < NVB; i++) {
      xb[i] = load_elem(x, dtype, b * NVB + i);
      if (isnan(xb[i]) || isinf(xb[i])) nonfinite = 1;
      else if (fabs(xb[i]) > ab) ab = fabs(xb[i]);
    }
    int code[NVB];
    if (nonfinite) {
      block_scales[b] = 0x7F;
      for (int i = 0; i < NVB; i++) code[i] = signbit(xb[i]) ? 8 : 0;
    } else {
      float q6 = (float)ab / 6.0f; /* fp32 division */
      float tb = q6 * S;           /* exact: power of two, no overflow */
      int sc = e4m3_code_nonneg(tb);
      block_scales[b] = (uint8_t)sc;
      float sv = (float)e4m3_value(sc);
      float r = sv > 0.0f ? S / sv : 0.0f; /* fp32 division */
      for (int i = 0; i < NVB; i++) {
        float v = (float)xb[i] * r; /* fp32 multiply */
        code[i] = (signbit(xb[i]) ? 8 : 0) | (e2m1_code(fabsf(v)) & 7);
      }
    }
    for (int tt = 0; tt < NVB / 2; tt++)
      codes[b * (NVB / 2) + tt] = (uint8_t)(code[2 * tt] | (code[2 * tt + 1] << 4));
  }
  leave_ieee(csr);
  return 0;
}

double mxrefnv_decode(int code, int block_scale, int tensor_scale) {
  if ((block_scale & 0x7F) == 0x7F) return NAN;
  double v = kGrid[code & 7] * e4m3_value(block_scale & 0x7F) * ldexp(1.0, -(tensor_scale - 127));
  if (block_scale & 0x80) v = -v; /* sign of the scale byte (never set by the quantizer) */
  return (code & 8) ? -v : v;
}

int mxrefnv_dequantize(const uint8_t *codes, const uint8_t *block_scales, int tensor_scale,
                       int64_t rows, int64_t k, int dtype, void *y) {
  if (rows < 0 || k <= 0 || k % NVB != 0) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!codes || !block_scales || !y) return -1;
  unsigned int csr = enter_ieee();
  const int64_t n = rows * k;
  for (int64_t i = 0; i < n; i++) {
    uint8_t byte = codes[i / 2];
    int c = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    store_elem(y, dtype, i, mxrefnv_decode(c, block_scales[i / NVB], tensor_scale));
  }
  leave_ieee(csr);
  return 0;
}

/* ======================================================================
 * MBS-Static ("Unveiling the Potential of Quantization with MXFP4",
 * technical summary section 2.B): MXFP4 quantization on 16-element base
 * blocks, whose power-of-two scales are corrected by a high-precision
 * factor with an 8-bit mantissa shared by each 128-element macro block;
 * the static variant computes that factor by a cheap approximation.
 * Readings where the page stops:
 *  - macro factor f = 1 + m/256, m = the 8-bit mantissa of r = a_M / 6
 *    (a_M = largest |x| of the macro block, division in fp32), rounded to
 *    nearest even and capped at 255; m = 0 when a_M is 0 or not finite, or
 *    when a_M / 6 underflows to zero in fp32. It carries the part of a_M / 6
 *    that a power of two cannot.
 *  - y = fl32(x * fl32(1 / f)); each 16-element sub-block takes the OCP
 *    byte of its largest |y| (floor(log2) - 2 + 127, clamped; 255 if it
 *    holds NaN/Inf), and each element the E2M1 code of y at that byte.
 *  - decode: E2M1 * 2^(s-127) * f, exact before the output rounding.
 * Storage: codes [rows, k/2], sub-block bytes [rows, k/16], macro mantissas
 * [rows, k/128]; k % 128 == 0.
 * ====================================================================== */

int mxrefmbs_macro_mantissa(double amax) {
  if (amax == 0.0 || isnan(amax) || isinf(amax)) return 0;
  float r = (float)amax / 6.0f; /* fp32 division */
  if (r == 0.0f) return 0;      /* a_M / 6 underflows: no mantissa, factor 1 */
  int e;
  double f = 2.0 * frexp((double)r, &e); /* [1, 2), exact */
  double t = (f - 1.0) * 256.0;          /* exact */
  double m = nearbyint(t);               /* round half even (default mode) */
  if (m > 255.0) m = 255.0;
  return (int)m;
}

int mxrefmbs_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                      uint8_t *sub_scales, uint8_t *macro_mant) {
  if (rows < 0 || k <= 0 || k % 128 != 0) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!x || !codes || !sub_scales || !macro_mant) return -1;
  unsigned int csr = enter_ieee();
  const int64_t n = rows * k;
  for (int64_t M = 0; M < n / 128; M++) {
    double xm[128], aM = 0.0;
    int nonfinite_macro = 0;
    for (int i = 0; i < 128; i++) {
      xm[i] = load_elem(x, dtype, M * 128 + i);
      if (isnan(xm[i]) || isinf(xm[i])) nonfinite_macro = 1;
      else if (fabs(xm[i]) > aM) aM = fabs(xm[i]);
    }
    int m = nonfinite_macro ? 0 : mxrefmbs_macro_mantissa(aM);
    macro_mant[M] = (uint8_t)m;
    const float f = 1.0f + (float)m / 256.0f;
    const float inv = 1.0f / f; /* fp32 division */
    for (int j = 0; j < 8; j++) {
      float y[16];
      double ay = 0.0;
      int nonfinite = 0;
      for (int i = 0; i < 16; i++) {
        double v = xm[16 * j + i];
        if (isnan(v) || isinf(v)) nonfinite = 1;
        y[i] = (float)v * inv; /* fp32 multiply */
        if (!isnan(y[i]) && fabs((double)y[i]) > ay) ay = fabs((double)y[i]);
      }
      int s = nonfinite ? 255 : mxref_ocp_scale(ay);
      sub_scales[M * 8 + j] = (uint8_t)s;
      int c[16];
      for (int i = 0; i < 16; i++)  /* a NaN/Inf sub-block keeps the signs of x */
        c[i] = (s == 255) ? (signbit(xm[16 * j + i]) ? 8 : 0) : mxref_encode((double)y[i], s);
      for (int t = 0; t < 8; t++)
        codes[(M * 128 + 16 * j) / 2 + t] = (uint8_t)(c[2 * t] | (c[2 * t + 1] << 4));
    }
  }
  leave_ieee(csr);
  return 0;
}

int mxrefmbs_dequantize(const uint8_t *codes, const uint8_t *sub_scales,
                        const uint8_t *macro_mant, int64_t rows, int64_t k, int dtype, void *y) {
  if (rows < 0 || k <= 0 || k % 128 != 0) return -2;
  if (dtype != MXREF_F32 && dtype != MXREF_BF16) return -3;
  if (rows == 0) return 0;
  if (!codes || !sub_scales || !macro_mant || !y) return -1;
  unsigned int csr = enter_ieee();
  const int64_t n = rows * k;
  for (int64_t i = 0; i < n; i++) {
    uint8_t byte = codes[i / 2];
    int c = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    double f = 1.0 + macro_mant[i / 128] / 256.0;
    store_elem(y, dtype, i, mxref_decode(c, sub_scales[i / 16]) * f);
  }
  leave_ieee(csr);
  return 0;
}
