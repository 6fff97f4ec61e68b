/* mxref.h - CPU oracle for OCP MXFP4 block quantization.
 *
 * TEST INFRASTRUCTURE. This is the plain, slow, scalar reference that the GPU
 * library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code, header, table or
 * constant with the GPU library, and includes nothing from it.
 *
 * All pointers are HOST pointers, caller-allocated. Layouts:
 *   x, y    [rows, k] row-major; dtype MXREF_F32 (float) or MXREF_BF16
 *           (uint16 bit patterns of bfloat16)
 *   codes   [rows, k/2] uint8, two E2M1 codes per byte, even element in
 *           the low nibble
 *   scales  [rows, k/32] uint8 E8M0 bytes (scale = 2^(byte-127), 255 = NaN)
 * `threads` splits rows over that many pthreads (<= 0 means 1).
 * Every function returns 0 on success, a negative value on a bad argument.
 */
#ifndef MXREF_H
#define MXREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MXREF_F32 = 0, MXREF_BF16 = 1 };
enum { MXREF_OCP = 0, MXREF_OAS = 1, MXREF_OAS_BITS = 2, MXREF_OAS_NF = 3 };

int mxref_quantize(const void *x, int dtype, int64_t rows, int64_t k, int mode,
                   uint8_t *codes, uint8_t *scales, int threads);
int mxref_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                     int64_t k, int dtype, void *y, int threads);
int mxref_fakequant(const void *x, int dtype, int64_t rows, int64_t k, int mode,
                    void *y, int threads);
/* block_mse may be NULL; tensor_sums (2 doubles: sum (x - x_hat)^2, sum x^2)
 * may be NULL. */
int mxref_block_mse(const void *x, int dtype, const uint8_t *codes,
                    const uint8_t *scales, int64_t rows, int64_t k,
                    float *block_mse, double *tensor_sums, int threads);

/* Single-block helpers exposed for the oracle's own pins. */
int mxref_ocp_scale(double amax);                 /* E8M0 byte of the OCP rule */
int mxref_encode(double x, int scale_byte);       /* 4-bit code of one element */
double mxref_decode(int code, int scale_byte);    /* exact value of one code   */
float mxref_oas_sse32(const double *x32, int c, int h); /* pinned fp32 SSE at c in units of 2^(h-127) */

/* MXFP8 with E4M3 elements: codes [rows, k] uint8 (one byte per element),
 * scales [rows, k/32] as above. OCP scale only. */
int mxref8_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                    uint8_t *scales, int threads);
int mxref8_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t k,
                      int dtype, void *y, int threads);
int mxref8_fakequant(const void *x, int dtype, int64_t rows, int64_t k, void *y, int threads);
int mxref8_scale(double amax);
int mxref8_encode(double x, int scale_byte);
double mxref8_decode(int code, int scale_byte);

/* NVFP4 comparator: 16-element blocks with E4M3 block scales and a per-tensor
 * power-of-two factor 2^t stored as the byte t + 127. codes [rows, k/2],
 * block_scales [rows, k/16] (E4M3 bytes), k % 16 == 0. Single-threaded. */
int mxrefnv_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                     uint8_t *block_scales, uint8_t *tensor_scale);
int mxrefnv_dequantize(const uint8_t *codes, const uint8_t *block_scales, int tensor_scale,
                       int64_t rows, int64_t k, int dtype, void *y);
int mxrefnv_tensor_exp(double amax);
double mxrefnv_decode(int code, int block_scale, int tensor_scale);

/* MBS-Static: 16-element E8M0 sub-blocks corrected by an 8-bit-mantissa
 * factor per 128-element macro block. codes [rows, k/2], sub_scales
 * [rows, k/16], macro_mant [rows, k/128]; k % 128 == 0. Single-threaded. */
int mxrefmbs_quantize(const void *x, int dtype, int64_t rows, int64_t k, uint8_t *codes,
                      uint8_t *sub_scales, uint8_t *macro_mant);
int mxrefmbs_dequantize(const uint8_t *codes, const uint8_t *sub_scales,
                        const uint8_t *macro_mant, int64_t rows, int64_t k, int dtype, void *y);
int mxrefmbs_macro_mantissa(double amax);

#ifdef __cplusplus
}
#endif
#endif
