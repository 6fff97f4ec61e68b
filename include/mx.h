/* mx.h - C ABI of the MI355X (gfx950) MXFP4 block-quantization library.
 *
 * Format (OCP microscaling, MXFP4):
 *   - an MX block is 32 contiguous elements of the last dimension sharing one
 *     scale (vLLM MXFP8/MXFP4 page, "MXFP8: Block-32 scaling" section and MX
 *     format table; Axolotl MXFP4 PR page, section 2 fixes the block at 32);
 *   - the scale is E8M0, a power of two 2^(s-127) stored as one byte s; 255
 *     is NaN (vLLM page, MX format table; "Unveiling the Potential of
 *     Quantization with MXFP4", technical summary section 1);
 *   - each element is E2M1 (sign, 2 exponent bits, 1 mantissa bit; values
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6; Axolotl page section 2, "Unveiling..."
 *     section 2.A), two codes per byte, the even element in the low nibble
 *     (vLLM page, "MXFP4: 4-bit MoE" section gives the two-per-byte packing
 *     and the k/2 last dimension).
 *
 * Layout: every tensor is contiguous row-major; leading dimensions are
 * flattened into `rows` by the caller (the vLLM page makes the weight
 * contiguous before quantizing). For x/y of shape [rows, k]:
 *   codes  uint8 [rows, k/2]     scales  uint8 [rows, k/32]
 * k must be a positive multiple of 32 (vLLM page, MXFP8 section: the input
 * dimension must be a multiple of 32); the block size is not a parameter.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers, allocated and owned by the
 *     caller (scratch too: mx_block_mse takes a workspace argument); the
 *     library allocates no device memory and keeps no state between calls.
 *     It is safe to call from several host threads.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Arguments are validated synchronously on the host; on MX_OK the work
 *     has been enqueued on `stream` and completes asynchronously. A device
 *     fault surfaces at the caller's next synchronization.
 *   - rows == 0 returns MX_OK without reading or writing any tensor
 *     (pointers may then be NULL); only mx_block_mse still enqueues the
 *     write of 0 to tensor_sums.
 *   - x, y, codes and scales must be 16-byte aligned (MX_ERR_ALIGN).
 *   - Outputs must not overlap inputs, except that every fake-quant entry
 *     point accepts y == x exactly (in place). Partial overlap is
 *     MX_ERR_ALIAS.
 *   - On any error nothing is launched and no output is touched.
 */
#ifndef MX_H
#define MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,   /* a required pointer is NULL                          */
  MX_ERR_SHAPE = 2,  /* rows < 0, k <= 0, k not a multiple of the block, or rows*k overflows */
  MX_ERR_DTYPE = 3,  /* dtype is not MX_F32 / MX_BF16                        */
  MX_ERR_MODE = 4,   /* mode is not an mx_scale_mode_t value                 */
  MX_ERR_ALIGN = 5,  /* a data pointer is not 16-byte aligned                */
  MX_ERR_HIP = 6,    /* the HIP launch failed; see mx_last_error_detail()    */
  MX_ERR_ALIAS = 7,  /* an output partially overlaps an input                */
  MX_ERR_WORKSPACE = 8 /* workspace NULL, misaligned or below the size needed  */
} mx_status_t;

typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype_t;

typedef enum {
  /* OCP rule: s = floor(log2(amax)) - 2 + 127, clamped to [0, 254], so the
     block maximum lands in [4, 8) and values above 6 saturate; s = 255 when
     the block holds a NaN or an infinity. amax == 0 gives s = 0. */
  MX_SCALE_OCP = 0,
  /* Overflow-aware scaling ("Unveiling the Potential of Quantization with
     MXFP4", technical summary section 2.A: take a smaller scale and let the
     top values saturate when that lowers the error). With s0 the OCP byte,
     a block with s0 >= 1 takes s0 - 1 when its squared error at s0 - 1 is
     strictly smaller than at s0; ties keep s0. The squared error is computed
     in fp32, in units of the larger candidate's scale 2^(s0-127) (so the
     choice does not depend on the block's magnitude), in one fixed order:
     each element error is d = (x - x_hat) * 2^(127-s0), exact, rounded once
     to fp32; elements 8g..8g+7 form group g (g = 0..3); within a group one
     accumulator takes the even positions and one the odd positions, each
     acc = fma(d, d, acc); group = even + odd; total = (g0 + g1) + (g2 + g3). */
  MX_SCALE_OAS = 1,
  /* Overflow-aware scaling in the page's own form ("Unveiling...", technical
     summary section 2.A): start from the no-overflow byte s_nf, the smallest
     byte with amax / 2^(s_nf-127) <= 6; when that normalized maximum lies in
     (3, 3.5], take s_nf - 1, so it maps to (6, 7] and saturates at 6 with no
     more relative error than rounding at s_nf would give, while every smaller
     value gains a binade. This is a test on amax's mantissa bits: relative to
     the OCP byte it is s0 + 1 when amax / 2^(s0-127) > 7, else s0. */
  MX_SCALE_OAS_BITS = 2,
  /* Error-driven form around the no-overflow byte: the block takes s_nf - 1
     when its squared error (the fp32 arithmetic above, in units of
     2^(s_nf-127)) is strictly smaller than at s_nf; ties keep s_nf. */
  MX_SCALE_OAS_NF = 3
  /* In the two page modes the scale byte never exceeds 252, the largest byte
     at which every code decodes to a finite fp32/bf16 value. */
} mx_scale_mode_t;

/* Quantize x [rows, k] (fp32 or bf16) to packed E2M1 codes [rows, k/2] and
 * E8M0 scales [rows, k/32]. Each element is rounded to the nearest E2M1
 * value of x / 2^(s-127), ties to the even code, saturating at 6; the sign
 * is kept (so -0 and negative values that round to zero give code 0x8).
 * In a NaN/Inf block every code is the element's sign bit alone.
 * Source: vLLM MXFP8/MXFP4 page (online quantization after loading,
 * "MXFP8: Block-32 scaling" and "MXFP4: 4-bit MoE" sections). */
mx_status_t mx_quantize(const void *x, mx_dtype_t x_dtype, int64_t rows,
                        int64_t k, mx_scale_mode_t mode, uint8_t *codes,
                        uint8_t *scales, void *stream);

/* Dequantize codes [rows, k/2] and scales [rows, k/32] to y [rows, k] in
 * y_dtype: y = +-E2M1(code) * 2^(s-127), exact for s <= 252; s = 253, 254
 * may overflow to +-Inf; s = 255 gives the canonical quiet NaN (fp32
 * 0x7FC00000, bf16 0x7FC0) for every element of the block.
 * Source: vLLM MXFP8/MXFP4 page ("Why this design": bf16 weights converted
 * at load time and used in the low-precision format). */
mx_status_t mx_dequantize(const uint8_t *codes, const uint8_t *scales,
                          int64_t rows, int64_t k, mx_dtype_t y_dtype, void *y,
                          void *stream);

/* Fused quantize -> dequantize: y = dequantize(quantize(x, mode)) in x's
 * dtype, with nothing else written. y may equal x (in place).
 * Source: Axolotl MXFP4 PR page, sections 2-3 (fake-quantization of weights
 * and activations for quantization-aware training, block size 32). */
mx_status_t mx_fakequant(const void *x, mx_dtype_t dtype, int64_t rows,
                         int64_t k, mx_scale_mode_t mode, void *y,
                         void *stream);

/* Quantization error of x against (codes, scales): per block
 * SSE = sum_i (x_i - x_hat_i)^2 in fp64, with x_hat_i the value
 * mx_dequantize returns in x's dtype; block_mse[b] = (float)(SSE_b / 32).
 * tensor_sums (two device doubles, overwritten) receives
 *   tensor_sums[0] = sum of all block SSEs (tensor MSE = [0] / (rows * k)),
 *   tensor_sums[1] = sum of x_i^2 (QSNR = 10 log10([1] / [0]) dB),
 * both in fp64. Either output may be NULL (both NULL is MX_ERR_NULL).
 * block_mse must be 4-byte aligned and tensor_sums 8-byte aligned. Both
 * outputs are deterministic: the tensor sums are taken in a fixed order
 * (per-workgroup partial sums, then ordered sums of them in one or two
 * levels), never with atomics.
 * workspace: device scratch for those partial sums, needed only when
 * tensor_sums != NULL; at least mx_block_mse_workspace_size(rows, k) bytes,
 * 8-byte aligned, not overlapping any argument. Its contents on entry do not
 * matter; calls that share a workspace must be ordered (same stream).
 * Source: MXFP4 wiki page, example 2 (MSE as the quantization error);
 * "Unveiling..." section 2.B (block SSE as the objective) and sections 3-4
 * (QSNR). */
mx_status_t mx_block_mse(const void *x, mx_dtype_t x_dtype,
                         const uint8_t *codes, const uint8_t *scales,
                         int64_t rows, int64_t k, float *block_mse,
                         double *tensor_sums, void *workspace,
                         size_t workspace_bytes, void *stream);

/* mx_block_mse without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The partial sums behind tensor_sums live
 * in a fixed 32 KiB device array inside the library (2 x 2048 doubles); the
 * launch caps its grid at 2048 workgroups so that every shape fits (larger
 * tensors loop over their tiles, which is slower than mx_block_mse on
 * tensors above ~1.7e7 elements). Each GPU holds its own copy from the first
 * call on that GPU (the device of `stream`, or the current device for the
 * null stream) until the process ends. The call allocates nothing.
 * block_mse equals mx_block_mse's bit for bit; tensor_sums too up to
 * 16,777,216 elements (the same grid), and to a relative 1e-6 above (the
 * partial sums fall on other workgroups). Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents (nothing in it needs
 * clearing: a call writes each partial before reading it): calls that may
 * run at the same time on one GPU (unordered streams) race and can return
 * wrong tensor_sums, so order them on one stream. A call with
 * tensor_sums == NULL does not use the array. Other arguments, alignment,
 * aliasing and error conventions as mx_block_mse. */
mx_status_t mx_block_mse_noalloc(const void *x, mx_dtype_t x_dtype,
                                 const uint8_t *codes, const uint8_t *scales,
                                 int64_t rows, int64_t k, float *block_mse,
                                 double *tensor_sums, void *stream);

/* Bytes of workspace mx_block_mse (and mx_quantize_fused) needs for a
 * [rows, k] tensor when asked for tensor_sums: 16 bytes per 4096 elements
 * (one partial pair per workgroup), plus 16 bytes per 8192 of those pairs
 * when there are more than 8192 (a second summing level); e.g. 131,072
 * bytes for 8192 x 4096 and 11,011,392 bytes for 2.8e9 elements (0.4 % of a
 * bf16 input). 0 for an invalid shape. */
size_t mx_block_mse_workspace_size(int64_t rows, int64_t k);

/* One pass over x for the QAT / calibration loop that quantizes and then
 * measures what it lost (the MXFP4 wiki page's example 2 quantizes, then
 * dequantizes and reports the MSE): codes and scales as mx_quantize, plus,
 * when the pointers are not NULL, y [rows, k] in x's dtype as
 * mx_dequantize of those codes (= mx_fakequant), block_mse and tensor_sums
 * as mx_block_mse of those codes. x is read once instead of three times.
 * codes, scales, y and block_mse equal the separate calls bit for bit;
 * tensor_sums equal them to a relative 1e-6 (the summation order of the
 * partial sums may differ). Workspace, alignment and error conventions as
 * mx_quantize and mx_block_mse; no written range may overlap x, another
 * output or the workspace. */
mx_status_t mx_quantize_fused(const void *x, mx_dtype_t x_dtype, int64_t rows,
                              int64_t k, mx_scale_mode_t mode, uint8_t *codes,
                              uint8_t *scales, void *y, float *block_mse,
                              double *tensor_sums, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ---- MXFP8 (E4M3 elements) ------------------------------------------------
 * vLLM MXFP8/MXFP4 page, "MXFP8: Block-32 scaling" section: online MXFP8
 * quantization produces FP8 values plus one uint8 scale per 32 elements of
 * the (multiple-of-32) input dimension; MX format table: MXFP8 = E4M3 (or
 * E5M2) elements, block 32, E8M0 scale. Here: E4M3 ("fn": no infinities,
 * NaN = S.1111.111, largest magnitude 448), one code byte per element,
 * codes uint8 [rows, k], scales uint8 [rows, k/32]. Scale byte:
 * floor(log2 amax) - 8 + 127 (8 is the exponent of 448), clamped to
 * [0, 254]; 255 for a NaN/Inf block (codes = sign bit alone). Elements:
 * nearest E4M3 value of x / 2^(s-127), ties to the even code, saturating at
 * +-448. Decoding a NaN code (0x7F/0xFF) or scale byte 255 gives the
 * canonical quiet NaN; bf16 outputs are rounded to nearest even (values
 * below bf16's subnormal step occur at scale bytes 0..3). Same pointer,
 * alignment, aliasing and error conventions as the MXFP4 entry points. */
mx_status_t mx_quantize_mxfp8(const void *x, mx_dtype_t x_dtype, int64_t rows,
                              int64_t k, uint8_t *codes, uint8_t *scales,
                              void *stream);
mx_status_t mx_dequantize_mxfp8(const uint8_t *codes, const uint8_t *scales,
                                int64_t rows, int64_t k, mx_dtype_t y_dtype,
                                void *y, void *stream);
/* y = mx_dequantize_mxfp8(mx_quantize_mxfp8(x)) in x's dtype; y may equal x. */
mx_status_t mx_fakequant_mxfp8(const void *x, mx_dtype_t dtype, int64_t rows,
                               int64_t k, void *y, void *stream);

/* ---- NVFP4 comparator ---------------------------------------------------------
 * For comparisons with the format MXFP4 is measured against ("Unveiling the
 * Potential of Quantization with MXFP4", technical summary section 1: NVFP4
 * shares one scale per 16 elements, stored as E4M3). Elements E2M1, codes
 * uint8 [rows, k/2] (two per byte, even element low); block scales uint8
 * [rows, k/16] as E4M3 bytes; k must be a multiple of 16. A per-tensor
 * factor S = 2^t, the largest power of two with S * amax <= 6 * 448 (amax:
 * largest finite |x|; t = 0 when it is 0; t <= 127), keeps the block scales
 * inside E4M3; one device byte tensor_scale holds t + 127. Block scale:
 * E4M3 nearest-even of min((a_b / 6) * S, 448) (fp32 division by 6);
 * element: E2M1 nearest-even, saturating, of x * (S / s_b) in fp32 (the
 * factor by IEEE fp32 division; 0 when s_b is 0). Decoding gives
 * (E2M1 * s_b) / S exactly, then rounds to bf16 if asked. A block holding
 * NaN/Inf gets block scale 0x7F and sign-only codes and decodes to NaN.
 * Quantize reads x twice (tensor maximum, then the blocks) and needs a
 * workspace of mx_nvfp4_workspace_size(rows, k) bytes (4-byte aligned): one
 * 4-byte maximum per first-pass workgroup (at most 2048) and one word for
 * the tensor exponent, so 8,196 bytes cover every shape.
 * rows == 0 does nothing. Other conventions as above. */
size_t mx_nvfp4_workspace_size(int64_t rows, int64_t k);
/* y = mx_dequantize_nvfp4(mx_quantize_nvfp4(x)) in x's dtype, fused (x is
 * still read twice: the tensor maximum, then the blocks); y may equal x.
 * Same workspace as mx_quantize_nvfp4. For quantization-aware training
 * in this format, which the Axolotl MXFP4 QAT page's quantization-config
 * section lists beside MXFP4 (NVFP4 with a group size of 16). */
mx_status_t mx_fakequant_nvfp4(const void *x, mx_dtype_t dtype, int64_t rows,
                               int64_t k, void *y, void *workspace,
                               size_t workspace_bytes, void *stream);
mx_status_t mx_quantize_nvfp4(const void *x, mx_dtype_t x_dtype, int64_t rows,
                              int64_t k, uint8_t *codes, uint8_t *block_scales,
                              uint8_t *tensor_scale, void *workspace,
                              size_t workspace_bytes, void *stream);
mx_status_t mx_dequantize_nvfp4(const uint8_t *codes,
                                const uint8_t *block_scales,
                                const uint8_t *tensor_scale, int64_t rows,
                                int64_t k, mx_dtype_t y_dtype, void *y,
                                void *stream);

/* ---- MBS-Static ------------------------------------------------------------
 * "Unveiling the Potential of Quantization with MXFP4", technical summary
 * section 2.B (Macro Block Scaling): E2M1 elements with one E8M0 scale per
 * 16-element sub-block, corrected by an 8-bit mantissa factor per
 * 128-element macro block; k must be a multiple of 128. Layouts: codes
 * uint8 [rows, k/2] (two per byte, even element low), sub_scales uint8
 * [rows, k/16] (E8M0 bytes), macro_mant uint8 [rows, k/128]. Per macro
 * block with largest |x| a_M: m = the 8-bit mantissa of fl32(a_M / 6)
 * rounded to nearest even and capped at 255 (0 for a zero or non-finite
 * macro block, or where a_M / 6 underflows to zero); f = 1 + m/256;
 * y = fl32(x * fl32(1/f)). Each sub-block takes the OCP byte of its largest
 * |y| (floor(log2) - 2 + 127, clamped at 0) and the E2M1 codes of y at that
 * byte (nearest, ties even, saturating at 6); a sub-block holding NaN/Inf
 * gets byte 255 and the signs of x as codes. Decoding gives
 * E2M1 * 2^(s-127) * f exactly, rounded to bf16 if asked; byte 255 decodes
 * to the canonical quiet NaN. rows == 0 does nothing; same pointer,
 * alignment (all four arrays 16-byte aligned), aliasing and error
 * conventions as the MXFP4 entry points. */
mx_status_t mx_quantize_mbs(const void *x, mx_dtype_t x_dtype, int64_t rows,
                            int64_t k, uint8_t *codes, uint8_t *sub_scales,
                            uint8_t *macro_mant, void *stream);
/* y = mx_dequantize_mbs(mx_quantize_mbs(x)) in x's dtype, fused; y may
 * equal x. */
mx_status_t mx_fakequant_mbs(const void *x, mx_dtype_t dtype, int64_t rows,
                             int64_t k, void *y, void *stream);
mx_status_t mx_dequantize_mbs(const uint8_t *codes, const uint8_t *sub_scales,
                              const uint8_t *macro_mant, int64_t rows,
                              int64_t k, mx_dtype_t y_dtype, void *y,
                              void *stream);

/* ---- Many tensors in one call ---------------------------------------------
 * QAT fake-quantizes every Linear weight on each forward pass and a
 * converted checkpoint quantizes every one of them (Axolotl MXFP4 QAT page,
 * QATConfig section: weights of each Linear layer); vLLM's online path does
 * the same for each expert's weights ("MXFP4: 4-bit MoE" section). These
 * entry points take a list of separate tensors and cover them with a few
 * launches instead of one per tensor (tensors of similar size share one, at
 * most MX_MULTI_MAX = 60 per launch), with results identical to the
 * single-tensor calls.
 *
 * `tensors` is a HOST array of `count` descriptors, read during the call
 * only; every pointer inside is a device pointer, 16-byte aligned. All
 * tensors share `dtype` and `mode`; each has its own rows and k (k % 32 ==
 * 0; rows == 0 skips it). mx_quantize_multi uses x, codes [rows, k/2] and
 * scales [rows, k/32]; mx_fakequant_multi uses x and y [rows, k] (y may
 * equal x). No output may overlap another tensor's input or output
 * (inputs may be shared): MX_ERR_ALIAS. count == 0 does nothing; count < 0
 * is MX_ERR_SHAPE. On a per-tensor validation error nothing is launched and
 * mx_last_error_detail() names the tensor (for an overlap, one of the two).
 * Validation sorts the byte ranges: host cost O(count log count). */
typedef struct {
  const void *x;   /* input [rows, k] */
  void *y;         /* mx_fakequant_multi: output [rows, k]; else unused */
  uint8_t *codes;  /* mx_quantize_multi: [rows, k/2]; else unused */
  uint8_t *scales; /* mx_quantize_multi: [rows, k/32]; else unused */
  int64_t rows;
  int64_t k;
} mx_tensor_t;
mx_status_t mx_quantize_multi(const mx_tensor_t *tensors, int count,
                              mx_dtype_t dtype, mx_scale_mode_t mode,
                              void *stream);
mx_status_t mx_fakequant_multi(const mx_tensor_t *tensors, int count,
                               mx_dtype_t dtype, mx_scale_mode_t mode,
                               void *stream);

/* Error reporting of this interface (no operation of the method, so no
 * passage defines it): the pages describe no error conventions; these two
 * calls only report the mx_status_t values above. */

/* Static, human-readable name of a status code (never NULL; unknown values
 * give "unknown mx_status_t"). The string is owned by the library. */
const char *mx_status_string(mx_status_t s);

/* Detail of the calling thread's most recent failure that recorded one
 * ("" if none): the HIP error text of an MX_ERR_HIP, or which tensor of a
 * multi-tensor call failed validation. The string is owned by the library
 * and valid until that thread's next call. */
const char *mx_last_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* MX_H */
