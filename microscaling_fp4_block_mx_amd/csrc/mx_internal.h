// mx_internal.h - launchers shared by the C ABI (mx_api.cpp) and the kernels.
#ifndef MX_INTERNAL_H
#define MX_INTERNAL_H
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx.h"

// nitems = rows * k / 8 (one item = 8 elements = 4 code bytes); callers have
// validated shapes, alignment and aliasing.
hipError_t mxi_launch_quantize(const void *x, int bf16, int mode, int64_t nitems,
                               uint8_t *codes, uint8_t *scales, hipStream_t st);
hipError_t mxi_launch_fakequant(const void *x, int bf16, int mode, int64_t nitems, void *y,
                                hipStream_t st);
hipError_t mxi_launch_dequantize(const uint8_t *codes, const uint8_t *scales, int bf16,
                                 int64_t nitems, void *y, hipStream_t st);
// Doubles of partial-sum space an error launch over nitems items needs for
// its fastest grid (the workspace size).
size_t mxi_block_mse_partials(int64_t nitems);
// partial: the partial-sum space (partial_space doubles; a smaller space
// than mxi_block_mse_partials caps the grid, still correct as long as it
// holds the 2 * 2048 doubles of one sum group).
hipError_t mxi_launch_block_mse(const void *x, int bf16, const uint8_t *codes,
                                const uint8_t *scales, int64_t nitems, float *block_mse,
                                double *tensor_sums, double *partial, int64_t partial_space,
                                hipStream_t st);
// The library's fixed device scratch for block-error partial sums: its size
// in doubles (every launch's partials fit), and its address on device dev
// (looked up once per device).
size_t mxi_scratch_partials();
hipError_t mxi_scratch_address(int dev, double **out);
// Quantize plus, optionally, y (x's dtype), block MSE and tensor sums in
// one pass; partial sums as mxi_launch_block_mse (same count).
hipError_t mxi_launch_quantize_fused(const void *x, int bf16, int mode, int64_t nitems,
                                     uint8_t *codes, uint8_t *scales, void *y, float *block_mse,
                                     double *tensor_sums, double *partial, int64_t partial_space,
                                     hipStream_t st);
// MXFP8 (E4M3): codes are one byte per element.
hipError_t mxi_launch_quantize8(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                uint8_t *scales, hipStream_t st);
hipError_t mxi_launch_dequantize8(const uint8_t *codes, const uint8_t *scales, int bf16,
                                  int64_t nitems, void *y, hipStream_t st);
hipError_t mxi_launch_fakequant8(const void *x, int bf16, int64_t nitems, void *y,
                                 hipStream_t st);
// NVFP4 comparator (nitems = rows * k / 8, even).
size_t mxi_nvfp4_partials(int64_t nitems);
// y != NULL: fused fake-quant into y (codes, block_scales, tensor_scale unused).
hipError_t mxi_launch_quantize_nv(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                  uint8_t *block_scales, uint8_t *tensor_scale,
                                  uint32_t *partial, void *y, hipStream_t st);
hipError_t mxi_launch_dequantize_nv(const uint8_t *codes, const uint8_t *block_scales,
                                    const uint8_t *tensor_scale, int bf16, int64_t nitems, void *y,
                                    hipStream_t st);
// MBS-Static (nitems = rows * k / 8, a multiple of 16).
// y != NULL: fused fake-quant into y (codes, sub_scales, macro_mant unused).
hipError_t mxi_launch_quantize_mbs(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                   uint8_t *sub_scales, uint8_t *macro_mant, void *y,
                                   hipStream_t st);
hipError_t mxi_launch_dequantize_mbs(const uint8_t *codes, const uint8_t *sub_scales,
                                     const uint8_t *macro_mant, int bf16, int64_t nitems, void *y,
                                     hipStream_t st);
// Many tensors in one call: launches of at most MX_MULTI_MAX tensors of
// similar size (empty ones skipped); 60 descriptors are 1,920 bytes of
// kernel arguments.
#ifndef MX_MULTI_MAX
#define MX_MULTI_MAX 60
#endif
struct MxiTensor {
  const void *x;
  void *out;        // quantize: codes; fake-quant: y
  uint8_t *scales;  // quantize only
  int64_t nitems;   // rows * k / 8
};
hipError_t mxi_launch_multi(const MxiTensor *t, int count, int bf16, int mode, int fakequant,
                            hipStream_t st);
// Launch plan of a multi-tensor call (host only; see mx_kernels.hip). C
// linkage, so the host tests can check it without a GPU.
extern "C" int mxi_multi_plan(const int64_t *nitems, int count, int64_t tile, int max_per_launch, int *order,
                   int *first, int64_t *gx);
#endif
