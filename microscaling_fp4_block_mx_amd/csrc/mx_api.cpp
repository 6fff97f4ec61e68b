// mx_api.cpp - C ABI of the MXFP4 library: synchronous host-side argument
// validation, then one asynchronous launch on the caller's stream.
// Every check here runs before any HIP call, so the error paths can be
// exercised on a machine without a GPU.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include <hip/hip_runtime.h>

#include "mx_internal.h"

namespace {

thread_local char g_detail[256] = "";

constexpr int64_t kBlock = 32;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mx_status_t check_shape(int64_t rows, int64_t k) {
  if (rows < 0 || k <= 0 || k % kBlock != 0) return MX_ERR_SHAPE;
  // rows * k elements, each up to 4 bytes wide, must be addressable.
  if (rows > 0 && k > (INT64_MAX / 8) / rows) return MX_ERR_SHAPE;
  return MX_OK;
}

mx_status_t check_shape_n(int64_t rows, int64_t k, int64_t multiple) {
  if (rows < 0 || k <= 0 || k % multiple != 0) return MX_ERR_SHAPE;
  if (rows > 0 && k > (INT64_MAX / 8) / rows) return MX_ERR_SHAPE;
  return MX_OK;
}
mx_status_t check_shape16(int64_t rows, int64_t k) { return check_shape_n(rows, k, 16); }

bool dtype_ok(int d) { return d == MX_F32 || d == MX_BF16; }
bool mode_ok(int m) { return m >= MX_SCALE_OCP && m <= MX_SCALE_OAS_NF; }
int64_t elem_bytes(int d) { return d == MX_F32 ? 4 : 2; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

mx_status_t finish(hipError_t e) {
  if (e == hipSuccess) return MX_OK;
  strncpy(g_detail, hipGetErrorString(e), sizeof g_detail - 1);
  g_detail[sizeof g_detail - 1] = 0;
  return MX_ERR_HIP;
}

}  // namespace

extern "C" {

mx_status_t mx_quantize(const void *x, mx_dtype_t x_dtype, int64_t rows, int64_t k,
                        mx_scale_mode_t mode, uint8_t *codes, uint8_t *scales, void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (!mode_ok(mode)) return MX_ERR_MODE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t nx = n * elem_bytes(x_dtype);
  if (overlap(x, nx, codes, n / 2) || overlap(x, nx, scales, n / kBlock) ||
      overlap(codes, n / 2, scales, n / kBlock))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize(x, x_dtype == MX_BF16, mode, n / 8, codes, scales,
                                    static_cast<hipStream_t>(stream)));
}

mx_status_t mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t k,
                          mx_dtype_t y_dtype, void *y, void *stream) {
  if (!dtype_ok(y_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!codes || !scales || !y) return MX_ERR_NULL;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t ny = n * elem_bytes(y_dtype);
  if (overlap(y, ny, codes, n / 2) || overlap(y, ny, scales, n / kBlock)) return MX_ERR_ALIAS;
  return finish(mxi_launch_dequantize(codes, scales, y_dtype == MX_BF16, n / 8, y,
                                      static_cast<hipStream_t>(stream)));
}

mx_status_t mx_fakequant(const void *x, mx_dtype_t dtype, int64_t rows, int64_t k,
                         mx_scale_mode_t mode, void *y, void *stream) {
  if (!dtype_ok(dtype)) return MX_ERR_DTYPE;
  if (!mode_ok(mode)) return MX_ERR_MODE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !y) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return MX_ERR_ALIGN;
  const int64_t nb = rows * k * elem_bytes(dtype);
  if (x != y && overlap(x, nb, y, nb)) return MX_ERR_ALIAS;
  return finish(mxi_launch_fakequant(x, dtype == MX_BF16, mode, rows * k / 8, y,
                                     static_cast<hipStream_t>(stream)));
}

size_t mx_block_mse_workspace_size(int64_t rows, int64_t k) {
  if (check_shape(rows, k) != MX_OK) return 0;
  const size_t n = mxi_block_mse_partials(rows * k / 8);
  return (n > 0 ? n : 1) * sizeof(double);
}

mx_status_t mx_block_mse(const void *x, mx_dtype_t x_dtype, const uint8_t *codes,
                         const uint8_t *scales, int64_t rows, int64_t k, float *block_mse,
                         double *tensor_sums, void *workspace, size_t workspace_bytes,
                         void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (!block_mse && !tensor_sums) return MX_ERR_NULL;
  if (tensor_sums) {
    if ((reinterpret_cast<uintptr_t>(tensor_sums) & 7u) != 0) return MX_ERR_ALIGN;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0 ||
        workspace_bytes < mx_block_mse_workspace_size(rows, k))
      return MX_ERR_WORKSPACE;
    if (overlap(tensor_sums, 16, workspace, (int64_t)workspace_bytes)) return MX_ERR_ALIAS;
  }
  if (rows == 0) {
    // an empty tensor has zero error; still a device write, so it is enqueued
    if (!tensor_sums) return MX_OK;
    return finish(mxi_launch_block_mse(nullptr, 0, nullptr, nullptr, 0, nullptr, tensor_sums,
                                       static_cast<double *>(workspace),
                                       (int64_t)(workspace_bytes / sizeof(double)),
                                       static_cast<hipStream_t>(stream)));
  }
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGN;
  if (block_mse && (reinterpret_cast<uintptr_t>(block_mse) & 3u) != 0) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t nx = n * elem_bytes(x_dtype);
  const int64_t nbm = 4 * (n / kBlock);
  if (block_mse && (overlap(block_mse, nbm, x, nx) || overlap(block_mse, nbm, codes, n / 2) ||
                    overlap(block_mse, nbm, scales, n / kBlock)))
    return MX_ERR_ALIAS;
  if (tensor_sums) {
    const int64_t nw = (int64_t)workspace_bytes;
    if (overlap(tensor_sums, 16, x, nx) || overlap(tensor_sums, 16, codes, n / 2) ||
        overlap(tensor_sums, 16, scales, n / kBlock) ||
        (block_mse && overlap(tensor_sums, 16, block_mse, nbm)) || overlap(workspace, nw, x, nx) ||
        overlap(workspace, nw, codes, n / 2) || overlap(workspace, nw, scales, n / kBlock) ||
        (block_mse && overlap(workspace, nw, block_mse, nbm)))
      return MX_ERR_ALIAS;
  }
  return finish(mxi_launch_block_mse(x, x_dtype == MX_BF16, codes, scales, n / 8, block_mse,
                                     tensor_sums, static_cast<double *>(workspace),
                                     (int64_t)(workspace_bytes / sizeof(double)),
                                     static_cast<hipStream_t>(stream)));
}

mx_status_t mx_block_mse_noalloc(const void *x, mx_dtype_t x_dtype, const uint8_t *codes,
                                 const uint8_t *scales, int64_t rows, int64_t k, float *block_mse,
                                 double *tensor_sums, void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (!block_mse && !tensor_sums) return MX_ERR_NULL;
  if (tensor_sums && (reinterpret_cast<uintptr_t>(tensor_sums) & 7u) != 0) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  if (rows > 0) {
    if (!x || !codes || !scales) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGN;
    if (block_mse && (reinterpret_cast<uintptr_t>(block_mse) & 3u) != 0) return MX_ERR_ALIGN;
    const int64_t nx = n * elem_bytes(x_dtype);
    const int64_t nbm = 4 * (n / kBlock);
    if (block_mse && (overlap(block_mse, nbm, x, nx) || overlap(block_mse, nbm, codes, n / 2) ||
                      overlap(block_mse, nbm, scales, n / kBlock)))
      return MX_ERR_ALIAS;
    if (tensor_sums && (overlap(tensor_sums, 16, x, nx) || overlap(tensor_sums, 16, codes, n / 2) ||
                        overlap(tensor_sums, 16, scales, n / kBlock) ||
                        (block_mse && overlap(tensor_sums, 16, block_mse, nbm))))
      return MX_ERR_ALIAS;
  } else if (!tensor_sums) {
    return MX_OK;
  }
  double *partial = nullptr;
  if (tensor_sums) {
    // every shape's partial sums fit the fixed scratch: with less space than
    // its fastest grid needs, the launch caps its grid at one sum group
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                          : hipGetDevice(&dev);
    if (e == hipSuccess) e = mxi_scratch_address(dev, &partial);
    if (e != hipSuccess) return finish(e);
  }
  if (rows == 0)  // an empty tensor has zero error; still a device write
    return finish(mxi_launch_block_mse(nullptr, 0, nullptr, nullptr, 0, nullptr, tensor_sums,
                                       partial, (int64_t)mxi_scratch_partials(),
                                       static_cast<hipStream_t>(stream)));
  return finish(mxi_launch_block_mse(x, x_dtype == MX_BF16, codes, scales, n / 8, block_mse,
                                     tensor_sums, partial, (int64_t)mxi_scratch_partials(),
                                     static_cast<hipStream_t>(stream)));
}

mx_status_t mx_quantize_fused(const void *x, mx_dtype_t x_dtype, int64_t rows, int64_t k,
                              mx_scale_mode_t mode, uint8_t *codes, uint8_t *scales, void *y,
                              float *block_mse, double *tensor_sums, void *workspace,
                              size_t workspace_bytes, void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (!mode_ok(mode)) return MX_ERR_MODE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (tensor_sums) {
    if ((reinterpret_cast<uintptr_t>(tensor_sums) & 7u) != 0) return MX_ERR_ALIGN;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0 ||
        workspace_bytes < mx_block_mse_workspace_size(rows, k))
      return MX_ERR_WORKSPACE;
  }
  if (rows == 0) {
    if (!tensor_sums) return MX_OK;
    if (overlap(tensor_sums, 16, workspace, (int64_t)workspace_bytes)) return MX_ERR_ALIAS;
    return finish(mxi_launch_quantize_fused(nullptr, 0, 0, 0, nullptr, nullptr, nullptr, nullptr,
                                            tensor_sums, static_cast<double *>(workspace),
                                            (int64_t)(workspace_bytes / sizeof(double)),
                                            static_cast<hipStream_t>(stream)));
  }
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || (y && !aligned16(y)))
    return MX_ERR_ALIGN;
  if (block_mse && (reinterpret_cast<uintptr_t>(block_mse) & 3u) != 0) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t nx = n * elem_bytes(x_dtype);
  // every written range against x and against each other
  struct R {
    const void *p;
    int64_t n;
  } out[5] = {{codes, n / 2}, {scales, n / kBlock}, {y, nx}, {block_mse, 4 * (n / kBlock)},
              {tensor_sums, 16}};
  for (int i = 0; i < 5; i++) {
    if (!out[i].p) continue;
    if (overlap(out[i].p, out[i].n, x, nx)) return MX_ERR_ALIAS;
    if (tensor_sums && overlap(out[i].p, out[i].n, workspace, (int64_t)workspace_bytes))
      return MX_ERR_ALIAS;
    for (int j = i + 1; j < 5; j++)
      if (out[j].p && overlap(out[i].p, out[i].n, out[j].p, out[j].n)) return MX_ERR_ALIAS;
  }
  if (tensor_sums && overlap(workspace, (int64_t)workspace_bytes, x, nx)) return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize_fused(x, x_dtype == MX_BF16, mode, n / 8, codes, scales, y,
                                          block_mse, tensor_sums,
                                          tensor_sums ? static_cast<double *>(workspace) : nullptr,
                                          (int64_t)(workspace_bytes / sizeof(double)),
                                          static_cast<hipStream_t>(stream)));
}

mx_status_t mx_quantize_mxfp8(const void *x, mx_dtype_t x_dtype, int64_t rows, int64_t k,
                              uint8_t *codes, uint8_t *scales, void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !codes || !scales) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t nx = n * elem_bytes(x_dtype);
  if (overlap(x, nx, codes, n) || overlap(x, nx, scales, n / kBlock) ||
      overlap(codes, n, scales, n / kBlock))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize8(x, x_dtype == MX_BF16, n / 8, codes, scales,
                                     static_cast<hipStream_t>(stream)));
}

mx_status_t mx_dequantize_mxfp8(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                int64_t k, mx_dtype_t y_dtype, void *y, void *stream) {
  if (!dtype_ok(y_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!codes || !scales || !y) return MX_ERR_NULL;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t ny = n * elem_bytes(y_dtype);
  if (overlap(y, ny, codes, n) || overlap(y, ny, scales, n / kBlock)) return MX_ERR_ALIAS;
  return finish(mxi_launch_dequantize8(codes, scales, y_dtype == MX_BF16, n / 8, y,
                                       static_cast<hipStream_t>(stream)));
}

mx_status_t mx_fakequant_mxfp8(const void *x, mx_dtype_t dtype, int64_t rows, int64_t k,
                               void *y, void *stream) {
  if (!dtype_ok(dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !y) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return MX_ERR_ALIGN;
  const int64_t nb = rows * k * elem_bytes(dtype);
  if (x != y && overlap(x, nb, y, nb)) return MX_ERR_ALIAS;
  return finish(mxi_launch_fakequant8(x, dtype == MX_BF16, rows * k / 8, y,
                                      static_cast<hipStream_t>(stream)));
}

size_t mx_nvfp4_workspace_size(int64_t rows, int64_t k) {
  if (check_shape16(rows, k) != MX_OK) return 0;
  const size_t n = mxi_nvfp4_partials(rows * k / 8);
  return (n > 0 ? n : 1) * sizeof(uint32_t);
}

mx_status_t mx_quantize_nvfp4(const void *x, mx_dtype_t x_dtype, int64_t rows, int64_t k,
                              uint8_t *codes, uint8_t *block_scales, uint8_t *tensor_scale,
                              void *workspace, size_t workspace_bytes, void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape16(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !codes || !block_scales || !tensor_scale) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(block_scales)) return MX_ERR_ALIGN;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0 ||
      workspace_bytes < mx_nvfp4_workspace_size(rows, k))
    return MX_ERR_WORKSPACE;
  const int64_t n = rows * k;
  const int64_t nx = n * elem_bytes(x_dtype), nw = (int64_t)workspace_bytes;
  if (overlap(x, nx, codes, n / 2) || overlap(x, nx, block_scales, n / 16) ||
      overlap(codes, n / 2, block_scales, n / 16) || overlap(tensor_scale, 1, x, nx) ||
      overlap(tensor_scale, 1, codes, n / 2) || overlap(tensor_scale, 1, block_scales, n / 16) ||
      overlap(workspace, nw, x, nx) || overlap(workspace, nw, codes, n / 2) ||
      overlap(workspace, nw, block_scales, n / 16) || overlap(workspace, nw, tensor_scale, 1))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize_nv(x, x_dtype == MX_BF16, n / 8, codes, block_scales,
                                       tensor_scale, static_cast<uint32_t *>(workspace), nullptr,
                                       static_cast<hipStream_t>(stream)));
}

mx_status_t mx_dequantize_nvfp4(const uint8_t *codes, const uint8_t *block_scales,
                                const uint8_t *tensor_scale, int64_t rows, int64_t k,
                                mx_dtype_t y_dtype, void *y, void *stream) {
  if (!dtype_ok(y_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape16(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!codes || !block_scales || !tensor_scale || !y) return MX_ERR_NULL;
  if (!aligned16(codes) || !aligned16(block_scales) || !aligned16(y)) return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t ny = n * elem_bytes(y_dtype);
  if (overlap(y, ny, codes, n / 2) || overlap(y, ny, block_scales, n / 16) ||
      overlap(y, ny, tensor_scale, 1))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_dequantize_nv(codes, block_scales, tensor_scale, y_dtype == MX_BF16,
                                         n / 8, y, static_cast<hipStream_t>(stream)));
}

mx_status_t mx_quantize_mbs(const void *x, mx_dtype_t x_dtype, int64_t rows, int64_t k,
                            uint8_t *codes, uint8_t *sub_scales, uint8_t *macro_mant,
                            void *stream) {
  if (!dtype_ok(x_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape_n(rows, k, 128)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !codes || !sub_scales || !macro_mant) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(sub_scales) || !aligned16(macro_mant))
    return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t nx = n * elem_bytes(x_dtype);
  if (overlap(x, nx, codes, n / 2) || overlap(x, nx, sub_scales, n / 16) ||
      overlap(x, nx, macro_mant, n / 128) || overlap(codes, n / 2, sub_scales, n / 16) ||
      overlap(codes, n / 2, macro_mant, n / 128) ||
      overlap(sub_scales, n / 16, macro_mant, n / 128))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize_mbs(x, x_dtype == MX_BF16, n / 8, codes, sub_scales,
                                        macro_mant, nullptr, static_cast<hipStream_t>(stream)));
}

mx_status_t mx_fakequant_nvfp4(const void *x, mx_dtype_t dtype, int64_t rows, int64_t k,
                               void *y, void *workspace, size_t workspace_bytes, void *stream) {
  if (!dtype_ok(dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape16(rows, k)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !y) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return MX_ERR_ALIGN;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0 ||
      workspace_bytes < mx_nvfp4_workspace_size(rows, k))
    return MX_ERR_WORKSPACE;
  const int64_t nb = rows * k * elem_bytes(dtype), nw = (int64_t)workspace_bytes;
  if ((x != y && overlap(x, nb, y, nb)) || overlap(workspace, nw, x, nb) ||
      overlap(workspace, nw, y, nb))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize_nv(x, dtype == MX_BF16, rows * k / 8, nullptr, nullptr,
                                       nullptr, static_cast<uint32_t *>(workspace), y,
                                       static_cast<hipStream_t>(stream)));
}

mx_status_t mx_fakequant_mbs(const void *x, mx_dtype_t dtype, int64_t rows, int64_t k, void *y,
                             void *stream) {
  if (!dtype_ok(dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape_n(rows, k, 128)) return s;
  if (rows == 0) return MX_OK;
  if (!x || !y) return MX_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return MX_ERR_ALIGN;
  const int64_t nb = rows * k * elem_bytes(dtype);
  if (x != y && overlap(x, nb, y, nb)) return MX_ERR_ALIAS;
  return finish(mxi_launch_quantize_mbs(x, dtype == MX_BF16, rows * k / 8, nullptr, nullptr,
                                        nullptr, y, static_cast<hipStream_t>(stream)));
}

mx_status_t mx_dequantize_mbs(const uint8_t *codes, const uint8_t *sub_scales,
                              const uint8_t *macro_mant, int64_t rows, int64_t k,
                              mx_dtype_t y_dtype, void *y, void *stream) {
  if (!dtype_ok(y_dtype)) return MX_ERR_DTYPE;
  if (mx_status_t s = check_shape_n(rows, k, 128)) return s;
  if (rows == 0) return MX_OK;
  if (!codes || !sub_scales || !macro_mant || !y) return MX_ERR_NULL;
  if (!aligned16(codes) || !aligned16(sub_scales) || !aligned16(macro_mant) || !aligned16(y))
    return MX_ERR_ALIGN;
  const int64_t n = rows * k;
  const int64_t ny = n * elem_bytes(y_dtype);
  if (overlap(y, ny, codes, n / 2) || overlap(y, ny, sub_scales, n / 16) ||
      overlap(y, ny, macro_mant, n / 128))
    return MX_ERR_ALIAS;
  return finish(mxi_launch_dequantize_mbs(codes, sub_scales, macro_mant, y_dtype == MX_BF16,
                                          n / 8, y, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Byte range one tensor of a multi call reads (in) or writes (out).
struct Span {
  const void *p;
  int64_t n;
  int owner;
  bool out;
};

// The latest-ending earlier span, and the latest-ending one of any other
// owner: enough to tell whether some earlier span of an owner other than o
// reaches past a point.
struct Reach {
  uintptr_t end1 = 0, end2 = 0;
  int owner1 = -1;
  void add(uintptr_t end, int owner) {
    if (owner == owner1) {
      end1 = end > end1 ? end : end1;
    } else if (end > end1) {
      end2 = end1;
      end1 = end;
      owner1 = owner;
    } else if (end > end2) {
      end2 = end;
    }
  }
  bool other_reaches(uintptr_t point, int o) const {
    return (owner1 != o ? end1 : end2) > point;
  }
};

// A tensor one of whose spans overlaps another tensor's output (or whose
// output overlaps another tensor's span), or -1. Sorted by
// start, every overlapping pair is seen when its later-starting member
// arrives: an output is checked against every earlier span, an input
// against every earlier output. O(n log n).
int cross_overlap(std::vector<Span> &spans) {
  std::sort(spans.begin(), spans.end(), [](const Span &a, const Span &b) {
    return reinterpret_cast<uintptr_t>(a.p) < reinterpret_cast<uintptr_t>(b.p);
  });
  Reach any, outs;
  for (const Span &q : spans) {
    const uintptr_t start = reinterpret_cast<uintptr_t>(q.p);
    if (q.out && any.other_reaches(start, q.owner)) return q.owner;
    if (!q.out && outs.other_reaches(start, q.owner)) return q.owner;
    const uintptr_t end = start + (uintptr_t)q.n;
    any.add(end, q.owner);
    if (q.out) outs.add(end, q.owner);
  }
  return -1;
}

void set_detail_tensor(int i, const char *what) {
  snprintf(g_detail, sizeof g_detail, "tensor %d: %s", i, what);
}

mx_status_t multi(const mx_tensor_t *tensors, int count, mx_dtype_t dtype,
                  mx_scale_mode_t mode, bool fakequant, void *stream) {
  if (!dtype_ok(dtype)) return MX_ERR_DTYPE;
  if (!mode_ok(mode)) return MX_ERR_MODE;
  if (count < 0) return MX_ERR_SHAPE;
  if (count == 0) return MX_OK;
  if (!tensors) return MX_ERR_NULL;
  std::vector<MxiTensor> launch;
  std::vector<Span> spans;
  launch.reserve(count);
  for (int i = 0; i < count; i++) {
    const mx_tensor_t &t = tensors[i];
    if (mx_status_t s = check_shape(t.rows, t.k)) {
      set_detail_tensor(i, "shape");
      return s;
    }
    if (t.rows == 0) continue;
    const int64_t n = t.rows * t.k;
    const int64_t nx = n * elem_bytes(dtype);
    if (fakequant) {
      if (!t.x || !t.y) {
        set_detail_tensor(i, "NULL pointer");
        return MX_ERR_NULL;
      }
      if (!aligned16(t.x) || !aligned16(t.y)) {
        set_detail_tensor(i, "alignment");
        return MX_ERR_ALIGN;
      }
      if (t.x != t.y && overlap(t.x, nx, t.y, nx)) {
        set_detail_tensor(i, "y partially overlaps x");
        return MX_ERR_ALIAS;
      }
      spans.push_back({t.x, nx, i, false});
      spans.push_back({t.y, nx, i, true});
      launch.push_back({t.x, t.y, nullptr, n / 8});
    } else {
      if (!t.x || !t.codes || !t.scales) {
        set_detail_tensor(i, "NULL pointer");
        return MX_ERR_NULL;
      }
      if (!aligned16(t.x) || !aligned16(t.codes) || !aligned16(t.scales)) {
        set_detail_tensor(i, "alignment");
        return MX_ERR_ALIGN;
      }
      if (overlap(t.x, nx, t.codes, n / 2) || overlap(t.x, nx, t.scales, n / kBlock) ||
          overlap(t.codes, n / 2, t.scales, n / kBlock)) {
        set_detail_tensor(i, "an output overlaps an input");
        return MX_ERR_ALIAS;
      }
      spans.push_back({t.x, nx, i, false});
      spans.push_back({t.codes, n / 2, i, true});
      spans.push_back({t.scales, n / kBlock, i, true});
      launch.push_back({t.x, t.codes, t.scales, n / 8});
    }
  }
  // no tensor's output may touch another tensor's input or output (inputs
  // may be shared)
  if (int bad = cross_overlap(spans); bad >= 0) {
    set_detail_tensor(bad, "overlaps another tensor's output, or its output another tensor's data");
    return MX_ERR_ALIAS;
  }
  if (launch.empty()) return MX_OK;
  return finish(mxi_launch_multi(launch.data(), (int)launch.size(), dtype == MX_BF16, mode,
                                 fakequant ? 1 : 0, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

mx_status_t mx_quantize_multi(const mx_tensor_t *tensors, int count, mx_dtype_t dtype,
                              mx_scale_mode_t mode, void *stream) {
  return multi(tensors, count, dtype, mode, false, stream);
}

mx_status_t mx_fakequant_multi(const mx_tensor_t *tensors, int count, mx_dtype_t dtype,
                               mx_scale_mode_t mode, void *stream) {
  return multi(tensors, count, dtype, mode, true, stream);
}

const char *mx_status_string(mx_status_t s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: need rows >= 0 and k a positive multiple of the block (32; 16 for NVFP4; 128 for MBS-Static)";
    case MX_ERR_DTYPE: return "MX_ERR_DTYPE: dtype must be MX_F32 or MX_BF16";
    case MX_ERR_MODE: return "MX_ERR_MODE: mode must be an mx_scale_mode_t value (0..3)";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: data pointers must be 16-byte aligned";
    case MX_ERR_HIP: return "MX_ERR_HIP: HIP launch failed";
    case MX_ERR_ALIAS: return "MX_ERR_ALIAS: an output overlaps an input";
    case MX_ERR_WORKSPACE: return "MX_ERR_WORKSPACE: workspace missing, misaligned or too small";
  }
  return "unknown mx_status_t";
}

const char *mx_last_error_detail(void) { return g_detail; }

}  // extern "C"
