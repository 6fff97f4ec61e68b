// bench_ceiling.hip - reference streaming kernels the benchmark times beside
// the MXFP4 kernels, to show what HBM allows for the same traffic shape on
// this part. They are not part of the library and compute nothing of the
// format: each moves exactly the bytes of one MXFP4 operation with as little
// arithmetic as the compiler allows, in the streaming form that measured
// fastest for these traffic shapes on multi-GB tensors: 256-thread
// workgroups, one item of 16 bytes per thread, one tile per workgroup (no
// grid cap), non-temporal 16-byte loads and stores. (On the 5.6 GB weight
// buffer a copy ran at 81 % of 8 TB/s with one item per thread and 70 % with
// four on a grid capped at 196,608 workgroups.)
//
//   mxc_quantize_shape: per 16-byte item read, one 4-byte word written (the
//     code word) and, for every 4th item, one byte (the scale byte): the
//     traffic of bf16 quantize, 2 + 1/2 + 1/32 bytes per element.
//   mxc_dequantize_shape: the reverse, per item one 4-byte word and the
//     byte of its group of 4 items read (every lane loads it, as dequantize
//     does), 16 bytes written: the traffic of bf16 dequantize.
//   mxc_block_mse_shape: per item 16 bytes, one 4-byte word and the byte of
//     its group read, and for every 4th item one 4-byte word written: the
//     traffic of bf16 block MSE with its per-block output, 2 + 1/2 + 1/32 +
//     1/8 bytes per element.
//   mxc_copy: 16 bytes read and 16 bytes written per item.
//   mxc_read / mxc_write: only the loads / only the stores of a copy.
//   mxc_empty: one workgroup that does nothing (the launch floor).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kItems = 1;
constexpr int64_t kGridCap = 0x7FFFFFFF;

unsigned grid_for(int64_t nitems) {
  const int64_t tile = (int64_t)kThreads * kItems;
  int64_t g = (nitems + tile - 1) / tile;
  if (g > kGridCap) g = kGridCap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

// Visits every item index of [0, nitems) once: full tiles load all items
// first; the partial tile checks each index.
template <typename Load, typename Use>
__device__ __forceinline__ void tiles(int64_t nitems, Load load, Use use) {
  const int64_t tile = (int64_t)kThreads * kItems;
  const int64_t nfull = nitems / tile;
  int64_t t = blockIdx.x;
  for (; t < nfull; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kItems; u++) load(u, base + u * kThreads);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kItems; u++) use(u, base + u * kThreads);
  }
  if (t == nfull && nfull * tile < nitems) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kItems; u++)
      if (base + u * kThreads < nitems) load(u, base + u * kThreads);
#pragma unroll
    for (int u = 0; u < kItems; u++)
      if (base + u * kThreads < nitems) use(u, base + u * kThreads);
  }
}

__global__ __launch_bounds__(kThreads) void k_ceiling_quantize_shape(
    const u32x4 *__restrict__ x, uint32_t *__restrict__ words, uint8_t *__restrict__ bytes,
    int64_t nitems) {
  u32x4 v[kItems];
  tiles(
      nitems, [&](int u, int64_t it) { v[u] = __builtin_nontemporal_load(x + it); },
      [&](int u, int64_t it) {
        words[it] = v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        if ((threadIdx.x & 3) == 0) bytes[it >> 2] = (uint8_t)(v[u][0] >> 24);
      });
}

__global__ __launch_bounds__(kThreads) void k_ceiling_dequantize_shape(
    const uint32_t *__restrict__ words, const uint8_t *__restrict__ bytes,
    u32x4 *__restrict__ y, int64_t nitems) {
  uint32_t w[kItems], b[kItems];
  tiles(
      nitems,
      [&](int u, int64_t it) {
        w[u] = words[it];
        b[u] = bytes[it >> 2];
      },
      [&](int u, int64_t it) {
        const uint32_t v = w[u] ^ b[u];
        __builtin_nontemporal_store(u32x4{v, v, v, v}, y + it);
      });
}

__global__ __launch_bounds__(kThreads) void k_ceiling_block_mse_shape(
    const u32x4 *__restrict__ x, const uint32_t *__restrict__ words,
    const uint8_t *__restrict__ bytes, uint32_t *__restrict__ out, int64_t nitems) {
  u32x4 v[kItems];
  uint32_t w[kItems], b[kItems];
  tiles(
      nitems,
      [&](int u, int64_t it) {
        v[u] = __builtin_nontemporal_load(x + it);
        w[u] = words[it];
        b[u] = bytes[it >> 2];
      },
      [&](int u, int64_t it) {
        if ((threadIdx.x & 3) == 0) out[it >> 2] = v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3] ^ w[u] ^ b[u];
      });
}

__global__ __launch_bounds__(kThreads) void k_ceiling_copy(const u32x4 *__restrict__ x,
                                                           u32x4 *__restrict__ y,
                                                           int64_t nitems) {
  u32x4 v[kItems];
  tiles(
      nitems, [&](int u, int64_t it) { v[u] = __builtin_nontemporal_load(x + it); },
      [&](int u, int64_t it) { __builtin_nontemporal_store(v[u], y + it); });
}

__global__ __launch_bounds__(kThreads) void k_ceiling_read(const u32x4 *__restrict__ x,
                                                           uint32_t *__restrict__ sink,
                                                           int64_t nitems) {
  u32x4 v[kItems];
  uint32_t acc = 0;
  tiles(
      nitems, [&](int u, int64_t it) { v[u] = __builtin_nontemporal_load(x + it); },
      [&](int u, int64_t) { acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]; });
  // one word per workgroup, so the loads stay live
  acc = __builtin_amdgcn_readfirstlane(acc);
  if (threadIdx.x == 0 && acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void k_ceiling_write(u32x4 *__restrict__ y,
                                                            int64_t nitems) {
  tiles(
      nitems, [&](int, int64_t) {},
      [&](int, int64_t it) {
        const uint32_t w = (uint32_t)it;
        __builtin_nontemporal_store(u32x4{w, w, w, w}, y + it);
      });
}

__global__ void k_ceiling_empty() {}

}  // namespace

extern "C" {

// nitems: number of 16-byte items of the input (8 bf16 elements each).
int mxc_quantize_shape(const void *x, int64_t nitems, void *words, void *bytes, void *stream) {
  hipLaunchKernelGGL(k_ceiling_quantize_shape, dim3(grid_for(nitems)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(x),
                     static_cast<uint32_t *>(words), static_cast<uint8_t *>(bytes), nitems);
  return (int)hipGetLastError();
}

// words: nitems 4-byte words; bytes: nitems / 4 bytes; y: nitems 16-byte items.
int mxc_dequantize_shape(const void *words, const void *bytes, int64_t nitems, void *y,
                         void *stream) {
  hipLaunchKernelGGL(k_ceiling_dequantize_shape, dim3(grid_for(nitems)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint32_t *>(words),
                     static_cast<const uint8_t *>(bytes), static_cast<u32x4 *>(y), nitems);
  return (int)hipGetLastError();
}

// x: nitems 16-byte items; words: nitems 4-byte words; bytes: nitems / 4
// bytes; out: nitems / 4 4-byte words.
int mxc_block_mse_shape(const void *x, const void *words, const void *bytes, int64_t nitems,
                        void *out, void *stream) {
  hipLaunchKernelGGL(k_ceiling_block_mse_shape, dim3(grid_for(nitems)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(x),
                     static_cast<const uint32_t *>(words), static_cast<const uint8_t *>(bytes),
                     static_cast<uint32_t *>(out), nitems);
  return (int)hipGetLastError();
}

int mxc_copy(const void *x, void *y, int64_t nitems, void *stream) {
  hipLaunchKernelGGL(k_ceiling_copy, dim3(grid_for(nitems)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(x),
                     static_cast<u32x4 *>(y), nitems);
  return (int)hipGetLastError();
}

// sink: at least as many 4-byte words as workgroups (nitems / 256, rounded up).
int mxc_read(const void *x, int64_t nitems, void *sink, void *stream) {
  hipLaunchKernelGGL(k_ceiling_read, dim3(grid_for(nitems)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(x),
                     static_cast<uint32_t *>(sink), nitems);
  return (int)hipGetLastError();
}

int mxc_write(void *y, int64_t nitems, void *stream) {
  hipLaunchKernelGGL(k_ceiling_write, dim3(grid_for(nitems)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(y), nitems);
  return (int)hipGetLastError();
}

int mxc_empty(void *stream) {
  hipLaunchKernelGGL(k_ceiling_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

}  // extern "C"
