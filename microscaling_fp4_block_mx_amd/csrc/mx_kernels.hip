// mx_kernels.hip - gfx950 kernels for OCP MXFP4 block quantization.
//
// Work decomposition (all ops): the tensor is a flat run of 32-element MX
// blocks (rows are contiguous and k % 32 == 0, so block b covers elements
// 32b..32b+31 and owns scale byte b and code bytes 16b..16b+15). A block is
// handled by a quad of 4 adjacent lanes; lane q of the quad owns elements
// 8q..8q+7 ("item" = 8 elements = one 16-byte bf16 load, one 32-bit code
// word). A wave64 covers 16 blocks per item step: 1 KiB of bf16 in, 256 B of
// codes and 16 B of scales out, all contiguous.
//
// Cross-lane work inside a quad (block amax, block squared error) uses DPP
// quad permutations, so quads must always be whole: every launch covers a
// multiple of 4 items and the per-thread item stride is a multiple of 4.
//
// Element conversion uses the gfx950 scaled FP4 converts:
//   v_cvt_scalef32_pk_fp4_{bf16,f32}: two values / 2^(s-127) -> two E2M1
//     codes in one byte (first value in the low nibble), nearest with ties
//     to the even code, saturating at +-6;
//   v_cvt_scalef32_pk_{bf16,f32}_fp4: one byte of two codes -> two values
//     E2M1 * 2^(s-127).
// The scale operand is passed as the fp32 bit pattern s << 23, whose
// exponent field is the E8M0 byte. These were checked against the CPU
// oracle over every finite bf16 pair at scale bytes 0..252 (subnormal inputs
// included) and over every code byte at every scale byte before adoption;
// the one difference, the NaN produced for scale byte 255 (0xFFC00000
// instead of the canonical 0x7FC00000), is corrected here.
//
// Format facts (E2M1 grid 0, .5, 1, 1.5, 2, 3, 4, 6; E8M0 scale 2^(s-127);
// two codes per byte, even element low) are stated with their sources in
// include/mx.h. The MXFP4 kernels (quantize, fake-quant, dequantize, block
// error, and the one pass that does all of them from one read of x) come
// first; later sections hold the multi-tensor launch and the other formats
// on the same item layout (MXFP8, the NVFP4 comparator, MBS-Static).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_internal.h"

namespace mxk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef MX_UNROLL
#define MX_UNROLL 4
#endif
// Most workgroups a streaming launch uses (beyond it, workgroups loop over
// tiles). Measured on a 2.1e9-element bf16 tensor: 196,608 (768 per CU)
// beat 65,536 by 5 % (quantize) and 3 % (dequantize) with fake-quant level,
// while 8,192-32,768 were slower. Tensors below ~200 M elements get one tile
// per workgroup either way.
#ifndef MX_GRID_CAP
#define MX_GRID_CAP 196608
#endif
constexpr int kThreads = 256;
constexpr int kUnroll = MX_UNROLL;  // items per thread per grid-stride step
constexpr uint32_t kNaN32 = 0x7FC00000u;
constexpr uint32_t kNaN16x2 = 0x7FC07FC0u;

// ---- cross-lane helpers (quad = 4 adjacent lanes) --------------------------

// quad_perm [1,0,3,2] and [2,3,0,1]: exchange with lane^1 and lane^2.
// bound_ctrl is set on every DPP move here: the source lane always lies in
// the same quad (or 16-lane row), and quads and rows enter and leave the
// ragged tail whole, so no lane reads a missing or inactive one and the
// flag changes no result; it lets the compiler fold the move into the ALU
// op that uses it (one DPP op instead of a move, a wait state and the op).
__device__ __forceinline__ uint32_t dpp_x1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_x2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp_x1(v));
  v = max(v, dpp_x2(v));
  return v;
}

// (p0 + p1) + (p2 + p3) on every lane of the quad; fp32 addition commutes,
// so all four lanes hold the same bits.
__device__ __forceinline__ float quad_sum_f32(float p) {
  p = p + __uint_as_float(dpp_x1(__float_as_uint(p)));
  p = p + __uint_as_float(dpp_x2(__float_as_uint(p)));
  return p;
}

__device__ __forceinline__ double dpp_x1_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = dpp_x1((uint32_t)u), hi = dpp_x1((uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp_x2_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = dpp_x2((uint32_t)u), hi = dpp_x2((uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double quad_sum_f64(double p) {
  p = p + dpp_x1_f64(p);
  p = p + dpp_x2_f64(p);
  return p;
}

// ---- memory helpers -----------------------------------------------------------

// Streaming accesses. Each bf16 item is one 16-byte access and a wave's 64
// accesses cover 1 KiB contiguously, so bf16 tensors are read and written
// with the non-temporal hint (no reuse; fewer dirty L2 lines to write back
// at the end of the kernel). fp32 items take two 16-byte accesses whose
// per-instruction footprint is strided (32-byte lane pitch): fp32 loads,
// and the small code/scale accesses, stay on the default cache policy,
// which measured faster for them; fp32 stores are regrouped through LDS into
// contiguous non-temporal stores (store_item).
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void st(T *p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---- items -----------------------------------------------------------------

// Raw bits of one item: 8 elements. bf16 uses w[0..3] (two elements per
// word, even element in the low half); fp32 uses w[0..7].
template <bool BF16>
struct Item {
  uint32_t w[BF16 ? 4 : 8];
};

// One item's 8 elements. (fp32 items are read directly, two 16-byte loads
// per lane: a variant that read 1 KiB-contiguous units and swapped them into
// place through LDS measured no faster, unlike the stores below.)
template <bool BF16>
__device__ __forceinline__ void load_item(const void *base, int64_t it, Item<BF16> &x) {
  if constexpr (BF16) {
    const u32x4 d = ld<true>(reinterpret_cast<const u32x4 *>(base) + it);
#pragma unroll
    for (int j = 0; j < 4; j++) x.w[j] = d[j];
  } else {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(base) + 2 * it;
    const u32x4 a = ld<false>(p), b = ld<false>(p + 1);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      x.w[j] = a[j];
      x.w[4 + j] = b[j];
    }
  }
}

// Store the output words of one item (bf16: 4 words, fp32: 8 words).
//
// An fp32 item is 32 bytes, so two direct 16-byte stores per lane leave
// every store instruction writing half of each 32-byte span (lane pitch 32
// bytes). When the whole wave is active its 64 items are consecutive, so
// the wave first passes its 2 KiB through LDS: lane j writes its two
// 16-byte halves to units 2j and 2j+1, then lane L stores units L and
// 64 + L, and each store instruction writes 1 KiB contiguously with the
// non-temporal hint (measured: fp32 dequantize 29.4 -> 22.5 us on 32 Mi
// elements). A partly active wave (the ragged tail) stores directly.
template <bool BF16>
__device__ __forceinline__ void store_item(void *base, int64_t it,
                                           const uint32_t (&y)[BF16 ? 4 : 8]) {
  if constexpr (BF16) {
    st<true>(reinterpret_cast<u32x4 *>(base) + it, u32x4{y[0], y[1], y[2], y[3]});
  } else {
    u32x4 *p = reinterpret_cast<u32x4 *>(base) + 2 * it;
    const u32x4 lo = {y[0], y[1], y[2], y[3]}, hi = {y[4], y[5], y[6], y[7]};
    if (__builtin_amdgcn_read_exec() == ~0ull) {
      __shared__ u32x4 xpose[kThreads / 64][128];
      u32x4 *w = xpose[threadIdx.x >> 6];
      const int lane = (int)(threadIdx.x & 63);
      w[2 * lane] = lo;
      w[2 * lane + 1] = hi;
      // the other lanes' writes must land before the reads (one wave: LDS
      // runs its instructions in order; the fences keep the compiler's order)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const u32x4 a = w[lane], b = w[64 + lane];
      // and every read here before the next item's writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      u32x4 *q = p - 2 * lane;  // the wave's first item
      st<true>(q + lane, a);
      st<true>(q + 64 + lane, b);
    } else {
      st<false>(p, lo);
      st<false>(p + 1, hi);
    }
  }
}

// Element i of the item widened to fp32 (exact).
template <bool BF16>
__device__ __forceinline__ float elem(const Item<BF16> &x, int i) {
  if constexpr (BF16) return __uint_as_float((i & 1) ? (x.w[i >> 1] & 0xFFFF0000u) : (x.w[i >> 1] << 16));
  return __uint_as_float(x.w[i]);
}

// Largest |x| bit pattern of the item, in fp32 layout (bf16 widened).
template <bool BF16>
__device__ __forceinline__ uint32_t item_amax_bits(const Item<BF16> &x) {
  if constexpr (BF16) {
    u16x2 m = __builtin_bit_cast(u16x2, x.w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 4; j++)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x.w[j] & 0x7FFF7FFFu));
    return (uint32_t)max(m.x, m.y) << 16;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) m = max(m, x.w[j] & 0x7FFFFFFFu);
    return m;
  }
}

// ---- the format --------------------------------------------------------------

// E8M0 byte of the OCP rule from the block's largest |x| bit pattern:
// floor(log2 amax) - 2 + 127 = exponent field - 2 (0 for zero/subnormal
// amax), 255 for a NaN/Inf block.
__device__ __forceinline__ uint32_t ocp_scale_byte(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 255u;
  const uint32_t e = amax_bits >> 23;
  return e > 2u ? e - 2u : 0u;
}

// Scale operand of the converts for byte s.
__device__ __forceinline__ float scale_operand(uint32_t s) { return __uint_as_float(s << 23); }

// fl32(a / 6) for the non-negative fp32 pattern a. From 2^-125 up, the
// product with fl32(1/6) plus one fma residual correction is the correctly
// rounded quotient (checked against IEEE division for every fp32 value in
// that range); below it, where the quotient is subnormal, IEEE division.
__device__ __forceinline__ float div6_fast(float a) {
  constexpr float kSixth = 1.0f / 6.0f;
  const float q0 = a * kSixth;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, a), kSixth, q0);
}
__device__ __forceinline__ float div6(uint32_t a_bits) {
  const float a = __uint_as_float(a_bits);
  if (__builtin_expect(a_bits < 0x01000000u, 0)) return a / 6.0f;
  return div6_fast(a);
}


// 8 codes of the item at scale byte s (finite block), packed in one word,
// element i in nibble i.
template <bool BF16>
__device__ __forceinline__ uint32_t encode_item(const Item<BF16> &x, uint32_t s) {
  const float sc = scale_operand(s);
  uint32_t r = 0;
  if constexpr (BF16) {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x.w[0]), sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x.w[1]), sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x.w[2]), sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x.w[3]), sc, 3);
  } else {
    const float *f = reinterpret_cast<const float *>(x.w);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[0], f[1], sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[2], f[3], sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[4], f[5], sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[6], f[7], sc, 3);
  }
  return r;
}

// Codes of a NaN/Inf block: the sign bit alone.
template <bool BF16>
__device__ __forceinline__ uint32_t sign_codes(const Item<BF16> &x) {
  uint32_t r = 0;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; j++)
      r |= (((x.w[j] >> 12) & 0x8u) | ((x.w[j] >> 24) & 0x80u)) << (8 * j);
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) r |= ((x.w[i] >> 31) << 3) << (4 * i);
  }
  return r;
}

// Decode the 8 codes of word c at byte s into output words: bf16 gives 4
// words (two elements each), fp32 gives 8. Byte 255 gives canonical NaNs.
template <bool BF16>
__device__ __forceinline__ void decode_item(uint32_t c, uint32_t s, uint32_t (&y)[BF16 ? 4 : 8]) {
  const float sc = scale_operand(s);
  if constexpr (BF16) {
    y[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0));
    y[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1));
    y[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2));
    y[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3));
    if (__builtin_expect(s == 255u, 0)) {
#pragma unroll
      for (int j = 0; j < 4; j++) y[j] = kNaN16x2;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f32x2 v;
      switch (j) {
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 3); break;
      }
      y[2 * j] = __float_as_uint(v.x);
      y[2 * j + 1] = __float_as_uint(v.y);
    }
    if (__builtin_expect(s == 255u, 0)) {
#pragma unroll
      for (int j = 0; j < 8; j++) y[j] = kNaN32;
    }
  }
}

// The 8 decoded values of word c at byte s as fp32 (Inf/NaN passed through).
__device__ __forceinline__ void decode_f32(uint32_t c, uint32_t s, float (&q)[8]) {
  const float sc = scale_operand(s);
  f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 0);
  f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 1);
  f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 2);
  f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 3);
  q[0] = v0.x; q[1] = v0.y; q[2] = v1.x; q[3] = v1.y;
  q[4] = v2.x; q[5] = v2.y; q[6] = v3.x; q[7] = v3.y;
}

// Lane share of the pinned fp32 block squared error at scale byte c:
// d = x - x_hat in fp32, even positions in one fma accumulator, odd in
// another, lane share = even + odd. Returns the candidate's codes too.
template <bool BF16>
__device__ __forceinline__ float lane_sse(const Item<BF16> &x, uint32_t c, uint32_t &codes) {
  codes = encode_item<BF16>(x, c);
  float q[8];
  decode_f32(codes, c, q);
  float acc_e = 0.0f, acc_o = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float d0 = elem<BF16>(x, i) - q[i];
    const float d1 = elem<BF16>(x, i + 1) - q[i + 1];
    acc_e = __builtin_fmaf(d0, d0, acc_e);
    acc_o = __builtin_fmaf(d1, d1, acc_o);
  }
  return acc_e + acc_o;
}

// Block scale byte and this lane's 8 codes (all quad lanes agree on s).
//
// Modes (bytes as in include/mx.h): with s0 the OCP byte and v0 the block
// maximum over 2^(s0-127) (in [4, 8) whenever the exponent field e of amax is
// >= 2), the no-overflow byte is s0 + 1 exactly when v0 > 6, i.e. when amax's
// mantissa field exceeds 0x400000; the page's halving test ((3, 3.5] under
// the no-overflow scale) leaves s0 + 1 only when v0 > 7, i.e. mantissa field
// > 0x600000. Both are capped at 252 so every code decodes finite.
//
// Error-driven modes compare a high byte h with h - 1 by the pinned fp32
// SSE. h - 1 is evaluated only when it can win: at h - 1 the block maximum
// (> 3 * 2^(h-127)) saturates to 3 * 2^(h-127), so that element alone
// contributes fl(d * d) with d = amax - 3 * 2^(h-127) (exact in fp32), and the
// pinned sum only grows as non-negative terms are added (rounding is
// monotone). Hence SSE32(h - 1) >= fl(d * d); when SSE32(h) <= fl(d * d) the
// strict test SSE32(h - 1) < SSE32(h) must fail and h is kept without
// computing it. The decision is identical to evaluating both candidates.
template <bool BF16, int MODE>
__device__ __forceinline__ uint32_t quantize_item(const Item<BF16> &x, uint32_t &codes) {
  const uint32_t amax = quad_max_u32(item_amax_bits<BF16>(x));
  const uint32_t s0 = ocp_scale_byte(amax);
  if (__builtin_expect(s0 == 255u, 0)) {
    codes = sign_codes<BF16>(x);
    return s0;
  }
  const uint32_t mant = amax & 0x7FFFFFu;
  const bool normalized = (amax >> 23) >= 2u;  // v0 in [4, 8)
  if constexpr (MODE == MX_SCALE_OCP || MODE == MX_SCALE_OAS_BITS) {
    uint32_t s = s0;
    if (MODE == MX_SCALE_OAS_BITS && normalized && mant > 0x600000u) s = min(s0 + 1u, 252u);
    codes = encode_item<BF16>(x, s);
    return s;
  } else {
    uint32_t h = s0;
    if (MODE == MX_SCALE_OAS_NF && normalized && mant > 0x400000u) h = min(s0 + 1u, 252u);
    if (h == 0u) {
      codes = encode_item<BF16>(x, h);
      return h;
    }
    uint32_t c_hi;
    const float sse_hi = quad_sum_f32(lane_sse<BF16>(x, h, c_hi));
    const float d_top = __uint_as_float(amax) - __builtin_amdgcn_ldexpf(3.0f, (int)h - 127);
    const float bound = d_top * d_top;
    codes = c_hi;
    if (sse_hi > bound) {  // uniform over the quad: same sums, same amax
      uint32_t c_low;
      const float sse_low = quad_sum_f32(lane_sse<BF16>(x, h - 1u, c_low));
      if (sse_low < sse_hi) {  // strict: a tie keeps h
        codes = c_low;
        return h - 1u;
      }
    }
    return h;
  }
}

// ---- kernels -----------------------------------------------------------------

// Grid-stride over tiles of kThreads * U items; each thread's U items are
// spaced kThreads apart so every load instruction is coalesced, and the loads
// of a tile come ahead of its arithmetic (the backend may still sink a load
// whose value is first used past a divergent branch below the first item's
// work: OAS quantize issues one load, then three, which measured faster than
// forcing all four ahead). Full tiles run without bounds
// checks; the one partial tile (if any) is handled by the workgroup whose
// stride lands on it, with per-item checks.
template <int U, typename Load, typename Use>
__device__ __forceinline__ void tile_loop(int64_t nitems, Load load, Use use) {
  const int64_t tile = (int64_t)kThreads * U;
  const int64_t nfull = nitems / tile;
  int64_t t = blockIdx.x;
  for (; t < nfull; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++) load(u, base + u * kThreads);
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic
#pragma unroll
    for (int u = 0; u < U; u++) use(u, base + u * kThreads);
  }
  if (t == nfull && nfull * tile < nitems) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * kThreads < nitems) load(u, base + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; u++)  // whole quads (16-lane rows) drop out together
      if (base + u * kThreads < nitems) use(u, base + u * kThreads);
  }
}

// Items per thread per tile for the streaming kernels: kUnroll bf16 items,
// a quarter as many fp32 items (an fp32 item is two 16-byte accesses). One
// fp32 item per thread doubles the workgroups in flight, which measured
// 2-4 % faster than two for fp32 quantize, dequantize and MXFP8 on both a
// 4 Mi-element and a 32 Mi-element tensor. (Kernels whose workspace size is
// fixed per shape, whatever the dtype, keep kUnroll for both.)
template <bool BF16>
constexpr int kU = BF16 ? kUnroll : (kUnroll >= 4 ? kUnroll / 4 : 1);

// Items per thread for the MXFP4 kernels, by what the kernel does (measured
// each op alone): bf16 quantize in the OCP, OAS and OAS_BITS modes keeps kU
// (two items per thread was 7 % slower on 8192x4096, eight 3-13 % slower), while bf16 dequantize
// and OAS_NF quantize take two (2-12 % faster: fewer registers and more
// workgroups in flight for the longer per-item work or the write-heavy
// stream). Fake-quant takes two items in both dtypes (one fp32 item was 5 %
// slower on fp32 1024x4096). The multi-tensor launch uses the same numbers;
// its tile offsets depend on them.
enum { kKindQuantize = 0, kKindFakequant = 1, kKindDequantize = 2 };
constexpr int unroll_of(bool bf16, int mode, int kind) {
  if (kind == kKindFakequant) return 2;
  if (!bf16) return kU<false>;
  return kind == kKindQuantize && mode != MX_SCALE_OAS_NF ? kU<true> : 2;
}

template <bool BF16, int MODE>
__global__ __launch_bounds__(kThreads) void k_quantize(const void *__restrict__ x,
                                                       uint32_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales,
                                                       int64_t nitems) {
  constexpr int U = unroll_of(BF16, MODE, kKindQuantize);
  Item<BF16> xv[U];
  tile_loop<U>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t it) {
        uint32_t c;
        const uint32_t s = quantize_item<BF16, MODE>(xv[u], c);
        st<false>(codes + it, c);
        if ((threadIdx.x & 3) == 0) st<false>(scales + (it >> 2), (uint8_t)s);
      });
}

template <bool BF16, int MODE>
__global__ __launch_bounds__(kThreads) void k_fakequant(const void *x, void *y, int64_t nitems) {
  constexpr int U = unroll_of(BF16, MODE, kKindFakequant);
  Item<BF16> xv[U];
  tile_loop<U>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t it) {
        uint32_t c;
        const uint32_t s = quantize_item<BF16, MODE>(xv[u], c);
        uint32_t out[BF16 ? 4 : 8];
        decode_item<BF16>(c, s, out);
        store_item<BF16>(y, it, out);
      });
}

// ---- many tensors in one launch ------------------------------------------------
//
// A list of separate tensors (say every Linear weight of a model) quantized
// or fake-quantized by one launch: a launch per tensor pays the per-kernel
// ramp-up and drain each time (a 3 Mi-element weight runs at a quarter of the
// streaming rate on its own). The descriptors travel by value in the kernel
// arguments (no device table, nothing to copy or allocate; capturable). Tile
// t of the launch belongs to the tensor whose first tile is the largest
// tile0 <= t (a binary search on uniform values, so scalar work); a
// tensor's last tile may be partial and takes the per-item checks.

template <int U, typename Load, typename Use>
__device__ __forceinline__ void tile_at(int64_t t, int64_t nitems, Load load, Use use) {
  const int64_t tile = (int64_t)kThreads * U;
  const int64_t base = t * tile + threadIdx.x;
  if ((t + 1) * tile <= nitems) {
#pragma unroll
    for (int u = 0; u < U; u++) load(u, base + u * kThreads);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; u++) use(u, base + u * kThreads);
  } else {
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * kThreads < nitems) load(u, base + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; u++)  // whole quads drop out together
      if (base + u * kThreads < nitems) use(u, base + u * kThreads);
  }
}

struct MultiDesc {
  const void *x;    // input [rows, k]
  void *out;        // quantize: codes; fake-quant: y
  uint8_t *scales;  // quantize: scales; fake-quant: unused
  int64_t nitems;   // rows * k / 8
  int64_t tile0;    // first tile of this tensor in the launch
};
struct MultiArgs {
  int count;
  int64_t ntiles;  // tiles of the whole launch
  MultiDesc d[MX_MULTI_MAX];
};

__device__ __forceinline__ int multi_find(const MultiArgs &a, int64_t t) {
  int lo = 0, hi = a.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.d[mid].tile0 <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <bool BF16, int MODE, bool FQ>
__global__ __launch_bounds__(kThreads) void k_multi(const MultiArgs a) {
  constexpr int U = unroll_of(BF16, MODE, FQ ? kKindFakequant : kKindQuantize);
  Item<BF16> xv[U];
  for (int64_t t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
    const int j = multi_find(a, t);
    const MultiDesc &d = a.d[j];
    const void *x = d.x;
    tile_at<U>(
        t - d.tile0, d.nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
        [&](int u, int64_t it) {
          uint32_t c;
          const uint32_t s = quantize_item<BF16, MODE>(xv[u], c);
          if constexpr (FQ) {
            uint32_t out[BF16 ? 4 : 8];
            decode_item<BF16>(c, s, out);
            store_item<BF16>(d.out, it, out);
          } else {
            st<false>(static_cast<uint32_t *>(d.out) + it, c);
            if ((threadIdx.x & 3) == 0) st<false>(d.scales + (it >> 2), (uint8_t)s);
          }
        });
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequantize(const uint32_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         void *__restrict__ y, int64_t nitems) {
  constexpr int U = unroll_of(BF16, 0, kKindDequantize);
  uint32_t cw[U], sb[U];
  tile_loop<U>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(scales + (it >> 2));
      },
      [&](int u, int64_t it) {
        uint32_t out[BF16 ? 4 : 8];
        decode_item<BF16>(cw[u], sb[u], out);
        store_item<BF16>(y, it, out);
      });
}

// Block error. Per block: SSE = sum (x - x_hat)^2 in fp64 (quad sum in a
// fixed order), block_mse = (float)(SSE / 32). The tensor sums (SSE and
// sum x^2) are taken in two stages with fixed order and no atomics: each
// workgroup writes its two sums to partial[2 * blockIdx.x + {0, 1}] (lane
// sums, then a butterfly over the wave, then the waves in order), and
// k_sum_partials adds the partials.
// Block error of one item against (c, s): the fp64 SSE of the quad's block,
// summed in a fixed order (per lane, then quad_sum_f64), written as
// block_mse[block] = SSE / 32 by the quad's lane 0 when block_mse is set;
// lane 0 also adds the SSE to `mine`, and every lane adds its sum of x^2 to
// `mine_sq` (tensor sums).
template <bool BF16, bool SUMS>
__device__ __forceinline__ void mse_item(const Item<BF16> &x, uint32_t c, uint32_t s, int64_t it,
                                         float *__restrict__ block_mse, double &mine,
                                         double &mine_sq) {
  float q[8];
  decode_f32(c, s, q);
  double acc = 0.0, acc_sq = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const double xi = (double)elem<BF16>(x, i);
    const double d = xi - (double)q[i];
    acc = __builtin_fma(d, d, acc);
    if constexpr (SUMS) acc_sq = __builtin_fma(xi, xi, acc_sq);
  }
  if constexpr (SUMS) {
    // materialize here, so the eight widened x values die now instead
    // of living across the quad sum (keeps the kernel at full occupancy)
    __asm__ volatile("" : "+v"(acc_sq));
    mine_sq += acc_sq;
  }
  const double sse = quad_sum_f64(acc);
  if ((threadIdx.x & 3) == 0) {
    if (block_mse) st<false>(block_mse + (it >> 2), (float)(sse * (1.0 / 32.0)));
    if constexpr (SUMS) mine += sse;
  }
}

// The workgroup's two tensor sums, in a fixed order (butterfly over each
// wave, then the waves in turn), to partial[2 * blockIdx.x + {0, 1}].
__device__ __forceinline__ void write_partials(double mine, double mine_sq,
                                               double *__restrict__ partial) {
  __shared__ double wave_part[2][kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mine += __shfl_xor(mine, off, 64);
    mine_sq += __shfl_xor(mine_sq, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    wave_part[0][threadIdx.x >> 6] = mine;
    wave_part[1][threadIdx.x >> 6] = mine_sq;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; w++) t += wave_part[threadIdx.x][w];
    partial[2 * blockIdx.x + threadIdx.x] = t;
  }
}

// Items per thread of the block-MSE kernel, both dtypes (it sizes the grid,
// hence the workspace, per shape): two measured 3 % faster than four on bf16
// 8192x4096 with the same per-block results.
constexpr int kMseU = 2;

template <bool BF16, bool SUMS>
__global__ __launch_bounds__(kThreads) void k_block_mse(const void *__restrict__ x,
                                                        const uint32_t *__restrict__ codes,
                                                        const uint8_t *__restrict__ scales,
                                                        float *__restrict__ block_mse,
                                                        double *__restrict__ partial,
                                                        int64_t nitems) {
  double mine = 0.0;     // sum of the block SSEs this lane reports (q == 0 lanes)
  double mine_sq = 0.0;  // sum of x^2 over this lane's elements
  Item<BF16> xv[kMseU];
  uint32_t cw[kMseU], sb[kMseU];
  tile_loop<kMseU>(
      nitems,
      [&](int u, int64_t it) {
        load_item<BF16>(x, it, xv[u]);
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(scales + (it >> 2));
      },
      [&](int u, int64_t it) {
        mse_item<BF16, SUMS>(xv[u], cw[u], sb[u], it, block_mse, mine, mine_sq);
      });
  if constexpr (SUMS) write_partials(mine, mine_sq, partial);
}

// One pass: quantize, and optionally the dequantized tensor y (x's dtype)
// and the block / tensor error of the new codes, all from the x already in
// registers. Same item code as k_quantize, k_fakequant and k_block_mse, so
// the outputs equal those three calls in sequence (the tensor sums up to
// their summation order: this launch's grid is the block-MSE grid).
template <bool BF16, int MODE, bool SUMS>
__global__ __launch_bounds__(kThreads) void k_quantize_fused(const void *__restrict__ x,
                                                             uint32_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales,
                                                             void *__restrict__ y,
                                                             float *__restrict__ block_mse,
                                                             double *__restrict__ partial,
                                                             int64_t nitems) {
  double mine = 0.0, mine_sq = 0.0;
  const bool err = block_mse != nullptr || SUMS;
  // (the grid is sized like the block-MSE grid but with kUnroll items per
  // thread, so the block-MSE workspace holds its partials; the grid stride
  // makes any per-thread count correct. Two bf16 items per thread, as for
  // fake-quant: 2.4 % faster than four on 8192x4096.)
  constexpr int U = BF16 ? 2 : kU<false>;
  Item<BF16> xv[U];
  tile_loop<U>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t it) {
        uint32_t c;
        const uint32_t s = quantize_item<BF16, MODE>(xv[u], c);
        st<false>(codes + it, c);
        if ((threadIdx.x & 3) == 0) st<false>(scales + (it >> 2), (uint8_t)s);
        if (y) {  // uniform
          uint32_t out[BF16 ? 4 : 8];
          decode_item<BF16>(c, s, out);
          store_item<BF16>(y, it, out);
        }
        if (err) mse_item<BF16, SUMS>(xv[u], c, s, it, block_mse, mine, mine_sq);
      });
  if constexpr (SUMS) write_partials(mine, mine_sq, partial);
}

#ifndef MX_MSE_GRID_CAP
#define MX_MSE_GRID_CAP 2048
#endif
constexpr int kSumPer = MX_MSE_GRID_CAP / kThreads;  // partial pairs per thread
static_assert(kSumPer * kThreads == MX_MSE_GRID_CAP, "grid cap must be a multiple of 256");

// One workgroup: out[j] = sum over i of partial[2i + j] for j = 0, 1, n <=
// MX_MSE_GRID_CAP pairs. The kernel is latency-bound, so every thread issues
// all of its loads (pairs t, t + 256, ...) before the first add; the sums then
// run in a fixed order (per thread in pair order, a butterfly over the wave,
// the four waves in order), so the result is deterministic. n == 0 writes 0.
__global__ __launch_bounds__(kThreads) void k_sum_partials(const double *__restrict__ partial,
                                                           int n, double *__restrict__ out) {
  __shared__ double wave_part[2][kThreads / 64];
  if (n <= 0) {
    if (threadIdx.x < 2) out[threadIdx.x] = 0.0;
    return;
  }
  // unconditional loads of a clamped (in-bounds) index, so none waits on a
  // branch; pairs past n are then replaced by zero
  double v0[kSumPer], v1[kSumPer];
#pragma unroll
  for (int j = 0; j < kSumPer; j++) {
    const int i = (int)threadIdx.x + j * kThreads;
    const int ic = min(i, n - 1);
    const double a = partial[2 * ic], b = partial[2 * ic + 1];
    v0[j] = i < n ? a : 0.0;
    v1[j] = i < n ? b : 0.0;
  }
  double t0 = 0.0, t1 = 0.0;
#pragma unroll
  for (int j = 0; j < kSumPer; j++) {
    t0 += v0[j];
    t1 += v1[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    t0 += __shfl_xor(t0, off, 64);
    t1 += __shfl_xor(t1, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    wave_part[0][threadIdx.x >> 6] = t0;
    wave_part[1][threadIdx.x >> 6] = t1;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) t += wave_part[threadIdx.x][w];
    out[threadIdx.x] = t;
  }
}

// ---- MXFP8 (E4M3 elements) --------------------------------------------------
//
// Same blocks and lane layout; one code byte per element, so an item's 8
// codes are two 32-bit words (8 bytes per lane, 512 contiguous bytes per
// wave). Scale: floor(log2 amax) - 8 + 127 = exponent field - 8 (0 below),
// 255 for NaN/Inf blocks. Elements use the gfx950 scaled FP8 converts
// (v_cvt_scalef32_pk_fp8_{bf16,f32}: two values / 2^(s-127) -> two E4M3
// bytes, first value in the low byte, nearest-even; v_cvt_scalef32_pk_
// {bf16,f32}_fp8 back). These matched the oracle on every finite bf16 value
// at every scale byte the rule produces, and every code byte at every scale
// byte, with two differences handled here: the encode does not saturate
// (values past the 448 midpoint become NaN), so elements are first clamped
// to +-448 * 2^(s-127) (an unsigned min of the |x| bit patterns, which order
// like the values); and NaN decodes carry the sign bit, so NaN outputs are
// rewritten to the canonical quiet NaN.

__device__ __forceinline__ uint32_t mxfp8_scale_byte(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 255u;
  const uint32_t e = amax_bits >> 23;
  return e > 8u ? e - 8u : 0u;
}

// 8 E4M3 codes of the item at scale byte s (finite block), element i in
// byte i of the pair of words.
template <bool BF16>
__device__ __forceinline__ u32x2 encode8_item(const Item<BF16> &x, uint32_t s) {
  const float sc = scale_operand(s);
  s16x2 w0 = {0, 0}, w1 = {0, 0};
  if constexpr (BF16) {
    // 448 * 2^(s-127) as bf16 bits (exponent field s + 8 <= 254 for finite input)
    const uint32_t lim = ((s + 8u) << 7) | 0x60u;
    const u16x2 lim2 = {(uint16_t)lim, (uint16_t)lim};
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u16x2 a = __builtin_bit_cast(u16x2, x.w[j] & 0x7FFF7FFFu);
      c[j] = (x.w[j] & 0x80008000u) | __builtin_bit_cast(uint32_t, __builtin_elementwise_min(a, lim2));
    }
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w0, __builtin_bit_cast(bf16x2, c[0]), sc, false);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w0, __builtin_bit_cast(bf16x2, c[1]), sc, true);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w1, __builtin_bit_cast(bf16x2, c[2]), sc, false);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w1, __builtin_bit_cast(bf16x2, c[3]), sc, true);
  } else {
    const float lim = __uint_as_float(((s + 8u) << 23) | 0x600000u);
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; i++) f[i] = __builtin_amdgcn_fmed3f(__uint_as_float(x.w[i]), -lim, lim);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, f[0], f[1], sc, false);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, f[2], f[3], sc, true);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, f[4], f[5], sc, false);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, f[6], f[7], sc, true);
  }
  return u32x2{__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1)};
}

// Codes of a NaN/Inf block: the sign bit alone, one byte per element.
template <bool BF16>
__device__ __forceinline__ u32x2 sign_codes8(const Item<BF16> &x) {
  uint32_t b[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t sgn = BF16 ? (x.w[i >> 1] >> ((i & 1) ? 31 : 15)) & 1u : x.w[i] >> 31;
    b[i >> 2] |= (sgn << 7) << (8 * (i & 3));
  }
  return u32x2{b[0], b[1]};
}

template <bool BF16>
__device__ __forceinline__ uint32_t quantize8_item(const Item<BF16> &x, u32x2 &codes) {
  const uint32_t s = mxfp8_scale_byte(quad_max_u32(item_amax_bits<BF16>(x)));
  if (__builtin_expect(s == 255u, 0)) {
    codes = sign_codes8<BF16>(x);
    return s;
  }
  codes = encode8_item<BF16>(x, s);
  return s;
}

// Decode 8 E4M3 codes at byte s into output words (bf16: 4, fp32: 8). NaN
// codes and byte 255 give the canonical quiet NaN.
template <bool BF16>
__device__ __forceinline__ void decode8_item(u32x2 c, uint32_t s, uint32_t (&y)[BF16 ? 4 : 8]) {
  const float sc = scale_operand(s);
  if constexpr (BF16) {
    y[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, false));
    y[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, true));
    y[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, false));
    y[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, true));
#pragma unroll
    for (int j = 0; j < 4; j++) {
      // a NaN half (exponent all ones, mantissa non-zero) loses its sign bit
      const u16x2 a = __builtin_bit_cast(u16x2, y[j] & 0x7FFF7FFFu);
      const s16x2 nan = a > (u16x2){0x7F80, 0x7F80};  // lanes: -1 where NaN
      const uint32_t keep = ~(__builtin_bit_cast(uint32_t, nan) & 0x80008000u);
      y[j] &= keep;
    }
    if (__builtin_expect(s == 255u, 0)) {
#pragma unroll
      for (int j = 0; j < 4; j++) y[j] = kNaN16x2;
    }
  } else {
    f32x2 v[4];
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[0], sc, false);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[0], sc, true);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[1], sc, false);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[1], sc, true);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      y[2 * j] = __float_as_uint(v[j].x);
      y[2 * j + 1] = __float_as_uint(v[j].y);
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
      if ((y[i] & 0x7FFFFFFFu) > 0x7F800000u) y[i] = kNaN32;
    if (__builtin_expect(s == 255u, 0)) {
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = kNaN32;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_quantize8(const void *__restrict__ x,
                                                        u32x2 *__restrict__ codes,
                                                        uint8_t *__restrict__ scales,
                                                        int64_t nitems) {
  Item<BF16> xv[kU<BF16>];
  tile_loop<kU<BF16>>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t it) {
        u32x2 c;
        const uint32_t s = quantize8_item<BF16>(xv[u], c);
        st<false>(codes + it, c);
        if ((threadIdx.x & 3) == 0) st<false>(scales + (it >> 2), (uint8_t)s);
      });
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequantize8(const u32x2 *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          void *__restrict__ y, int64_t nitems) {
  u32x2 cw[kU<BF16>];
  uint32_t sb[kU<BF16>];
  tile_loop<kU<BF16>>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(scales + (it >> 2));
      },
      [&](int u, int64_t it) {
        uint32_t out[BF16 ? 4 : 8];
        decode8_item<BF16>(cw[u], sb[u], out);
        store_item<BF16>(y, it, out);
      });
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_fakequant8(const void *x, void *y, int64_t nitems) {
  constexpr int U = unroll_of(BF16, 0, kKindFakequant);  // as MXFP4 fake-quant (3 % faster)
  Item<BF16> xv[U];
  tile_loop<U>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t it) {
        u32x2 c;
        const uint32_t s = quantize8_item<BF16>(xv[u], c);
        uint32_t out[BF16 ? 4 : 8];
        decode8_item<BF16>(c, s, out);
        store_item<BF16>(y, it, out);
      });
}

// ---- NVFP4 comparator (16-element blocks, E4M3 block scales) ----------------
//
// Two lanes per 16-element block (an item is half a block); the pair's max
// is one DPP step. A per-tensor power of two S = 2^t, the largest with
// S * amax <= 2688 (6 * 448), keeps the block scales inside E4M3; amax is
// the largest finite |x| of the tensor (first pass, per-workgroup maxima).
// Block scale: E4M3 nearest-even of min((a_b / 6) * S, 448) (IEEE fp32
// division, exact power-of-two product); element: nearest-even E2M1,
// saturating, of x * (S / s_b) in fp32 (IEEE division for the reciprocal
// factor). E4M3 and E2M1 rounding use the scaled converts at scale 1.

#ifndef MX_NV_GRID_CAP
#define MX_NV_GRID_CAP 2048
#endif
constexpr int kNvPer = MX_NV_GRID_CAP / kThreads;  // first-pass maxima per thread
static_assert(kNvPer * kThreads == MX_NV_GRID_CAP, "grid cap must be a multiple of 256");

// Largest finite |x| bit pattern of the item (non-finite elements count as
// 0): the plain maximum when the item holds no NaN/Inf, else element by
// element.
template <bool BF16>
__device__ __forceinline__ uint32_t item_finite_amax_bits(const Item<BF16> &x) {
  const uint32_t all = item_amax_bits<BF16>(x);
  if (__builtin_expect(all < 0x7F800000u, 1)) return all;
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t a = __float_as_uint(elem<BF16>(x, i)) & 0x7FFFFFFFu;
    m = max(m, a < 0x7F800000u ? a : 0u);
  }
  return m;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_absmax_partials(const void *__restrict__ x,
                                                              uint32_t *__restrict__ partial,
                                                              int64_t nitems) {
  __shared__ uint32_t wave_max[kThreads / 64];
  uint32_t m = 0;
  Item<BF16> xv[kUnroll];
  tile_loop<kUnroll>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) { m = max(m, item_finite_amax_bits<BF16>(xv[u])); });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kThreads / 64; w++) t = max(t, wave_max[w]);
    partial[blockIdx.x] = t;
  }
}

// t of S = 2^t from the tensor amax bits: with amax = (1 + f) 2^(e - 127),
// 2^t * amax <= 1.3125 * 2^11 gives t = 138 - e when 1 + f <= 1.3125
// (mantissa field <= 0x280000), else 137 - e; capped at 127 (tiny or
// subnormal amax); amax == 0 gives t = 0.
__device__ __forceinline__ int nv_tensor_exp(uint32_t amax_bits) {
  if (amax_bits == 0u) return 0;
  const int e = (int)(amax_bits >> 23);
  const int t = (e == 0) ? 127 : ((amax_bits & 0x7FFFFFu) <= 0x280000u ? 138 - e : 137 - e);
  return t > 127 ? 127 : t;
}

__device__ __forceinline__ uint32_t dpp_x1_max(uint32_t v) { return max(v, dpp_x1(v)); }

// Decoding used by the fused fake-quant below (defined with the dequantize
// kernel).
template <bool BF16>
__device__ __forceinline__ void nv_decode_item(uint32_t c, uint32_t sbyte, float inv_s,
                                               uint32_t (&out)[BF16 ? 4 : 8]);

// FQ: fake-quant (y = dequantize(quantize(x)) in x's dtype; y may be x)
// instead of writing codes, block scales and the tensor byte.
template <bool BF16, bool FQ>
__global__ __launch_bounds__(kThreads) void k_quantize_nv(const void *x,
                                                          const uint32_t *__restrict__ partial,
                                                          int npartial,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ block_scales,
                                                          uint8_t *__restrict__ tensor_scale,
                                                          void *y, int64_t nitems) {
  // every workgroup reduces the first pass's maxima (max is order-free and
  // idempotent, so clamped duplicate loads are harmless; all loads are issued
  // before the first use), and fills a table of fl32(1 / v) for the E4M3
  // values v (code 0 -> 0; code 0x7F is NaN and never looked up)
  __shared__ uint32_t wave_max[kThreads / 64];
  __shared__ float rcp_e4m3[128];
  const float one = 1.0f;  // scale operand of the converts: 2^0
  uint32_t pv[kNvPer];
#pragma unroll
  for (int j = 0; j < kNvPer; j++) pv[j] = partial[min((int)threadIdx.x + j * kThreads, npartial - 1)];
  if (threadIdx.x < 128) {
    const float v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(threadIdx.x, one, false)[0];
    rcp_e4m3[threadIdx.x] = threadIdx.x == 0 ? 0.0f : 1.0f / v;
  }
  uint32_t a = 0;
#pragma unroll
  for (int j = 0; j < kNvPer; j++) a = max(a, pv[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kThreads / 64; w++) a = max(a, wave_max[w]);
  const int t = nv_tensor_exp(a);
  if (!FQ && blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = (uint8_t)(t + 127);
  const float S = __uint_as_float((uint32_t)(t + 127) << 23);
  const float inv_s = __uint_as_float((uint32_t)(127 - t) << 23);  // 2^-t

  Item<BF16> xv[kUnroll];
  tile_loop<kUnroll>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t it) {
        const uint32_t ab = dpp_x1_max(item_amax_bits<BF16>(xv[u]));  // NaN/Inf sort above
        uint32_t c;
        uint32_t sbyte;
        if (__builtin_expect(ab >= 0x7F800000u, 0)) {
          sbyte = 0x7Fu;
          c = sign_codes<BF16>(xv[u]);
        } else {
          const float q6 = div6(ab);
          const float tb = fminf(q6 * S, 448.0f);
          s16x2 w = {0, 0};
          w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, tb, tb, one, false);
          sbyte = (uint32_t)w[0] & 0xFFu;
          // S / s_b = 2^t * fl32(1 / s_b) exactly: scaling by a power of two
          // commutes with rounding, and 2^t / s_b is never subnormal (t >= -117,
          // s_b <= 448); both overflow to Inf together
          const float r = rcp_e4m3[sbyte] * S;
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; i++) v[i] = elem<BF16>(xv[u], i) * r;
          c = 0;
          c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[0], v[1], one, 0);
          c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[2], v[3], one, 1);
          c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[4], v[5], one, 2);
          c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[6], v[7], one, 3);
        }
        if constexpr (FQ) {
          uint32_t out[BF16 ? 4 : 8];
          nv_decode_item<BF16>(c, sbyte, inv_s, out);
          store_item<BF16>(y, it, out);
        } else {
          st<false>(codes + it, c);
          if ((threadIdx.x & 1) == 0) st<false>(block_scales + (it >> 1), (uint8_t)sbyte);
        }
      });
}

// Decoded values of one item: E2M1 code * s_b * 2^-t, exact in fp32 (at
// most 2 + 4 significant bits), rounded to bf16 if asked; block scale byte
// 0x7F (NaN) gives the canonical NaN.
template <bool BF16>
__device__ __forceinline__ void nv_decode_item(uint32_t c, uint32_t sbyte, float inv_s,
                                               uint32_t (&out)[BF16 ? 4 : 8]) {
  // s_b * 2^-t exactly (E4M3 decode with a power-of-two scale)
  const float sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sbyte, inv_s, false)[0];
  float q[8];
  decode_f32(c, 127u, q);  // E2M1 values at scale 1
  const bool nan = (sbyte & 0x7Fu) == 0x7Fu;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      const b2 p = {(__bf16)(q[2 * j] * sv), (__bf16)(q[2 * j + 1] * sv)};
      out[j] = nan ? kNaN16x2 : __builtin_bit_cast(uint32_t, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = nan ? kNaN32 : __float_as_uint(q[i] * sv);
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequantize_nv(const uint32_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ block_scales,
                                                            const uint8_t *__restrict__ tensor_scale,
                                                            void *__restrict__ y, int64_t nitems) {
  const int t = (int)*tensor_scale - 127;
  const float inv_s = __uint_as_float((uint32_t)(127 - t) << 23);  // 2^-t, scale operand
  uint32_t cw[kU<BF16>], sb[kU<BF16>];
  tile_loop<kU<BF16>>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(block_scales + (it >> 1));
      },
      [&](int u, int64_t it) {
        uint32_t out[BF16 ? 4 : 8];
        nv_decode_item<BF16>(cw[u], sb[u], inv_s, out);
        store_item<BF16>(y, it, out);
      });
}

// ---- MBS-Static (16-element sub-blocks, 8-bit-mantissa macro factor) ---------
//
// A 128-element macro block is one DPP row (16 lanes x 8 elements); a
// 16-element sub-block is a lane pair. Macro factor f = 1 + m/256, m the
// round-to-nearest-even 8-bit mantissa of fl32(a_M / 6) (capped at 255; 0 for
// a zero or non-finite macro block); y = fl32(x * fl32(1/f)); each sub-block
// takes the OCP byte of its largest |y| and the E2M1 codes of y at that
// byte (scaled convert); decoding is E2M1 * 2^(s-127) * f, exact in fp32
// (at most 2 + 9 significant bits). A sub-block holding NaN/Inf stores the
// NaN byte and the signs of x, as a NaN MXFP4 block does.

// rotate right by 4 / 8 lanes within each row of 16
__device__ __forceinline__ uint32_t dpp_ror4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
}
// Decoded values of one item: E2M1 * 2^(s-127) * (1 + m/256), exact in fp32
// (at most 2 + 9 significant bits), rounded to bf16 if asked; sub-block byte
// 255 gives the canonical NaN.
template <bool BF16>
__device__ __forceinline__ void mbs_decode_item(uint32_t c, uint32_t s, uint32_t m,
                                                uint32_t (&out)[BF16 ? 4 : 8]) {
  const float f = 1.0f + (float)m * (1.0f / 256.0f);
  float q[8];
  decode_f32(c, s, q);  // E2M1 * 2^(s-127); NaN for byte 255
  const bool nan = s == 255u;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      const b2 p = {(__bf16)(q[2 * j] * f), (__bf16)(q[2 * j + 1] * f)};
      out[j] = nan ? kNaN16x2 : __builtin_bit_cast(uint32_t, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = nan ? kNaN32 : __float_as_uint(q[i] * f);
  }
}

// The U items of one tile, in phases across the items (every item's macro
// maximum, then every factor, then every table read, then the codes) so the
// scheduler can overlap their long dependency chains; the rare cases (a
// subnormal quotient, a NaN/Inf sub-block) are patched afterwards under a
// branch that a wave without them skips.
template <bool BF16, int U, bool FQ>
__device__ __forceinline__ void mbs_tile(const Item<BF16> (&xv)[U], const float *inv_tab,
                                         uint32_t *__restrict__ codes,
                                         uint8_t *__restrict__ sub_scales,
                                         uint8_t *__restrict__ macro_mant, void *y, int64_t base,
                                         int64_t nitems, bool full) {
  uint32_t aS[U], aM[U], m[U], s[U], c[U];
  float inv[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t a8 = item_amax_bits<BF16>(xv[u]);
    aS[u] = max(a8, dpp_x1(a8));  // the sub-block's lane pair
    uint32_t v = max(aS[u], dpp_x2(aS[u]));
    v = max(v, dpp_ror4(v));
    aM[u] = max(v, dpp_ror8(v));  // the macro block's row of 16 lanes
  }
  // a_M / 6: the exact fast form (div6_fast) everywhere, then IEEE division
  // for the lanes below its range, under a branch taken only when a wave has
  // any (a macro maximum below 2^-125)
  float r[U];
  bool small = false;
#pragma unroll
  for (int u = 0; u < U; u++) {
    r[u] = div6_fast(__uint_as_float(aM[u]));
    small |= aM[u] - 1u < 0x00FFFFFFu;  // 0 < a_M < 2^-125
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(small) != 0, 0)) {
#pragma unroll
    for (int u = 0; u < U; u++)
      if (aM[u] - 1u < 0x00FFFFFFu) r[u] = __uint_as_float(aM[u]) / 6.0f;
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    // m = 0 for a zero or non-finite macro block, and where a_M / 6
    // underflows to zero (fp32 a_M below 4 * 2^-149): no mantissa
    const float t = __builtin_rintf((2.0f * __builtin_amdgcn_frexp_mantf(r[u]) - 1.0f) * 256.0f);
    const float tc = __builtin_fminf(__builtin_fmaxf(t, 0.0f), 255.0f);  // NaN -> 0
    m[u] = (aM[u] < 0x7F800000u && r[u] != 0.0f) ? (uint32_t)tc : 0u;
  }
#pragma unroll
  for (int u = 0; u < U; u++) inv[u] = inv_tab[m[u]];
#pragma unroll
  for (int u = 0; u < U; u++) {
    // largest |y| of the sub-block: rounding is monotone, so it equals
    // fl(max |x| * inv); NaN/Inf stay NaN/Inf and give byte 255
    s[u] = ocp_scale_byte(__float_as_uint(__uint_as_float(aS[u]) * inv[u]));
    const float sc = scale_operand(s[u]);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = elem<BF16>(xv[u], i) * inv[u];
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], sc, 3);
    c[u] = w;
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    if (__builtin_expect(s[u] == 255u, 0)) c[u] = sign_codes<BF16>(xv[u]);
    const int64_t it = base + u * kThreads;
    if (full || it < nitems) {  // whole rows of 16 lanes drop out together
      if constexpr (FQ) {
        uint32_t out[BF16 ? 4 : 8];
        mbs_decode_item<BF16>(c[u], s[u], m[u], out);
        store_item<BF16>(y, it, out);
      } else {
        st<false>(codes + it, c[u]);
        if ((threadIdx.x & 1) == 0) st<false>(sub_scales + (it >> 1), (uint8_t)s[u]);
        if ((threadIdx.x & 15) == 0) st<false>(macro_mant + (it >> 4), (uint8_t)m[u]);
      }
    }
  }
}

// FQ: fake-quant (y = dequantize(quantize(x)) in x's dtype; y may be x)
// instead of writing codes and bytes.
template <bool BF16, bool FQ>
__global__ __launch_bounds__(kThreads) void k_quantize_mbs(const void *x,
                                                           uint32_t *__restrict__ codes,
                                                           uint8_t *__restrict__ sub_scales,
                                                           uint8_t *__restrict__ macro_mant,
                                                           void *y, int64_t nitems) {
  // fl32(1 / f) for every macro mantissa m (f = 1 + m/256): IEEE division,
  // once per workgroup, so the per-item cost is one LDS read
  static_assert(kThreads == 256, "one table entry per thread");
  __shared__ float inv_tab[256];
  inv_tab[threadIdx.x] = 1.0f / (1.0f + (float)threadIdx.x * (1.0f / 256.0f));
  __syncthreads();
  constexpr int U = kU<BF16>;
  const int64_t tile = (int64_t)kThreads * U;
  const int64_t nfull = nitems / tile;
  Item<BF16> xv[U];
  int64_t t = blockIdx.x;
  for (; t < nfull; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++) load_item<BF16>(x, base + u * kThreads, xv[u]);
    __builtin_amdgcn_sched_barrier(0);
    mbs_tile<BF16, U, FQ>(xv, inv_tab, codes, sub_scales, macro_mant, y, base, nitems, true);
  }
  if (t == nfull && nfull * tile < nitems) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (base + u * kThreads < nitems) load_item<BF16>(x, base + u * kThreads, xv[u]);
      else xv[u] = Item<BF16>{};  // zeros: finite, so lanes past the end stay quiet
    }
    mbs_tile<BF16, U, FQ>(xv, inv_tab, codes, sub_scales, macro_mant, y, base, nitems, false);
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequantize_mbs(const uint32_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ sub_scales,
                                                             const uint8_t *__restrict__ macro_mant,
                                                             void *__restrict__ y, int64_t nitems) {
  // items per thread as MXFP4 dequantize (two for bf16: 2.5 % faster here)
  constexpr int U = unroll_of(BF16, 0, kKindDequantize);
  uint32_t cw[U], sb[U], mb[U];
  tile_loop<U>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(sub_scales + (it >> 1));
        mb[u] = ld<false>(macro_mant + (it >> 4));
      },
      [&](int u, int64_t it) {
        uint32_t out[BF16 ? 4 : 8];
        mbs_decode_item<BF16>(cw[u], sb[u], mb[u], out);
        store_item<BF16>(y, it, out);
      });
}

// ---- launchers -----------------------------------------------------------------

static unsigned grid_for(int64_t nitems, int64_t cap, int unroll = kUnroll) {
  const int64_t tile = (int64_t)kThreads * unroll;
  int64_t g = (nitems + tile - 1) / tile;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace mxk

using namespace mxk;

#define MX_DISPATCH_MULTI(BF16, FQ, MODE, G, B, ST, ARGS)                                 \
  switch (MODE) {                                                                          \
    case MX_SCALE_OAS:                                                                     \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OAS, FQ>), G, B, 0, ST, ARGS);            \
      break;                                                                               \
    case MX_SCALE_OAS_BITS:                                                                \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OAS_BITS, FQ>), G, B, 0, ST, ARGS);       \
      break;                                                                               \
    case MX_SCALE_OAS_NF:                                                                  \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OAS_NF, FQ>), G, B, 0, ST, ARGS);         \
      break;                                                                               \
    default:                                                                               \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OCP, FQ>), G, B, 0, ST, ARGS);            \
      break;                                                                               \
  }

#define MX_DISPATCH_MODE(KERNEL, BF16, MODE, G, B, ST, ...)                               \
  switch (MODE) {                                                                          \
    case MX_SCALE_OAS:                                                                     \
      hipLaunchKernelGGL((KERNEL<BF16, MX_SCALE_OAS>), G, B, 0, ST, __VA_ARGS__);          \
      break;                                                                               \
    case MX_SCALE_OAS_BITS:                                                                \
      hipLaunchKernelGGL((KERNEL<BF16, MX_SCALE_OAS_BITS>), G, B, 0, ST, __VA_ARGS__);     \
      break;                                                                               \
    case MX_SCALE_OAS_NF:                                                                  \
      hipLaunchKernelGGL((KERNEL<BF16, MX_SCALE_OAS_NF>), G, B, 0, ST, __VA_ARGS__);       \
      break;                                                                               \
    default:                                                                               \
      hipLaunchKernelGGL((KERNEL<BF16, MX_SCALE_OCP>), G, B, 0, ST, __VA_ARGS__);          \
      break;                                                                               \
  }

hipError_t mxi_launch_quantize(const void *x, int bf16, int mode, int64_t nitems,
                               uint8_t *codes, uint8_t *scales, hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, unroll_of(bf16, mode, kKindQuantize))), b(kThreads);
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  if (bf16) {
    MX_DISPATCH_MODE(k_quantize, true, mode, g, b, st, x, c, scales, nitems)
  } else {
    MX_DISPATCH_MODE(k_quantize, false, mode, g, b, st, x, c, scales, nitems)
  }
  return hipGetLastError();
}

hipError_t mxi_launch_fakequant(const void *x, int bf16, int mode, int64_t nitems, void *y,
                                hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, unroll_of(bf16, mode, kKindFakequant))), b(kThreads);
  if (bf16) {
    MX_DISPATCH_MODE(k_fakequant, true, mode, g, b, st, x, y, nitems)
  } else {
    MX_DISPATCH_MODE(k_fakequant, false, mode, g, b, st, x, y, nitems)
  }
  return hipGetLastError();
}

hipError_t mxi_launch_dequantize(const uint8_t *codes, const uint8_t *scales, int bf16,
                                 int64_t nitems, void *y, hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, unroll_of(bf16, 0, kKindDequantize))), b(kThreads);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  if (bf16)
    hipLaunchKernelGGL((k_dequantize<true>), g, b, 0, st, c, scales, y, nitems);
  else
    hipLaunchKernelGGL((k_dequantize<false>), g, b, 0, st, c, scales, y, nitems);
  return hipGetLastError();
}

// (the one-pass kernel's grid, sized with kUnroll items per thread, is
// never larger than this one, so the same workspace serves it)
size_t mxi_block_mse_partials(int64_t nitems) {
  return 2 * grid_for(nitems, MX_MSE_GRID_CAP, kMseU);
}

hipError_t mxi_launch_block_mse(const void *x, int bf16, const uint8_t *codes,
                                const uint8_t *scales, int64_t nitems, float *block_mse,
                                double *tensor_sums, double *partial, hipStream_t st) {
  const unsigned grid = grid_for(nitems, MX_MSE_GRID_CAP, kMseU);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  double *part = tensor_sums ? partial : nullptr;
  if (nitems > 0) {
    const dim3 g(grid), b(kThreads);
    if (bf16) {
      if (part)
        hipLaunchKernelGGL((k_block_mse<true, true>), g, b, 0, st, x, c, scales, block_mse, part,
                           nitems);
      else
        hipLaunchKernelGGL((k_block_mse<true, false>), g, b, 0, st, x, c, scales, block_mse,
                           part, nitems);
    } else {
      if (part)
        hipLaunchKernelGGL((k_block_mse<false, true>), g, b, 0, st, x, c, scales, block_mse,
                           part, nitems);
      else
        hipLaunchKernelGGL((k_block_mse<false, false>), g, b, 0, st, x, c, scales, block_mse,
                           part, nitems);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tensor_sums) {
    hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(kThreads), 0, st, partial,
                       nitems > 0 ? (int)grid : 0, tensor_sums);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t mxi_launch_quantize8(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                uint8_t *scales, hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, bf16 ? kU<true> : kU<false>)), b(kThreads);
  u32x2 *c = reinterpret_cast<u32x2 *>(codes);
  if (bf16)
    hipLaunchKernelGGL((k_quantize8<true>), g, b, 0, st, x, c, scales, nitems);
  else
    hipLaunchKernelGGL((k_quantize8<false>), g, b, 0, st, x, c, scales, nitems);
  return hipGetLastError();
}

hipError_t mxi_launch_dequantize8(const uint8_t *codes, const uint8_t *scales, int bf16,
                                  int64_t nitems, void *y, hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, bf16 ? kU<true> : kU<false>)), b(kThreads);
  const u32x2 *c = reinterpret_cast<const u32x2 *>(codes);
  if (bf16)
    hipLaunchKernelGGL((k_dequantize8<true>), g, b, 0, st, c, scales, y, nitems);
  else
    hipLaunchKernelGGL((k_dequantize8<false>), g, b, 0, st, c, scales, y, nitems);
  return hipGetLastError();
}

hipError_t mxi_launch_fakequant8(const void *x, int bf16, int64_t nitems, void *y,
                                 hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, unroll_of(bf16, 0, kKindFakequant))), b(kThreads);
  if (bf16)
    hipLaunchKernelGGL((k_fakequant8<true>), g, b, 0, st, x, y, nitems);
  else
    hipLaunchKernelGGL((k_fakequant8<false>), g, b, 0, st, x, y, nitems);
  return hipGetLastError();
}

size_t mxi_nvfp4_partials(int64_t nitems) { return grid_for(nitems, MX_NV_GRID_CAP); }

hipError_t mxi_launch_quantize_nv(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                  uint8_t *block_scales, uint8_t *tensor_scale,
                                  uint32_t *partial, void *y, hipStream_t st) {
  const unsigned gp = grid_for(nitems, MX_NV_GRID_CAP);
  const dim3 g(gp), b(kThreads);
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  if (bf16) {
    hipLaunchKernelGGL((k_absmax_partials<true>), dim3(gp), b, 0, st, x, partial, nitems);
    if (y)
      hipLaunchKernelGGL((k_quantize_nv<true, true>), g, b, 0, st, x, partial, (int)gp, c,
                         block_scales, tensor_scale, y, nitems);
    else
      hipLaunchKernelGGL((k_quantize_nv<true, false>), g, b, 0, st, x, partial, (int)gp, c,
                         block_scales, tensor_scale, y, nitems);
  } else {
    hipLaunchKernelGGL((k_absmax_partials<false>), dim3(gp), b, 0, st, x, partial, nitems);
    if (y)
      hipLaunchKernelGGL((k_quantize_nv<false, true>), g, b, 0, st, x, partial, (int)gp, c,
                         block_scales, tensor_scale, y, nitems);
    else
      hipLaunchKernelGGL((k_quantize_nv<false, false>), g, b, 0, st, x, partial, (int)gp, c,
                         block_scales, tensor_scale, y, nitems);
  }
  return hipGetLastError();
}

hipError_t mxi_launch_dequantize_nv(const uint8_t *codes, const uint8_t *block_scales,
                                    const uint8_t *tensor_scale, int bf16, int64_t nitems, void *y,
                                    hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, bf16 ? kU<true> : kU<false>)), b(kThreads);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  if (bf16)
    hipLaunchKernelGGL((k_dequantize_nv<true>), g, b, 0, st, c, block_scales, tensor_scale, y,
                       nitems);
  else
    hipLaunchKernelGGL((k_dequantize_nv<false>), g, b, 0, st, c, block_scales, tensor_scale, y,
                       nitems);
  return hipGetLastError();
}

hipError_t mxi_launch_quantize_mbs(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                   uint8_t *sub_scales, uint8_t *macro_mant, void *y,
                                   hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, bf16 ? kU<true> : kU<false>)), b(kThreads);
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  if (bf16) {
    if (y)
      hipLaunchKernelGGL((k_quantize_mbs<true, true>), g, b, 0, st, x, c, sub_scales, macro_mant,
                         y, nitems);
    else
      hipLaunchKernelGGL((k_quantize_mbs<true, false>), g, b, 0, st, x, c, sub_scales,
                         macro_mant, y, nitems);
  } else {
    if (y)
      hipLaunchKernelGGL((k_quantize_mbs<false, true>), g, b, 0, st, x, c, sub_scales,
                         macro_mant, y, nitems);
    else
      hipLaunchKernelGGL((k_quantize_mbs<false, false>), g, b, 0, st, x, c, sub_scales,
                         macro_mant, y, nitems);
  }
  return hipGetLastError();
}

hipError_t mxi_launch_dequantize_mbs(const uint8_t *codes, const uint8_t *sub_scales,
                                     const uint8_t *macro_mant, int bf16, int64_t nitems, void *y,
                                     hipStream_t st) {
  const dim3 g(grid_for(nitems, MX_GRID_CAP, unroll_of(bf16, 0, kKindDequantize))),
      b(kThreads);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  if (bf16)
    hipLaunchKernelGGL((k_dequantize_mbs<true>), g, b, 0, st, c, sub_scales, macro_mant, y, nitems);
  else
    hipLaunchKernelGGL((k_dequantize_mbs<false>), g, b, 0, st, c, sub_scales, macro_mant, y,
                       nitems);
  return hipGetLastError();
}

hipError_t mxi_launch_multi(const MxiTensor *t, int count, int bf16, int mode, int fakequant,
                            hipStream_t st) {
  // chunks of at most MX_MULTI_MAX non-empty tensors, one launch each
  int i = 0;
  while (i < count) {
    MultiArgs a;
    a.count = 0;
    int64_t tiles = 0;
    const int64_t tile =
        (int64_t)kThreads * unroll_of(bf16, mode, fakequant ? kKindFakequant : kKindQuantize);
    for (; i < count && a.count < MX_MULTI_MAX; i++) {
      if (t[i].nitems <= 0) continue;
      MultiDesc &d = a.d[a.count++];
      d.x = t[i].x;
      d.out = t[i].out;
      d.scales = t[i].scales;
      d.nitems = t[i].nitems;
      d.tile0 = tiles;
      tiles += (t[i].nitems + tile - 1) / tile;
    }
    if (a.count == 0) break;
    a.ntiles = tiles;
    const dim3 g((unsigned)(tiles < MX_GRID_CAP ? tiles : MX_GRID_CAP)), b(kThreads);
    if (bf16) {
      if (fakequant) { MX_DISPATCH_MULTI(true, true, mode, g, b, st, a) }
      else { MX_DISPATCH_MULTI(true, false, mode, g, b, st, a) }
    } else {
      if (fakequant) { MX_DISPATCH_MULTI(false, true, mode, g, b, st, a) }
      else { MX_DISPATCH_MULTI(false, false, mode, g, b, st, a) }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

#define MX_DISPATCH_FUSED(BF16, SUMS, MODE, G, B, ST, ...)                                 \
  switch (MODE) {                                                                          \
    case MX_SCALE_OAS:                                                                     \
      hipLaunchKernelGGL((k_quantize_fused<BF16, MX_SCALE_OAS, SUMS>), G, B, 0, ST, __VA_ARGS__); \
      break;                                                                               \
    case MX_SCALE_OAS_BITS:                                                                \
      hipLaunchKernelGGL((k_quantize_fused<BF16, MX_SCALE_OAS_BITS, SUMS>), G, B, 0, ST,   \
                         __VA_ARGS__);                                                     \
      break;                                                                               \
    case MX_SCALE_OAS_NF:                                                                  \
      hipLaunchKernelGGL((k_quantize_fused<BF16, MX_SCALE_OAS_NF, SUMS>), G, B, 0, ST,     \
                         __VA_ARGS__);                                                     \
      break;                                                                               \
    default:                                                                               \
      hipLaunchKernelGGL((k_quantize_fused<BF16, MX_SCALE_OCP, SUMS>), G, B, 0, ST, __VA_ARGS__); \
      break;                                                                               \
  }

hipError_t mxi_launch_quantize_fused(const void *x, int bf16, int mode, int64_t nitems,
                                     uint8_t *codes, uint8_t *scales, void *y, float *block_mse,
                                     double *tensor_sums, double *partial, hipStream_t st) {
  // the block-MSE grid, so the partial sums fit mx_block_mse_workspace_size
  const unsigned grid = grid_for(nitems, MX_MSE_GRID_CAP);
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  double *part = tensor_sums ? partial : nullptr;
  if (nitems > 0) {
    const dim3 g(grid), b(kThreads);
    if (bf16) {
      if (part) { MX_DISPATCH_FUSED(true, true, mode, g, b, st, x, c, scales, y, block_mse, part, nitems) }
      else { MX_DISPATCH_FUSED(true, false, mode, g, b, st, x, c, scales, y, block_mse, part, nitems) }
    } else {
      if (part) { MX_DISPATCH_FUSED(false, true, mode, g, b, st, x, c, scales, y, block_mse, part, nitems) }
      else { MX_DISPATCH_FUSED(false, false, mode, g, b, st, x, c, scales, y, block_mse, part, nitems) }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tensor_sums) {
    hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(kThreads), 0, st, partial,
                       nitems > 0 ? (int)grid : 0, tensor_sums);
    return hipGetLastError();
  }
  return hipSuccess;
}
