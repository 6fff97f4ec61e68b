// mx_kernels.hip - gfx950 kernels for OCP MXFP4 block quantization.
//
// Work decomposition (all ops): the tensor is a flat run of 32-element MX
// blocks (rows are contiguous and k % 32 == 0, so block b covers elements
// 32b..32b+31 and owns scale byte b and code bytes 16b..16b+15). A block is
// handled by a quad of 4 adjacent lanes; lane q of the quad owns elements
// 8q..8q+7 ("item" = 8 elements = one 16-byte bf16 load, one 32-bit code
// word). A wave64 covers 16 blocks per item step: 1 KiB of bf16 in, 256 B of
// codes and 16 B of scales out, all contiguous. (OAS_NF quantize of smaller
// bf16 tensors gives each block to a lane pair instead; see "two lanes per
// block".)
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

#include <algorithm>
#include <mutex>
#include <vector>

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
// Most workgroups a launch of the other formats' kernels uses below the
// multi-GB size (beyond it, workgroups loop over tiles). Measured on a
// 2.1e9-element bf16 tensor with four items per thread: 196,608 (768 per CU)
// beat 65,536 by 5 % (quantize) and 3 % (dequantize), while 8,192-32,768
// were slower. The MXFP4 single-tensor kernels, and the other formats'
// multi-GB bf16 tilings, are not capped (see kGridLimit). Below the cap
// every workgroup takes one tile: tensors up to ~1.6e9 elements with four
// items per thread, ~4e8 with one.
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

// rotate right by 4 / 8 lanes within each row of 16
__device__ __forceinline__ uint32_t dpp_ror4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
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

// Sum of the 16 lanes of a row on every lane of the row: the quad sums, then
// the other quads' sums rotated in (4 lanes, then 8), in one fixed order.
__device__ __forceinline__ double row_sum_f64(double p) {
  p = quad_sum_f64(p);
  uint64_t u = __double_as_longlong(p);
  p = p + __longlong_as_double(((uint64_t)dpp_ror4((uint32_t)(u >> 32)) << 32) |
                               dpp_ror4((uint32_t)u));
  u = __double_as_longlong(p);
  p = p + __longlong_as_double(((uint64_t)dpp_ror8((uint32_t)(u >> 32)) << 32) |
                               dpp_ror8((uint32_t)u));
  return p;
}

// ---- memory helpers -----------------------------------------------------------

// Streaming accesses. Each bf16 item is one 16-byte access and a wave's 64
// accesses cover 1 KiB contiguously, so bf16 tensors are read and written
// with the non-temporal hint (no reuse; fewer dirty L2 lines to write back
// at the end of the kernel). fp32 items take two 16-byte accesses whose
// per-instruction footprint is strided (32-byte lane pitch): fp32 loads,
// and the small code/scale accesses, stay on the default cache policy,
// which measured faster for them (the code-word stores of the narrow
// multi-GB quantize tilings excepted: see nt_codes); fp32 stores are
// regrouped through LDS into contiguous non-temporal stores (store_item).
// The per-block errors (one 4-byte store per quad) are stored
// non-temporally too: on the 2.8e9-element weight set block MSE with its
// tensor sums took 1197 us against 1226-1240 us on the default policy.
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

// Lane share of the pinned fp32 block squared error at candidate byte c,
// measured in units of the larger candidate's scale 2^(h-127) (h >= c): each
// element error is d = x * 2^(127-h) - x_hat * 2^(127-h), formed exactly and
// rounded once by one fma (x_hat is decoded straight at byte 127 + c - h);
// even positions go to one fma accumulator and odd to another, lane share =
// even + odd. Returns the candidate's codes too.
template <bool BF16>
__device__ __forceinline__ float lane_sse(const Item<BF16> &x, uint32_t c, uint32_t h,
                                          uint32_t &codes) {
  codes = encode_item<BF16>(x, c);
  float q[8];
  decode_f32(codes, 127u + c - h, q);
  const float unit = __uint_as_float((254u - h) << 23);  // 2^(127-h), 1 <= h <= 252
  float acc_e = 0.0f, acc_o = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float d0 = __builtin_fmaf(elem<BF16>(x, i), unit, -q[i]);
    const float d1 = __builtin_fmaf(elem<BF16>(x, i + 1), unit, -q[i + 1]);
    acc_e = __builtin_fmaf(d0, d0, acc_e);
    acc_o = __builtin_fmaf(d1, d1, acc_o);
  }
  return acc_e + acc_o;
}

// Block scale byte and this lane's codes, for either lane layout of a block
// (four lanes of 8 elements, or two lanes of 16). amax is the block's largest
// |x| bit pattern, held by every lane of the block; encode(s) returns this
// lane's codes at byte s, sign() its codes for a NaN/Inf block, and
// block_sse(c, h, codes) stores its codes at candidate byte c and returns the
// block's pinned fp32 error at c in units of 2^(h-127), summed over the
// block's lanes in the fixed order (every lane of the block gets the same
// bits, so the branches below are uniform over the block).
//
// Modes (bytes as in include/mx.h): with s0 the OCP byte and v0 the block
// maximum over 2^(s0-127) (in [4, 8) whenever the exponent field e of amax is
// >= 2), the no-overflow byte is s0 + 1 exactly when v0 > 6, i.e. when amax's
// mantissa field exceeds 0x400000; the page's halving test ((3, 3.5] under
// the no-overflow scale) leaves s0 + 1 only when v0 > 7, i.e. mantissa field
// > 0x600000. Both are capped at 252 so every code decodes finite.
//
// Error-driven modes compare a high byte h with h - 1 by the pinned fp32
// SSE (errors in units of 2^(h-127)). h - 1 is evaluated only when it can
// win: at h - 1 the block maximum (> 3 * 2^(h-127)) saturates to
// 3 * 2^(h-127), so that element alone contributes fl(d * d) with
// d = fl(amax * 2^(127-h) - 3), the same d the sum takes for it, and the
// pinned sum only grows as non-negative terms are added (rounding is
// monotone). Hence SSE32(h - 1) >= fl(d * d); when SSE32(h) <= fl(d * d) the
// strict test SSE32(h - 1) < SSE32(h) must fail and h is kept without
// computing it. The decision is identical to evaluating both candidates.
template <int MODE, typename Codes, typename Encode, typename Sign, typename BlockSse>
__device__ __forceinline__ uint32_t choose_scale(uint32_t amax, Codes &codes, Encode encode,
                                                 Sign sign, BlockSse block_sse) {
  const uint32_t s0 = ocp_scale_byte(amax);
  if (__builtin_expect(s0 == 255u, 0)) {
    codes = sign();
    return s0;
  }
  const uint32_t mant = amax & 0x7FFFFFu;
  const bool normalized = (amax >> 23) >= 2u;  // v0 in [4, 8)
  if constexpr (MODE == MX_SCALE_OCP || MODE == MX_SCALE_OAS_BITS) {
    uint32_t s = s0;
    if (MODE == MX_SCALE_OAS_BITS && normalized && mant > 0x600000u) s = min(s0 + 1u, 252u);
    codes = encode(s);
    return s;
  } else {
    uint32_t h = s0;
    if (MODE == MX_SCALE_OAS_NF && normalized && mant > 0x400000u) h = min(s0 + 1u, 252u);
    if (h == 0u) {
      codes = encode(h);
      return h;
    }
    Codes c_hi;
    const float sse_hi = block_sse(h, h, c_hi);
    const float d_top =
        __builtin_fmaf(__uint_as_float(amax), __uint_as_float((254u - h) << 23), -3.0f);
    const float bound = d_top * d_top;
    codes = c_hi;
    if (sse_hi > bound) {  // uniform over the block: same sums, same amax
      Codes c_low;
      const float sse_low = block_sse(h - 1u, h, c_low);
      if (sse_low < sse_hi) {  // strict: a tie keeps h
        codes = c_low;
        return h - 1u;
      }
    }
    return h;
  }
}

// Block scale byte and this lane's 8 codes, four lanes per block (all quad
// lanes agree on the byte).
template <bool BF16, int MODE>
__device__ __forceinline__ uint32_t quantize_item(const Item<BF16> &x, uint32_t &codes) {
  return choose_scale<MODE>(
      quad_max_u32(item_amax_bits<BF16>(x)), codes,
      [&](uint32_t s) { return encode_item<BF16>(x, s); },
      [&]() { return sign_codes<BF16>(x); },
      [&](uint32_t c, uint32_t h, uint32_t &out) {
        return quad_sum_f32(lane_sse<BF16>(x, c, h, out));
      });
}

// ---- two lanes per block (bf16) ----------------------------------------------
//
// A lane pair owns a block: 16 bf16 elements (32 bytes, two 16-byte loads)
// per lane, 8 code bytes out. The per-block work (maximum, byte, bound,
// decision) then runs on two lanes instead of four, which pays where the two
// error evaluations of OAS_NF make quantize arithmetic-bound; its loads are
// 16 bytes at a 32-byte lane pitch per instruction, which costs more than the
// quad layout's contiguous ones on larger tensors (see launch_quantize_t).
// The pinned error keeps its order: the even lane of the pair holds groups 0
// and 1, the odd lane groups 2 and 3, each lane forms (g0 + g1) or (g2 + g3)
// from its two groups (each even + odd accumulator as in lane_sse), and one
// pair exchange adds the two (fp32 addition commutes, so both lanes hold the
// same bits).
struct PairItem {
  uint32_t w[8];  // element 2j in the low half of w[j]
};
__device__ __forceinline__ void load_pair_item(const void *base, int64_t pit, PairItem &x) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(base) + 2 * pit;
  const u32x4 a = ld<true>(q), b = ld<true>(q + 1);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    x.w[j] = a[j];
    x.w[4 + j] = b[j];
  }
}
__device__ __forceinline__ uint32_t pair_amax_bits(const PairItem &x) {
  u16x2 m = __builtin_bit_cast(u16x2, x.w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int j = 1; j < 8; j++)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x.w[j] & 0x7FFF7FFFu));
  return (uint32_t)max(m.x, m.y) << 16;
}
// the lane's two 8-element halves as quad-layout items
__device__ __forceinline__ Item<true> pair_half(const PairItem &x, int half) {
  Item<true> r;
#pragma unroll
  for (int j = 0; j < 4; j++) r.w[j] = x.w[4 * half + j];
  return r;
}
__device__ __forceinline__ float pair_lane_sse(const PairItem &x, uint32_t c, uint32_t h,
                                               u32x2 &codes) {
  uint32_t c0, c1;
  const float ga = lane_sse<true>(pair_half(x, 0), c, h, c0);  // group 2 (lane & 1)
  const float gb = lane_sse<true>(pair_half(x, 1), c, h, c1);  // group 2 (lane & 1) + 1
  codes = u32x2{c0, c1};
  return ga + gb;
}
template <int MODE>
__device__ __forceinline__ uint32_t quantize_pair(const PairItem &x, u32x2 &codes) {
  const uint32_t a = pair_amax_bits(x);
  return choose_scale<MODE>(
      max(a, dpp_x1(a)), codes,
      [&](uint32_t s) {
        return u32x2{encode_item<true>(pair_half(x, 0), s), encode_item<true>(pair_half(x, 1), s)};
      },
      [&]() { return u32x2{sign_codes<true>(pair_half(x, 0)), sign_codes<true>(pair_half(x, 1))}; },
      [&](uint32_t c, uint32_t h, u32x2 &out) {
        const float p = pair_lane_sse(x, c, h, out);
        return p + __uint_as_float(dpp_x1(__float_as_uint(p)));
      });
}

// ---- kernels -----------------------------------------------------------------

// Grid-stride over tiles of NT * U items (NT threads per workgroup); each
// thread's U items are spaced NT apart so every load instruction is
// coalesced. A tile runs
// in three phases: every item's loads, every item's arithmetic (results kept
// in registers), every item's stores. The vector memory counter that a wave
// waits on for its loads also counts its stores, so a store issued between
// the loads of a tile and the wait for a later item's data makes that wait
// cover the store as well: storing each item before the next item's
// arithmetic stalled every wave on its own stores (block MSE on the 2.8e9-
// element weight set: 1465 us with the per-item store, 1188 us without any
// store). The backend may still sink a load whose value is first used past a
// divergent branch below the first item's arithmetic (OAS quantize issues one
// load, then three, which measured faster than forcing all four ahead). Full
// tiles run without bounds checks; the one partial tile (if any) is handled
// by the workgroup whose stride lands on it, with per-item checks.
//
// XCD_CHUNKS: workgroups are dispatched round-robin over the eight XCDs
// (workgroup b on XCD b mod 8), so by default each XCD walks tiles spaced
// eight apart across the whole tensor; with XCD_CHUNKS (and a grid that is a
// multiple of 8) workgroup b takes tile (b mod 8) G/8 + b/8 instead, so each
// XCD walks one contiguous eighth of the tensor (a bijection on the tiles,
// so the results do not change). On the 2.8e9-element weight set this made
// dequantize 2.5-3.3 % faster (also on the MoE experts), left fake-quant
// unchanged and made block MSE 4 % slower; quantize went 8 % slower at one
// item per 256 threads, and at two per 128 (with non-temporal code stores)
// 1.8 % faster in OCP and OAS_BITS, 1.2 % slower in OAS; runs of four tiles
// per XCD were slower for all of them.
template <int U, bool XCD_CHUNKS = false, int NT = kThreads, typename Load, typename Compute,
          typename Store>
__device__ __forceinline__ void tile_loop(int64_t nitems, Load load, Compute compute,
                                          Store store) {
  const int64_t tile = (int64_t)NT * U;
  const int64_t nfull = nitems / tile;
  int64_t t = blockIdx.x;
  if (XCD_CHUNKS && gridDim.x % 8u == 0u)
    t = (int64_t)(blockIdx.x % 8u) * (gridDim.x / 8u) + blockIdx.x / 8u;
  for (; t < nfull; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++) load(u, base + u * NT);
    __builtin_amdgcn_sched_barrier(0);  // every load ahead of the arithmetic
#pragma unroll
    for (int u = 0; u < U; u++) compute(u, base + u * NT);
    __builtin_amdgcn_sched_barrier(0);  // every item's arithmetic ahead of the stores
#pragma unroll
    for (int u = 0; u < U; u++) store(u, base + u * NT);
  }
  if (t == nfull && nfull * tile < nitems) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * NT < nitems) load(u, base + u * NT);
#pragma unroll
    for (int u = 0; u < U; u++)  // whole quads (16-lane rows) drop out together
      if (base + u * NT < nitems) compute(u, base + u * NT);
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * NT < nitems) store(u, base + u * NT);
  }
}

// The same walk for a kernel that stores nothing per item.
template <int U, typename Load, typename Use>
__device__ __forceinline__ void tile_loop(int64_t nitems, Load load, Use use) {
  tile_loop<U>(nitems, load, use, [](int, int64_t) {});
}

// The same walk with a per-workgroup prologue (tables, reductions, a
// barrier) that runs once the workgroup's first tile's loads are issued, so
// that its latency overlaps theirs instead of delaying them; every thread
// runs it. Later tiles load at the top of their iteration as in tile_loop.
template <int U, int NT = kThreads, typename Prologue, typename Load, typename Compute,
          typename Store>
__device__ __forceinline__ void tile_loop_pro(int64_t nitems, Prologue prologue, Load load,
                                              Compute compute, Store store) {
  const int64_t tile = (int64_t)NT * U;
  const int64_t nfull = nitems / tile;
  const bool partial = nfull * tile < nitems;
  const int64_t first = blockIdx.x;
  int64_t t = first;
  if (t < nfull) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++) load(u, base + u * NT);
  } else if (t == nfull && partial) {
    const int64_t base = t * tile + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * NT < nitems) load(u, base + u * NT);
  }
  prologue();
  for (; t < nfull; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
    if (t != first) {
#pragma unroll
      for (int u = 0; u < U; u++) load(u, base + u * NT);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load ahead of the arithmetic
#pragma unroll
    for (int u = 0; u < U; u++) compute(u, base + u * NT);
    __builtin_amdgcn_sched_barrier(0);  // every item's arithmetic ahead of the stores
#pragma unroll
    for (int u = 0; u < U; u++) store(u, base + u * NT);
  }
  if (t == nfull && partial) {
    const int64_t base = t * tile + threadIdx.x;
    if (t != first) {
#pragma unroll
      for (int u = 0; u < U; u++)
        if (base + u * NT < nitems) load(u, base + u * NT);
    }
#pragma unroll
    for (int u = 0; u < U; u++)  // whole lane pairs and quads drop out together
      if (base + u * NT < nitems) compute(u, base + u * NT);
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * NT < nitems) store(u, base + u * NT);
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

// Items per thread for the MXFP4 kernels, by what the kernel does and by
// tensor size (each op measured alone, with the three-phase tile loop).
// Below kLargeItems items (tensors below ~2e8 elements, 400 MB of bf16, which
// the 256 MB Infinity Cache may partly hold): bf16 quantize keeps kU in OCP,
// OAS and OAS_BITS (OAS with two items per thread was 2 % slower on
// 8192x4096, equal on 16384x8192), while OAS_NF quantize takes two (4 % faster on
// 8192x4096, where its two error evaluations per block make it
// arithmetic-bound; equal on 16384x8192; up to kPairItems items it runs the
// two-lanes-per-block kernel instead); bf16 dequantize and fake-quant take
// two (fewer registers and more workgroups in flight for the write-heavy
// stream; one fp32 fake-quant item was 5 % slower on fp32 1024x4096). Beyond
// it (multi-GB weight sets streamed once from HBM) fewer items per thread keep
// the memory that the resident workgroups touch at one time compact: on the
// 2.8e9-element Llama-3.2-3B weight set fake-quant with one item per thread
// was 5 % faster than two and dequantize keeps two; quantize takes two items
// per 128-thread workgroup in every mode, with non-temporal code stores (see
// threads_of and nt_codes). The multi-tensor launch picks by the items of
// the whole call.
#ifndef MX_LARGE_ITEMS
#define MX_LARGE_ITEMS (int64_t(3) << 23)
#endif
constexpr int64_t kLargeItems = MX_LARGE_ITEMS;
enum { kKindQuantize = 0, kKindFakequant = 1, kKindDequantize = 2 };
constexpr int unroll_of(bool bf16, int mode, int kind, bool large = false) {
  if (bf16 && large) {
    if (kind == kKindFakequant) return 1;
    return 2;  // quantize (every mode) and dequantize
  }
  if (kind == kKindFakequant) return 2;
  if (!bf16) return kU<false>;
  if (kind == kKindQuantize) return mode == MX_SCALE_OAS_NF ? 2 : kU<true>;
  return 2;
}

// Threads per workgroup of the bf16 quantize, fake-quant and dequantize
// kernels on multi-GB tensors (one tile per workgroup, so this is also the
// tile's width); everything else keeps kThreads. Measured on the 2.8e9-
// element Llama-3.2-3B weight set against 256 threads: OAS quantize with
// 128 4-6 % faster (64: up to 3 % slower, 512: 3 % slower), dequantize with
// 64 2.4 % faster and fake-quant with 64 faster in every mode (OCP 1.6-1.8 %,
// OAS 4 %, OAS_BITS 1.7 %, OAS_NF 5 %; 128 and 512 slower or equal), OAS_NF
// quantize with 128 threads and two items 3.6-5 % faster than 256 and four.
// With default-policy code stores quantize OCP and OAS_BITS were fastest at
// 256 threads with one item (64 and 128: 2-5 % slower; two or four items per
// thread 6-13 % slower); with the non-temporal code stores of the narrow
// tilings (nt_codes) 128 x 2 beats that too: OCP 1091 against 1130 us and
// OAS_BITS 1088 against 1122 us on the weight set, and the multi-tensor call
// over its 196 matrices 1110 against 1196 us (OCP) and 1107 against 1208 us
// (OAS_BITS); 128 x 1 was 5-6 % slower. A plain copy of the same buffer ran
// 3.4 % faster with 64 than with 256.
constexpr int threads_of(bool bf16, int mode, int kind, bool large = false) {
  (void)mode;
  if (!bf16 || !large) return kThreads;
  if (kind == kKindFakequant || kind == kKindDequantize) return 64;
  return 128;  // quantize, every mode
}

// Cache policy of the code-word stores of a quantize launch: non-temporal
// for the narrow multi-GB tilings (fewer than kThreads threads per
// workgroup: MXFP4 quantize's 128 x 2 in every mode, single-tensor and
// multi-tensor, and MXFP8's 64 x 1), default elsewhere. On the 2.8e9-element
// weight set OAS quantize took 1087 against 1122 us with the hint (OAS_NF
// unchanged), the multi-tensor OAS call 1086 against 1227 us, and MXFP8
// quantize of the MoE w13 experts 733 against 765 us; OCP quantize at 256 x 1
// was 2 % slower with it (at 128 x 2 it is faster than 256 x 1 without it:
// see threads_of) and MBS-Static quantize unchanged, so MBS keeps the
// default, as do the small-tensor tilings (on bf16 8192x4096 and 16384x8192
// the hint made OCP and OAS_BITS quantize 5-7 % and MXFP8 quantize 1-3 %
// slower, and the multi-GB 128 x 2 tiling with it was 3-4 % slower there
// than 256 x 4). The
// two-lanes-per-block OAS_NF kernel (k_quantize_pair, 8-byte code stores)
// takes the hint: on bf16 8192x4096 activations its median launch went from
// 17.1-18.4 to 16.3-16.9 us (same p10, a tighter spread).
constexpr bool nt_codes(int nt) { return nt < kThreads; }

template <bool BF16, int MODE, int U, int NT>
__global__ __launch_bounds__(NT) void k_quantize(const void *__restrict__ x,
                                                 uint32_t *__restrict__ codes,
                                                 uint8_t *__restrict__ scales, int64_t nitems) {
  Item<BF16> xv[U];
  uint32_t cw[U], sv[U];
  // per-XCD eighths for OCP and OAS_BITS on the multi-GB tiling: on the
  // 2.8e9-element weight set 1076 against 1096 us (OCP) and 1074 against
  // 1094 us (OAS_BITS); OAS was 1.2 % slower with the map, so the
  // error-driven modes keep launch order
  constexpr bool kXcd = NT == 128 && (MODE == MX_SCALE_OCP || MODE == MX_SCALE_OAS_BITS);
  tile_loop<U, kXcd, NT>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) { sv[u] = quantize_item<BF16, MODE>(xv[u], cw[u]); },
      [&](int u, int64_t it) {
        st<nt_codes(NT)>(codes + it, cw[u]);
        if ((threadIdx.x & 3) == 0) st<false>(scales + (it >> 2), (uint8_t)sv[u]);
      });
}

// bf16 quantize with two lanes per block (npitems = elements / 16).
template <int MODE, int U>
__global__ __launch_bounds__(kThreads) void k_quantize_pair(const void *__restrict__ x,
                                                            uint32_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales,
                                                            int64_t npitems) {
  PairItem xv[U];
  u32x2 cw[U];
  uint32_t sv[U];
  tile_loop<U>(
      npitems, [&](int u, int64_t pit) { load_pair_item(x, pit, xv[u]); },
      [&](int u, int64_t) { sv[u] = quantize_pair<MODE>(xv[u], cw[u]); },
      [&](int u, int64_t pit) {
        st<true>(reinterpret_cast<u32x2 *>(codes) + pit, cw[u]);  // see nt_codes
        if ((threadIdx.x & 1) == 0) st<false>(scales + (pit >> 1), (uint8_t)sv[u]);
      });
}
template <bool BF16, int MODE, int U, int NT>
__global__ __launch_bounds__(NT) void k_fakequant(const void *x, void *y, int64_t nitems) {
  Item<BF16> xv[U];
  uint32_t out[U][BF16 ? 4 : 8];
  tile_loop<U, false, NT>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) {
        uint32_t c;
        const uint32_t s = quantize_item<BF16, MODE>(xv[u], c);
        decode_item<BF16>(c, s, out[u]);
      },
      [&](int u, int64_t it) { store_item<BF16>(y, it, out[u]); });
}

// ---- many tensors in one launch ------------------------------------------------
//
// A list of separate tensors (say every Linear weight of a model) quantized
// or fake-quantized by one launch: a launch per tensor pays the per-kernel
// ramp-up and drain each time (a 3 Mi-element weight runs at a quarter of the
// streaming rate on its own). The descriptors travel by value in the kernel
// arguments (no device table, nothing to copy or allocate; capturable). A
// tensor's last tile may be partial and takes the per-item checks.

template <int U, int NT, typename Load, typename Compute, typename Store>
__device__ __forceinline__ void tile_at(int64_t t, int64_t nitems, Load load, Compute compute,
                                        Store store) {
  const int64_t tile = (int64_t)NT * U;
  const int64_t base = t * tile + threadIdx.x;
  if ((t + 1) * tile <= nitems) {
#pragma unroll
    for (int u = 0; u < U; u++) load(u, base + u * NT);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; u++) compute(u, base + u * NT);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; u++) store(u, base + u * NT);
  } else {
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * NT < nitems) load(u, base + u * NT);
#pragma unroll
    for (int u = 0; u < U; u++)  // whole quads drop out together
      if (base + u * NT < nitems) compute(u, base + u * NT);
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * NT < nitems) store(u, base + u * NT);
  }
}

struct MultiDesc {
  const void *x;    // input [rows, k]
  void *out;        // quantize: codes; fake-quant: y
  uint8_t *scales;  // quantize: scales; fake-quant: unused
  int64_t nitems;   // rows * k / 8
};
struct MultiArgs {
  MultiDesc d[MX_MULTI_MAX];
};

// Many tensors in one launch: workgroup (x, y) takes tile x of tensor y, so
// no workgroup searches for its tensor; tiles past a tensor's end do nothing
// (the host groups tensors of similar size into one launch). Items per
// thread and threads per workgroup follow the single-tensor kernels for the
// size of the whole call. On the 196
// Llama-3.2-3B matrices this ran 3 % (quantize OCP) and 5 % (fake-quant)
// faster than one 1-D grid whose workgroups found their tensor by a binary
// search over the tensors' first tiles, with four items per thread: with
// one item per thread that search cost 10 % more, since every tile waits
// on it before its loads issue; a 64-lane compare of the first tiles
// (one vector load) cost 25 %, a scalar compare of all of them 70 %.
template <bool BF16, int MODE, bool FQ, bool LARGE,
          int NT = threads_of(BF16, MODE, FQ ? kKindFakequant : kKindQuantize, LARGE)>
__global__ __launch_bounds__(NT) void k_multi(const MultiArgs a) {
  constexpr int U = unroll_of(BF16, MODE, FQ ? kKindFakequant : kKindQuantize, LARGE);
  Item<BF16> xv[U];
  uint32_t cw[U], sv[U], out[U][FQ ? (BF16 ? 4 : 8) : 1];
  const MultiDesc &d = a.d[blockIdx.y];
  const void *x = d.x;
  tile_at<U, NT>(
      blockIdx.x, d.nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) {
        sv[u] = quantize_item<BF16, MODE>(xv[u], cw[u]);
        if constexpr (FQ) decode_item<BF16>(cw[u], sv[u], out[u]);
      },
      [&](int u, int64_t it) {
        if constexpr (FQ) {
          store_item<BF16>(d.out, it, out[u]);
        } else {
          st<nt_codes(NT)>(static_cast<uint32_t *>(d.out) + it, cw[u]);
          if ((threadIdx.x & 3) == 0) st<false>(d.scales + (it >> 2), (uint8_t)sv[u]);
        }
      });
}

template <bool BF16, int U, int NT>
__global__ __launch_bounds__(NT) void k_dequantize(const uint32_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales,
                                                   void *__restrict__ y, int64_t nitems) {
  uint32_t cw[U], sb[U];
  uint32_t out[U][BF16 ? 4 : 8];
  tile_loop<U, true, NT>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(scales + (it >> 2));
      },
      [&](int u, int64_t) { decode_item<BF16>(cw[u], sb[u], out[u]); },
      [&](int u, int64_t it) { store_item<BF16>(y, it, out[u]); });
}

// Block error. Per block: SSE = sum (x - x_hat)^2 in fp64 (quad sum in a
// fixed order), block_mse = (float)(SSE / 32). The tensor sums (SSE and
// sum x^2) are taken in two stages with fixed order and no atomics: each
// workgroup writes its two sums to partial[2 * blockIdx.x + {0, 1}] (lane
// sums, then DPP sums within each 16-lane row, then the rows in order), and
// k_sum_partials adds the partials.
// Block error of one item against (c, s): the fp64 SSE of the quad's block,
// summed in a fixed order (per lane, then quad_sum_f64); returns the block's
// MSE, SSE / 32 as fp32, on every lane of the quad (the caller stores it
// from lane 0). Lane 0 of the quad also adds the SSE to `mine`, and every
// lane adds its sum of x^2 to `mine_sq` (tensor sums).
template <bool BF16, bool SUMS>
__device__ __forceinline__ float mse_item(const Item<BF16> &x, uint32_t c, uint32_t s,
                                          double &mine, double &mine_sq) {
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
  if constexpr (SUMS) mine += (threadIdx.x & 3) == 0 ? sse : 0.0;
  return (float)(sse * (1.0 / 32.0));
}

// The workgroup's two tensor sums, in a fixed order (DPP sums over each row
// of 16 lanes, then the rows in turn), to partial[2 * blockIdx.x + {0, 1}].
// Row sums through LDS cost fewer instructions than a 64-lane butterfly of
// cross-lane shuffles; every lane is active here.
__device__ __forceinline__ void write_partials(double mine, double mine_sq,
                                               double *__restrict__ partial) {
  __shared__ double row_part[2][kThreads / 16];
  mine = row_sum_f64(mine);
  mine_sq = row_sum_f64(mine_sq);
  if ((threadIdx.x & 15) == 0) {
    row_part[0][threadIdx.x >> 4] = mine;
    row_part[1][threadIdx.x >> 4] = mine_sq;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    double t = 0.0;
    for (int r = 0; r < kThreads / 16; r++) t += row_part[threadIdx.x][r];
    partial[2 * blockIdx.x + threadIdx.x] = t;
  }
}

// Items per thread of the block-MSE kernel, by tensor size only (the grid
// sizes the partial-sum workspace, which the caller sizes without a dtype):
// four up to kLargeItems items, two beyond. With one tile per workgroup
// (see mxi_launch_block_mse) four measured fastest on bf16 8192x4096 and
// 16384x8192 (74.6 % and 79.4 % of 8 TB/s without the tensor sums, against
// 71.1 % and 76.7 % with two), two on the 2.8e9-element weight set (77.5 %,
// against 73.8 % with four and 72.5 % with one).
constexpr int mse_unroll(bool large) { return large ? 2 : 4; }
// Items per thread of the one-pass kernel, both dtypes (it sizes the same
// workspace).
constexpr int kFusedU = 2;

template <bool BF16, bool SUMS, int U>
__global__ __launch_bounds__(kThreads) void k_block_mse(const void *__restrict__ x,
                                                        const uint32_t *__restrict__ codes,
                                                        const uint8_t *__restrict__ scales,
                                                        float *__restrict__ block_mse,
                                                        double *__restrict__ partial,
                                                        int64_t nitems) {
  double mine = 0.0;     // sum of the block SSEs this lane reports (q == 0 lanes)
  double mine_sq = 0.0;  // sum of x^2 over this lane's elements
  Item<BF16> xv[U];
  uint32_t cw[U], sb[U];
  float bm[U];
  tile_loop<U>(
      nitems,
      [&](int u, int64_t it) {
        load_item<BF16>(x, it, xv[u]);
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(scales + (it >> 2));
      },
      [&](int u, int64_t) { bm[u] = mse_item<BF16, SUMS>(xv[u], cw[u], sb[u], mine, mine_sq); },
      [&](int u, int64_t it) {
        if (block_mse && (threadIdx.x & 3) == 0) st<true>(block_mse + (it >> 2), bm[u]);
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
  // two items per thread in both dtypes (as for fake-quant: 2.4 % faster
  // than four on bf16 8192x4096); its grid is the largest an error launch
  // uses, which sizes the partial-sum workspace
  constexpr int U = kFusedU;
  Item<BF16> xv[U];
  uint32_t cw[U], sv[U], out[U][BF16 ? 4 : 8];
  float bm[U];
  tile_loop<U>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) {
        sv[u] = quantize_item<BF16, MODE>(xv[u], cw[u]);
        if (y) decode_item<BF16>(cw[u], sv[u], out[u]);  // uniform
        if (err) bm[u] = mse_item<BF16, SUMS>(xv[u], cw[u], sv[u], mine, mine_sq);
      },
      [&](int u, int64_t it) {
        st<false>(codes + it, cw[u]);
        if ((threadIdx.x & 3) == 0) st<false>(scales + (it >> 2), (uint8_t)sv[u]);
        if (y) store_item<BF16>(y, it, out[u]);
        if (block_mse && (threadIdx.x & 3) == 0) st<true>(block_mse + (it >> 2), bm[u]);
      });
  if constexpr (SUMS) write_partials(mine, mine_sq, partial);
}

// Partial sums of the tensor error: each workgroup of an error launch writes
// two (SSE, sum of x^2); one workgroup of k_sum_partials (1024 threads) adds
// up to kSumGroup pairs in a fixed order. An error launch uses at most
// kSumGroup^2 workgroups (beyond, workgroups loop over tiles), so at most two
// sum levels run: up to kSumGroup partial pairs (tensors up to ~3.4e7
// elements) go straight to the result, more go through one pair per
// kSumGroup first. (Groups of 2048 pairs put a second, dependent launch on
// the 8192x4096 one-pass call: 3.5 us more than its earlier 2048-workgroup
// grid.)
#ifndef MX_SUM_GROUP
#define MX_SUM_GROUP 8192
#endif
constexpr int64_t kSumGroup = MX_SUM_GROUP;
constexpr int kSumThreads = 1024;
constexpr int kSumPer = (int)(kSumGroup / kSumThreads);  // partial pairs per thread
static_assert(kSumPer * kSumThreads == kSumGroup, "sum group must be a multiple of 1024");
constexpr int64_t kPartialCap = kSumGroup * kSumGroup;

// Workgroup b: out[2b + j] = sum over i of partial[2(b kSumGroup + i) + j]
// for j = 0, 1 and the (up to kSumGroup) pairs i of its group; n pairs in
// all. The kernel is latency-bound, so every thread issues all of its loads
// (pairs t, t + 1024, ...) before the first add; the sums then run in a
// fixed order (per thread in pair order, a butterfly over the wave, the
// sixteen waves in order), so the result is deterministic. n == 0 writes 0.
__global__ __launch_bounds__(kSumThreads) void k_sum_partials(const double *__restrict__ partial,
                                                              int64_t n,
                                                              double *__restrict__ out) {
  __shared__ double wave_part[2][kSumThreads / 64];
  const int64_t first = (int64_t)blockIdx.x * kSumGroup;
  const int m = (int)(n - first < kSumGroup ? n - first : kSumGroup);  // pairs of this group
  double *o = out + 2 * blockIdx.x;
  if (m <= 0) {
    if (threadIdx.x < 2) o[threadIdx.x] = 0.0;
    return;
  }
  const double *p = partial + 2 * first;
  // unconditional loads of a clamped (in-bounds) index, so none waits on a
  // branch; pairs past m are then replaced by zero
  double v0[kSumPer], v1[kSumPer];
#pragma unroll
  for (int j = 0; j < kSumPer; j++) {
    const int i = (int)threadIdx.x + j * kSumThreads;
    const int ic = min(i, m - 1);
    const double a = p[2 * ic], b = p[2 * ic + 1];
    v0[j] = i < m ? a : 0.0;
    v1[j] = i < m ? b : 0.0;
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
    for (int w = 0; w < kSumThreads / 64; w++) t += wave_part[threadIdx.x][w];
    o[threadIdx.x] = t;
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

// Items per thread of MXFP8 quantize: two for bf16 (with the three-phase
// tile loop, 2.8 % faster than four on 8192x4096 activations; one was 6 %
// slower), kU for fp32.
template <bool BF16>
constexpr int kU8 = BF16 ? 2 : kU<false>;

template <bool BF16, int U, int NT>
__global__ __launch_bounds__(NT) void k_quantize8(const void *__restrict__ x,
                                                  u32x2 *__restrict__ codes,
                                                  uint8_t *__restrict__ scales, int64_t nitems) {
  Item<BF16> xv[U];
  u32x2 cw[U];
  uint32_t sv[U];
  tile_loop<U, false, NT>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) { sv[u] = quantize8_item<BF16>(xv[u], cw[u]); },
      [&](int u, int64_t it) {
        st<nt_codes(NT)>(codes + it, cw[u]);
        if ((threadIdx.x & 3) == 0) st<false>(scales + (it >> 2), (uint8_t)sv[u]);
      });
}

template <bool BF16, int U, int NT>
__global__ __launch_bounds__(NT) void k_dequantize8(const u32x2 *__restrict__ codes,
                                                    const uint8_t *__restrict__ scales,
                                                    void *__restrict__ y, int64_t nitems) {
  u32x2 cw[U];
  uint32_t sb[U];
  uint32_t out[U][BF16 ? 4 : 8];
  tile_loop<U, false, NT>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(scales + (it >> 2));
      },
      [&](int u, int64_t) { decode8_item<BF16>(cw[u], sb[u], out[u]); },
      [&](int u, int64_t it) { store_item<BF16>(y, it, out[u]); });
}

template <bool BF16, int U, int NT>
__global__ __launch_bounds__(NT) void k_fakequant8(const void *x, void *y, int64_t nitems) {
  Item<BF16> xv[U];
  uint32_t out[U][BF16 ? 4 : 8];
  tile_loop<U, false, NT>(
      nitems, [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) {
        u32x2 c;
        const uint32_t s = quantize8_item<BF16>(xv[u], c);
        decode8_item<BF16>(c, s, out[u]);
      },
      [&](int u, int64_t it) { store_item<BF16>(y, it, out[u]); });
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

// Forward declaration (defined below with the tensor factor's rule).
__device__ __forceinline__ int nv_tensor_exp(uint32_t amax_bits);

// One workgroup: the tensor exponent t from the npartial first-pass maxima,
// to partial[npartial] for the block pass of a multi-GB tensor (and t + 127
// to *tensor_scale when it is not null), so that pass's workgroups, one per
// tile, read one word instead of reducing the maxima each.
__global__ __launch_bounds__(kThreads) void k_nv_prepare(uint32_t *__restrict__ partial,
                                                         int npartial,
                                                         uint8_t *__restrict__ tensor_scale) {
  __shared__ uint32_t wave_max[kThreads / 64];
  uint32_t pv[kNvPer];
#pragma unroll
  for (int j = 0; j < kNvPer; j++) pv[j] = partial[min((int)threadIdx.x + j * kThreads, npartial - 1)];
  uint32_t a = 0;
#pragma unroll
  for (int j = 0; j < kNvPer; j++) a = max(a, pv[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) a = max(a, wave_max[w]);
    const int t = nv_tensor_exp(a);
    partial[npartial] = (uint32_t)t;
    if (tensor_scale) *tensor_scale = (uint8_t)(t + 127);
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
// The NVFP4 block pass. PRE: the tensor exponent t was reduced once by
// k_nv_prepare and sits at partial[npartial] (the multi-GB launch: one tile
// per workgroup, NT threads, U items); otherwise every workgroup reduces the
// npartial maxima itself.
template <bool BF16, bool FQ, bool PRE, int U, int NT>
__device__ __forceinline__ void nv_block_pass(const void *x, const uint32_t *__restrict__ partial,
                                              int npartial, uint32_t *__restrict__ codes,
                                              uint8_t *__restrict__ block_scales,
                                              uint8_t *__restrict__ tensor_scale, void *y,
                                              int64_t nitems) {
  static_assert(PRE || NT == kThreads, "the in-kernel reduction assumes kThreads");
  static_assert(NT >= 128 && NT % 64 == 0, "the table takes 128 threads");
  // every workgroup reduces the first pass's maxima (max is order-free and
  // idempotent, so clamped duplicate loads are harmless; all loads are issued
  // before the first use), or reads their reduction (PRE), and fills a table
  // of fl32(1 / v) for the E4M3 values v (code 0 -> 0; code 0x7F is NaN and
  // never looked up), once its first tile's loads are in flight
  __shared__ uint32_t wave_max[NT / 64];
  __shared__ float rcp_e4m3[128];
  const float one = 1.0f;  // scale operand of the converts: 2^0
  float S = 0.0f, inv_s = 0.0f;
  Item<BF16> xv[U];
  uint32_t cw[U], sv[U], out[U][FQ ? (BF16 ? 4 : 8) : 1];
  tile_loop_pro<U, NT>(
      nitems,
      [&]() {
        if constexpr (PRE) {
          const int t = (int)partial[npartial];
          if (threadIdx.x < 128) {
            const float v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(threadIdx.x, one, false)[0];
            rcp_e4m3[threadIdx.x] = threadIdx.x == 0 ? 0.0f : 1.0f / v;
          }
          __syncthreads();
          S = __uint_as_float((uint32_t)(t + 127) << 23);
          inv_s = __uint_as_float((uint32_t)(127 - t) << 23);  // 2^-t
        } else {
        uint32_t pv[kNvPer];
#pragma unroll
        for (int j = 0; j < kNvPer; j++)
          pv[j] = partial[min((int)threadIdx.x + j * kThreads, npartial - 1)];
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
        S = __uint_as_float((uint32_t)(t + 127) << 23);
        inv_s = __uint_as_float((uint32_t)(127 - t) << 23);  // 2^-t
        }
      },
      [&](int u, int64_t it) { load_item<BF16>(x, it, xv[u]); },
      [&](int u, int64_t) {
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
        if constexpr (FQ) nv_decode_item<BF16>(c, sbyte, inv_s, out[u]);
        cw[u] = c;
        sv[u] = sbyte;
      },
      [&](int u, int64_t it) {
        if constexpr (FQ) {
          store_item<BF16>(y, it, out[u]);
        } else {
          st<nt_codes(NT)>(codes + it, cw[u]);
          if ((threadIdx.x & 1) == 0) st<false>(block_scales + (it >> 1), (uint8_t)sv[u]);
        }
      });
}

// The block pass: 2048 workgroups looping over tiles, each reducing the
// first pass's maxima itself.
template <bool BF16, bool FQ>
__global__ __launch_bounds__(kThreads) void k_quantize_nv(const void *x,
                                                          const uint32_t *__restrict__ partial,
                                                          int npartial,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ block_scales,
                                                          uint8_t *__restrict__ tensor_scale,
                                                          void *y, int64_t nitems) {
  nv_block_pass<BF16, FQ, false, kUnroll, kThreads>(x, partial, npartial, codes, block_scales,
                                                    tensor_scale, y, nitems);
}

// The block pass on multi-GB tensors: one tile of NT threads x U items per
// workgroup, the tensor exponent read from partial[npartial] (k_nv_prepare).
template <bool BF16, bool FQ, int U, int NT>
__global__ __launch_bounds__(NT) void k_quantize_nv_big(const void *x,
                                                        const uint32_t *__restrict__ partial,
                                                        int npartial,
                                                        uint32_t *__restrict__ codes,
                                                        uint8_t *__restrict__ block_scales,
                                                        uint8_t *__restrict__ tensor_scale,
                                                        void *y, int64_t nitems) {
  nv_block_pass<BF16, FQ, true, U, NT>(x, partial, npartial, codes, block_scales, tensor_scale,
                                       y, nitems);
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
  uint32_t out[kU<BF16>][BF16 ? 4 : 8];
  tile_loop<kU<BF16>>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(block_scales + (it >> 1));
      },
      [&](int u, int64_t) { nv_decode_item<BF16>(cw[u], sb[u], inv_s, out[u]); },
      [&](int u, int64_t it) { store_item<BF16>(y, it, out[u]); });
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
template <bool BF16, int U, bool FQ, int NT>
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
    const int64_t it = base + u * NT;
    if (full || it < nitems) {  // whole rows of 16 lanes drop out together
      if constexpr (FQ) {
        uint32_t out[BF16 ? 4 : 8];
        mbs_decode_item<BF16>(c[u], s[u], m[u], out);
        store_item<BF16>(y, it, out);
      } else {
        st<true>(codes + it, c[u]);  // non-temporal: see tiling_mbs
        if ((threadIdx.x & 1) == 0) st<false>(sub_scales + (it >> 1), (uint8_t)s[u]);
        if ((threadIdx.x & 15) == 0) st<false>(macro_mant + (it >> 4), (uint8_t)m[u]);
      }
    }
  }
}

// FQ: fake-quant (y = dequantize(quantize(x)) in x's dtype; y may be x)
// instead of writing codes and bytes.
template <bool BF16, bool FQ, int U, int NT>
__global__ __launch_bounds__(NT) void k_quantize_mbs(const void *x, uint32_t *__restrict__ codes,
                                                     uint8_t *__restrict__ sub_scales,
                                                     uint8_t *__restrict__ macro_mant, void *y,
                                                     int64_t nitems) {
  static_assert(256 % NT == 0, "whole table entries per thread");
  __shared__ float inv_tab[256];
  const int64_t tile = (int64_t)NT * U;
  const int64_t nfull = nitems / tile;
  Item<BF16> xv[U];
  const auto load_tile = [&](int64_t t) {
    const int64_t base = t * tile + threadIdx.x;
    if (t < nfull) {
#pragma unroll
      for (int u = 0; u < U; u++) load_item<BF16>(x, base + u * NT, xv[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (base + u * NT < nitems) load_item<BF16>(x, base + u * NT, xv[u]);
        else xv[u] = Item<BF16>{};  // zeros: finite, so lanes past the end stay quiet
      }
    }
  };
  // The first tile's loads go out before the table is built, so they are in
  // flight while it is (with one tile per workgroup on multi-GB tensors the
  // table would otherwise delay every load).
  int64_t t = blockIdx.x;
  const bool has_tile = t < nfull || (t == nfull && nfull * tile < nitems);
  if (has_tile) load_tile(t);
  // fl32(1 / f) for every macro mantissa m (f = 1 + m/256): IEEE division,
  // once per workgroup, so the per-item cost is one LDS read
  for (int e = threadIdx.x; e < 256; e += NT) inv_tab[e] = 1.0f / (1.0f + (float)e * (1.0f / 256.0f));
  __syncthreads();
  for (; t < nfull; t += gridDim.x) {
    if (t != (int64_t)blockIdx.x) load_tile(t);
    __builtin_amdgcn_sched_barrier(0);
    mbs_tile<BF16, U, FQ, NT>(xv, inv_tab, codes, sub_scales, macro_mant, y, t * tile + threadIdx.x,
                              nitems, true);
  }
  if (t == nfull && nfull * tile < nitems) {
    if (t != (int64_t)blockIdx.x) load_tile(t);
    mbs_tile<BF16, U, FQ, NT>(xv, inv_tab, codes, sub_scales, macro_mant, y, t * tile + threadIdx.x,
                              nitems, false);
  }
}

template <bool BF16, int U, int NT>
__global__ __launch_bounds__(NT) void k_dequantize_mbs(const uint32_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ sub_scales,
                                                       const uint8_t *__restrict__ macro_mant,
                                                       void *__restrict__ y, int64_t nitems) {
  uint32_t cw[U], sb[U], mb[U];
  uint32_t out[U][BF16 ? 4 : 8];
  tile_loop<U, false, NT>(
      nitems,
      [&](int u, int64_t it) {
        cw[u] = ld<false>(codes + it);
        sb[u] = ld<false>(sub_scales + (it >> 1));
        mb[u] = ld<false>(macro_mant + (it >> 4));
      },
      [&](int u, int64_t) { mbs_decode_item<BF16>(cw[u], sb[u], mb[u], out[u]); },
      [&](int u, int64_t it) { store_item<BF16>(y, it, out[u]); });
}

// ---- launchers -----------------------------------------------------------------

static unsigned grid_for(int64_t nitems, int64_t cap, int unroll = kUnroll, int nt = kThreads) {
  const int64_t tile = (int64_t)nt * unroll;
  int64_t g = (nitems + tile - 1) / tile;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace mxk

using namespace mxk;

#define MX_DISPATCH_MULTI(BF16, FQ, L, MODE, G, B, ST, ARGS)                              \
  switch (MODE) {                                                                          \
    case MX_SCALE_OAS:                                                                     \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OAS, FQ, L>), G, B, 0, ST, ARGS);         \
      break;                                                                               \
    case MX_SCALE_OAS_BITS:                                                                \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OAS_BITS, FQ, L>), G, B, 0, ST, ARGS);    \
      break;                                                                               \
    case MX_SCALE_OAS_NF:                                                                  \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OAS_NF, FQ, L>), G, B, 0, ST, ARGS);      \
      break;                                                                               \
    default:                                                                               \
      hipLaunchKernelGGL((k_multi<BF16, MX_SCALE_OCP, FQ, L>), G, B, 0, ST, ARGS);         \
      break;                                                                               \
  }

// The MXFP4 streaming kernels launch one tile per workgroup (a grid stride
// only past the launch limit): on the 2.8e9-element weight set a cap of
// 196,608 workgroups, whose second round of tiles streams a second region of
// memory at the same time, was 1-5 % slower than no cap.
constexpr int64_t kGridLimit = 0x7FFFFFFF;
// bf16 OAS_NF quantize takes the two-lanes-per-block layout up to this many
// items (67,108,864 elements). On Student-t activations (8.4e6 to 2.0e8
// elements, rotated buffers) it was 6-9 % faster up to 3.4e7 elements, 2 %
// at 6.7e7, and 1-5 % slower from 1.0e8 up; for OAS quantize it was slower at
// every size measured.
constexpr int64_t kPairItems = int64_t(1) << 23;

template <bool BF16, int MODE>
static void launch_quantize_t(const void *x, uint32_t *c, uint8_t *s, int64_t nitems,
                              hipStream_t st) {
  if constexpr (BF16 && MODE == MX_SCALE_OAS_NF) {
    if (nitems <= kPairItems) {  // nitems is a multiple of 4 (k % 32 == 0)
      const int64_t np = nitems / 2;
      hipLaunchKernelGGL((k_quantize_pair<MODE, 1>), dim3(grid_for(np, kGridLimit, 1)),
                         dim3(kThreads), 0, st, x, c, s, np);
      return;
    }
  }
  if (nitems >= kLargeItems) {
    constexpr int U = unroll_of(BF16, MODE, kKindQuantize, true);
    constexpr int NT = threads_of(BF16, MODE, kKindQuantize, true);
    hipLaunchKernelGGL((k_quantize<BF16, MODE, U, NT>), dim3(grid_for(nitems, kGridLimit, U, NT)),
                       dim3(NT), 0, st, x, c, s, nitems);
  } else {
    constexpr int U = unroll_of(BF16, MODE, kKindQuantize, false);
    constexpr int NT = threads_of(BF16, MODE, kKindQuantize, false);
    hipLaunchKernelGGL((k_quantize<BF16, MODE, U, NT>), dim3(grid_for(nitems, kGridLimit, U, NT)),
                       dim3(NT), 0, st, x, c, s, nitems);
  }
}

template <bool BF16, int MODE>
static void launch_fakequant_t(const void *x, void *y, int64_t nitems, hipStream_t st) {
  if (nitems >= kLargeItems) {
    constexpr int U = unroll_of(BF16, MODE, kKindFakequant, true);
    constexpr int NT = threads_of(BF16, MODE, kKindFakequant, true);
    hipLaunchKernelGGL((k_fakequant<BF16, MODE, U, NT>), dim3(grid_for(nitems, kGridLimit, U, NT)),
                       dim3(NT), 0, st, x, y, nitems);
  } else {
    constexpr int U = unroll_of(BF16, MODE, kKindFakequant, false);
    constexpr int NT = threads_of(BF16, MODE, kKindFakequant, false);
    hipLaunchKernelGGL((k_fakequant<BF16, MODE, U, NT>), dim3(grid_for(nitems, kGridLimit, U, NT)),
                       dim3(NT), 0, st, x, y, nitems);
  }
}

template <bool BF16>
static void launch_dequantize_t(const uint32_t *c, const uint8_t *s, void *y, int64_t nitems,
                                hipStream_t st) {
  if (nitems >= kLargeItems) {
    constexpr int U = unroll_of(BF16, 0, kKindDequantize, true);
    constexpr int NT = threads_of(BF16, 0, kKindDequantize, true);
    hipLaunchKernelGGL((k_dequantize<BF16, U, NT>), dim3(grid_for(nitems, kGridLimit, U, NT)),
                       dim3(NT), 0, st, c, s, y, nitems);
  } else {
    constexpr int U = unroll_of(BF16, 0, kKindDequantize, false);
    constexpr int NT = threads_of(BF16, 0, kKindDequantize, false);
    hipLaunchKernelGGL((k_dequantize<BF16, U, NT>), dim3(grid_for(nitems, kGridLimit, U, NT)),
                       dim3(NT), 0, st, c, s, y, nitems);
  }
}

#define MX_MODE_SWITCH(FN, BF16, MODE, ...)                                                 \
  switch (MODE) {                                                                          \
    case MX_SCALE_OAS: FN<BF16, MX_SCALE_OAS>(__VA_ARGS__); break;                         \
    case MX_SCALE_OAS_BITS: FN<BF16, MX_SCALE_OAS_BITS>(__VA_ARGS__); break;               \
    case MX_SCALE_OAS_NF: FN<BF16, MX_SCALE_OAS_NF>(__VA_ARGS__); break;                   \
    default: FN<BF16, MX_SCALE_OCP>(__VA_ARGS__); break;                                   \
  }

hipError_t mxi_launch_quantize(const void *x, int bf16, int mode, int64_t nitems,
                               uint8_t *codes, uint8_t *scales, hipStream_t st) {
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  if (bf16) {
    MX_MODE_SWITCH(launch_quantize_t, true, mode, x, c, scales, nitems, st)
  } else {
    MX_MODE_SWITCH(launch_quantize_t, false, mode, x, c, scales, nitems, st)
  }
  return hipGetLastError();
}

hipError_t mxi_launch_fakequant(const void *x, int bf16, int mode, int64_t nitems, void *y,
                                hipStream_t st) {
  if (bf16) {
    MX_MODE_SWITCH(launch_fakequant_t, true, mode, x, y, nitems, st)
  } else {
    MX_MODE_SWITCH(launch_fakequant_t, false, mode, x, y, nitems, st)
  }
  return hipGetLastError();
}

hipError_t mxi_launch_dequantize(const uint8_t *codes, const uint8_t *scales, int bf16,
                                 int64_t nitems, void *y, hipStream_t st) {
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  if (bf16)
    launch_dequantize_t<true>(c, scales, y, nitems, st);
  else
    launch_dequantize_t<false>(c, scales, y, nitems, st);
  return hipGetLastError();
}

// Doubles of partial-sum space an error launch with `grid` workgroups
// writes: its pairs, and the second-level pairs when there are more than
// one group of them.
static int64_t partial_doubles(int64_t grid) {
  return 2 * (grid + (grid > kSumGroup ? (grid + kSumGroup - 1) / kSumGroup : 0));
}

// The workspace an error launch over nitems items needs for one tile per
// workgroup: the one-pass grid (two items per thread) is the largest.
size_t mxi_block_mse_partials(int64_t nitems) {
  return (size_t)partial_doubles(grid_for(nitems, kPartialCap, kFusedU));
}

// Grid of an error launch: one tile per workgroup (a wave never waits for a
// store of its own: the stores of each workgroup's one tile come last) when
// the partial space holds that grid's sums, else one sum group of
// workgroups looping over the tiles (the fixed scratch of the call without
// a workspace). Without tensor sums there are no partials.
static unsigned error_grid(int64_t nitems, int u, bool sums, int64_t partial_space) {
  const unsigned g = grid_for(nitems, kPartialCap, u);
  if (!sums || partial_doubles(g) <= partial_space) return g;
  return grid_for(nitems, partial_space / 2 < kSumGroup ? partial_space / 2 : kSumGroup, u);
}

// Adds the `grid` partial pairs at `partial` into out[0..1]: one sum launch,
// or two when there are more than kSumGroup pairs (the second-level pairs go
// right after the first-level ones).
static hipError_t sum_partials(double *partial, int64_t grid, double *out, hipStream_t st) {
  if (grid <= kSumGroup) {
    hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(kSumThreads), 0, st, partial, grid, out);
    return hipGetLastError();
  }
  const int64_t groups = (grid + kSumGroup - 1) / kSumGroup;
  double *second = partial + 2 * grid;
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)groups), dim3(kSumThreads), 0, st, partial,
                     grid, second);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(kSumThreads), 0, st, second, groups, out);
  return hipGetLastError();
}

template <bool BF16, bool SUMS, int U>
static void launch_block_mse_t(const void *x, const uint32_t *c, const uint8_t *scales,
                               float *block_mse, double *part, unsigned grid, int64_t nitems,
                               hipStream_t st) {
  hipLaunchKernelGGL((k_block_mse<BF16, SUMS, U>), dim3(grid), dim3(kThreads), 0, st, x, c,
                     scales, block_mse, part, nitems);
}

template <bool BF16, bool SUMS>
static void launch_block_mse_u(bool large, const void *x, const uint32_t *c,
                               const uint8_t *scales, float *block_mse, double *part,
                               unsigned grid, int64_t nitems, hipStream_t st) {
  if (large)
    launch_block_mse_t<BF16, SUMS, mse_unroll(true)>(x, c, scales, block_mse, part, grid, nitems,
                                                     st);
  else
    launch_block_mse_t<BF16, SUMS, mse_unroll(false)>(x, c, scales, block_mse, part, grid,
                                                      nitems, st);
}

hipError_t mxi_launch_block_mse(const void *x, int bf16, const uint8_t *codes,
                                const uint8_t *scales, int64_t nitems, float *block_mse,
                                double *tensor_sums, double *partial, int64_t partial_space,
                                hipStream_t st) {
  const bool large = nitems >= kLargeItems;
  const unsigned grid = error_grid(nitems, mse_unroll(large), tensor_sums != nullptr,
                                   partial_space);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  double *part = tensor_sums ? partial : nullptr;
  if (nitems > 0) {
    if (bf16) {
      if (part) launch_block_mse_u<true, true>(large, x, c, scales, block_mse, part, grid, nitems, st);
      else launch_block_mse_u<true, false>(large, x, c, scales, block_mse, part, grid, nitems, st);
    } else {
      if (part) launch_block_mse_u<false, true>(large, x, c, scales, block_mse, part, grid, nitems, st);
      else launch_block_mse_u<false, false>(large, x, c, scales, block_mse, part, grid, nitems, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tensor_sums) return sum_partials(partial, nitems > 0 ? grid : 0, tensor_sums, st);
  return hipSuccess;
}

// ---- fixed device scratch (block error without a workspace) -------------------
//
// The tensor sums of the block-error launch go through per-workgroup partial
// sums, two doubles per workgroup. mx_block_mse_noalloc keeps them here
// instead of in a caller workspace: 2 * 2048 doubles (32 KiB), which holds
// every tensor size because that call's launch is capped at 2048 workgroups
// when its fastest grid needs more (see error_grid). Each GPU the library
// runs on holds its own copy, at its own address, until the process ends;
// every call on a GPU shares it. A launch writes every partial slot it reads
// before the sum kernel reads it, so nothing has to start at zero.
constexpr size_t kScratchDoubles = 2 * 2048;
static __device__ __align__(256) double scratch[kScratchDoubles];

size_t mxi_scratch_partials() { return kScratchDoubles; }

// Device address of `scratch` on device `dev`. In host code the array's name
// is a host-side stand-in, not a device address, so it is looked up with
// hipGetSymbolAddress, with that device current, once per device, and only
// the looked-up address is handed to kernels.
hipError_t mxi_scratch_address(int dev, double **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static double *addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<double *>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

// Tiling of the MXFP8 kernels: the grid-capped small-tensor tiling (fake-quant
// as MXFP4 fake-quant, 3 % faster) below kLargeItems items, and on multi-GB
// bf16 tensors one tile per workgroup, no cap, 64-thread workgroups: on the
// 1.6e9-element MoE w13 experts quantize and fake-quant with one item per
// thread ran 12.6 % faster than the small-tensor tiling, dequantize with two
// 7.4 % faster (the XCD map of MXFP4 dequantize made it 3 % slower here; one
// item, or 256 threads, 2-6 % slower); dequantize later moved to two items
// per 128 threads (752 against 769 us on the w13 experts; four per 64:
// 844 us).
struct Tiling8 {
  int u, nt;
  int64_t cap;
};
constexpr Tiling8 tiling8(bool bf16, int kind, bool large) {
  if (bf16 && large) {
    if (kind == kKindQuantize) return {1, 64, kGridLimit};
    if (kind == kKindDequantize) return {2, 128, kGridLimit};
    return {1, 64, kGridLimit};
  }
  if (kind == kKindQuantize) return {bf16 ? kU8<true> : kU8<false>, kThreads, MX_GRID_CAP};
  if (kind == kKindDequantize) return {bf16 ? kU<true> : kU<false>, kThreads, MX_GRID_CAP};
  return {unroll_of(bf16, 0, kKindFakequant), kThreads, MX_GRID_CAP};
}

template <bool BF16, bool LARGE>
static void launch_quantize8_t(const void *x, int64_t nitems, u32x2 *c, uint8_t *scales,
                               hipStream_t st) {
  constexpr Tiling8 t = tiling8(BF16, kKindQuantize, LARGE);
  hipLaunchKernelGGL((k_quantize8<BF16, t.u, t.nt>), dim3(grid_for(nitems, t.cap, t.u, t.nt)),
                     dim3(t.nt), 0, st, x, c, scales, nitems);
}

hipError_t mxi_launch_quantize8(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                uint8_t *scales, hipStream_t st) {
  u32x2 *c = reinterpret_cast<u32x2 *>(codes);
  if (bf16 && nitems >= kLargeItems) launch_quantize8_t<true, true>(x, nitems, c, scales, st);
  else if (bf16) launch_quantize8_t<true, false>(x, nitems, c, scales, st);
  else launch_quantize8_t<false, false>(x, nitems, c, scales, st);
  return hipGetLastError();
}

template <bool BF16, bool LARGE>
static void launch_dequantize8_t(const u32x2 *c, const uint8_t *scales, int64_t nitems, void *y,
                                 hipStream_t st) {
  constexpr Tiling8 t = tiling8(BF16, kKindDequantize, LARGE);
  hipLaunchKernelGGL((k_dequantize8<BF16, t.u, t.nt>),
                     dim3(grid_for(nitems, t.cap, t.u, t.nt)), dim3(t.nt), 0, st, c, scales, y,
                     nitems);
}

hipError_t mxi_launch_dequantize8(const uint8_t *codes, const uint8_t *scales, int bf16,
                                  int64_t nitems, void *y, hipStream_t st) {
  const u32x2 *c = reinterpret_cast<const u32x2 *>(codes);
  if (bf16 && nitems >= kLargeItems) launch_dequantize8_t<true, true>(c, scales, nitems, y, st);
  else if (bf16) launch_dequantize8_t<true, false>(c, scales, nitems, y, st);
  else launch_dequantize8_t<false, false>(c, scales, nitems, y, st);
  return hipGetLastError();
}

template <bool BF16, bool LARGE>
static void launch_fakequant8_t(const void *x, int64_t nitems, void *y, hipStream_t st) {
  constexpr Tiling8 t = tiling8(BF16, kKindFakequant, LARGE);
  hipLaunchKernelGGL((k_fakequant8<BF16, t.u, t.nt>), dim3(grid_for(nitems, t.cap, t.u, t.nt)),
                     dim3(t.nt), 0, st, x, y, nitems);
}

hipError_t mxi_launch_fakequant8(const void *x, int bf16, int64_t nitems, void *y,
                                 hipStream_t st) {
  if (bf16 && nitems >= kLargeItems) launch_fakequant8_t<true, true>(x, nitems, y, st);
  else if (bf16) launch_fakequant8_t<true, false>(x, nitems, y, st);
  else launch_fakequant8_t<false, false>(x, nitems, y, st);
  return hipGetLastError();
}

// Workspace words of an NVFP4 call: one maximum per first-pass workgroup,
// then the tensor exponent the multi-GB path reduces them to.
size_t mxi_nvfp4_partials(int64_t nitems) { return grid_for(nitems, MX_NV_GRID_CAP) + 1; }

// The block pass on multi-GB bf16 tensors: k_nv_prepare reduces the maxima
// once, then one tile per workgroup with no grid cap, quantize two items per
// 128 threads (with non-temporal code stores, nt_codes) and fake-quant one
// per 256. On the 1.6e9-element MoE w13 experts both passes took 1081
// against 1384 us (quantize) and 1436 against 1749 us (fake-quant) for the
// 2048-workgroup grid that loops over tiles; 1 x 256, 1 x 128 and 4 x 256
// quantize took 1128-1177 us, 2 x 128, 1 x 128 and 4 x 256 fake-quant
// 1437-1596 us.
template <bool FQ>
static void launch_nv_large(const void *x, uint32_t *partial, unsigned gp, uint32_t *c,
                            uint8_t *block_scales, uint8_t *tensor_scale, void *y, int64_t nitems,
                            hipStream_t st) {
  constexpr int U = FQ ? 1 : 2, NT = FQ ? 256 : 128;
  hipLaunchKernelGGL(k_nv_prepare, dim3(1), dim3(kThreads), 0, st, partial, (int)gp,
                     FQ ? nullptr : tensor_scale);
  hipLaunchKernelGGL((k_quantize_nv_big<true, FQ, U, NT>),
                     dim3(grid_for(nitems, kGridLimit, U, NT)), dim3(NT), 0, st, x, partial,
                     (int)gp, c, block_scales, tensor_scale, y, nitems);
}

hipError_t mxi_launch_quantize_nv(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                  uint8_t *block_scales, uint8_t *tensor_scale,
                                  uint32_t *partial, void *y, hipStream_t st) {
  const unsigned gp = grid_for(nitems, MX_NV_GRID_CAP);
  const dim3 g(gp), b(kThreads);
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  if (bf16) {
    hipLaunchKernelGGL((k_absmax_partials<true>), dim3(gp), b, 0, st, x, partial, nitems);
    if (nitems >= kLargeItems) {
      if (y) launch_nv_large<true>(x, partial, gp, c, block_scales, tensor_scale, y, nitems, st);
      else launch_nv_large<false>(x, partial, gp, c, block_scales, tensor_scale, y, nitems, st);
    } else if (y)
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

// Tiling of the MBS-Static kernels, as for MXFP8: grid-capped below
// kLargeItems items (quantize four items per thread, dequantize two as MXFP4
// dequantize: 2.5 % faster), and on multi-GB bf16 tensors one tile per
// workgroup with no cap: quantize two items per 128-thread workgroup and
// fake-quant one per 256 threads (on the 1.6e9-element MoE w13 experts
// fake-quant 10 % faster than the small-tensor tiling; 64 x 1, 128 x 1 and
// 128 x 2 equal or up to 4 % slower), dequantize two items per 64 threads
// (3 % faster; 128 threads equal). Quantize stores its code words
// non-temporally at every size: on the MoE w13 experts 128 x 2 with the hint
// took 626 against 711 us for 256 x 1 without it (128 x 1: 734 us, 64 x 2:
// 686 us), on bf16 16384x8192 activations the hint alone 4 % less, on
// 8192x4096 the same.
struct TilingMbs {
  int u, nt;
  int64_t cap;
};
constexpr TilingMbs tiling_mbs(bool bf16, int kind, bool large) {
  if (bf16 && large) {
    if (kind == kKindDequantize) return {2, 64, kGridLimit};
    if (kind == kKindQuantize) return {2, 128, kGridLimit};
    return {1, 256, kGridLimit};  // fake-quant
  }
  if (kind == kKindDequantize) return {unroll_of(bf16, 0, kKindDequantize), kThreads, MX_GRID_CAP};
  return {bf16 ? kU<true> : kU<false>, kThreads, MX_GRID_CAP};
}

template <bool BF16, bool FQ, bool LARGE>
static void launch_quantize_mbs_t(const void *x, int64_t nitems, uint32_t *c, uint8_t *sub_scales,
                                  uint8_t *macro_mant, void *y, hipStream_t st) {
  constexpr TilingMbs t = tiling_mbs(BF16, FQ ? kKindFakequant : kKindQuantize, LARGE);
  hipLaunchKernelGGL((k_quantize_mbs<BF16, FQ, t.u, t.nt>),
                     dim3(grid_for(nitems, t.cap, t.u, t.nt)), dim3(t.nt), 0, st, x, c,
                     sub_scales, macro_mant, y, nitems);
}

hipError_t mxi_launch_quantize_mbs(const void *x, int bf16, int64_t nitems, uint8_t *codes,
                                   uint8_t *sub_scales, uint8_t *macro_mant, void *y,
                                   hipStream_t st) {
  uint32_t *c = reinterpret_cast<uint32_t *>(codes);
  const bool large = bf16 && nitems >= kLargeItems;
  if (bf16) {
    if (large) {
      if (y) launch_quantize_mbs_t<true, true, true>(x, nitems, c, sub_scales, macro_mant, y, st);
      else launch_quantize_mbs_t<true, false, true>(x, nitems, c, sub_scales, macro_mant, y, st);
    } else {
      if (y) launch_quantize_mbs_t<true, true, false>(x, nitems, c, sub_scales, macro_mant, y, st);
      else launch_quantize_mbs_t<true, false, false>(x, nitems, c, sub_scales, macro_mant, y, st);
    }
  } else {
    if (y) launch_quantize_mbs_t<false, true, false>(x, nitems, c, sub_scales, macro_mant, y, st);
    else launch_quantize_mbs_t<false, false, false>(x, nitems, c, sub_scales, macro_mant, y, st);
  }
  return hipGetLastError();
}

template <bool BF16, bool LARGE>
static void launch_dequantize_mbs_t(const uint32_t *c, const uint8_t *sub_scales,
                                    const uint8_t *macro_mant, int64_t nitems, void *y,
                                    hipStream_t st) {
  constexpr TilingMbs t = tiling_mbs(BF16, kKindDequantize, LARGE);
  hipLaunchKernelGGL((k_dequantize_mbs<BF16, t.u, t.nt>),
                     dim3(grid_for(nitems, t.cap, t.u, t.nt)), dim3(t.nt), 0, st, c, sub_scales,
                     macro_mant, y, nitems);
}

hipError_t mxi_launch_dequantize_mbs(const uint8_t *codes, const uint8_t *sub_scales,
                                     const uint8_t *macro_mant, int bf16, int64_t nitems, void *y,
                                     hipStream_t st) {
  const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
  if (bf16 && nitems >= kLargeItems)
    launch_dequantize_mbs_t<true, true>(c, sub_scales, macro_mant, nitems, y, st);
  else if (bf16)
    launch_dequantize_mbs_t<true, false>(c, sub_scales, macro_mant, nitems, y, st);
  else
    launch_dequantize_mbs_t<false, false>(c, sub_scales, macro_mant, nitems, y, st);
  return hipGetLastError();
}

// Launch plan of a multi-tensor call (host only): the non-empty tensors,
// largest first (stable), in launches of at most max_per_launch tensors whose
// tile counts are at least 7/8 of the launch's first one, so at most 1/8 of
// a launch's workgroups are idle. order[] receives the tensor indices in
// launch order, first[l] the position in order[] where launch l starts
// (first[L] = the number of non-empty tensors), gx[l] the tiles of launch
// l's first tensor (its grid's x size); each array holds count + 1 entries.
// Returns the number of launches L, or -1 if a tensor has more tiles than
// one grid dimension takes (nothing is then launched).
int mxi_multi_plan(const int64_t *nitems, int count, int64_t tile, int max_per_launch, int *order,
                   int *first, int64_t *gx) {
  int m = 0;
  for (int i = 0; i < count; i++)
    if (nitems[i] > 0) order[m++] = i;
  std::stable_sort(order, order + m, [&](int p, int q) { return nitems[p] > nitems[q]; });
  int launches = 0, i = 0;
  while (i < m) {
    const int64_t g = (nitems[order[i]] + tile - 1) / tile;
    if (g > kGridLimit) return -1;
    first[launches] = i;
    gx[launches++] = g;
    int n = 0;
    for (; i < m && n < max_per_launch; i++, n++)
      if (8 * ((nitems[order[i]] + tile - 1) / tile) < 7 * g) break;
  }
  first[launches] = m;
  return launches;
}

hipError_t mxi_launch_multi(const MxiTensor *t, int count, int bf16, int mode, int fakequant,
                            hipStream_t st) {
  const int kind = fakequant ? kKindFakequant : kKindQuantize;
  // the large-tensor tiling when the call as a whole streams that much
  int64_t total = 0;
  std::vector<int64_t> items(count);
  for (int i = 0; i < count; i++) {
    items[i] = t[i].nitems;
    total += t[i].nitems > 0 ? t[i].nitems : 0;
  }
  const bool large = bf16 && total >= kLargeItems;
  const int nt = large ? threads_of(true, mode, kind, true) : threads_of(bf16, mode, kind);
  const int64_t tile = (int64_t)nt * (large ? unroll_of(true, mode, kind, true)
                                            : unroll_of(bf16, mode, kind));
  std::vector<int> order(count + 1), first(count + 1);
  std::vector<int64_t> gx(count + 1);
  const int launches = mxi_multi_plan(items.data(), count, tile, MX_MULTI_MAX, order.data(),
                                      first.data(), gx.data());
  if (launches < 0) return hipErrorInvalidValue;
  for (int l = 0; l < launches; l++) {
    MultiArgs a;
    const int n = first[l + 1] - first[l];
    for (int j = 0; j < n; j++) {
      const MxiTensor &q = t[order[first[l] + j]];
      a.d[j] = {q.x, q.out, q.scales, q.nitems};
    }
    const dim3 g((unsigned)gx[l], (unsigned)n), b((unsigned)nt);
    if (bf16) {
      if (large) {
        if (fakequant) { MX_DISPATCH_MULTI(true, true, true, mode, g, b, st, a) }
        else { MX_DISPATCH_MULTI(true, false, true, mode, g, b, st, a) }
      } else {
        if (fakequant) { MX_DISPATCH_MULTI(true, true, false, mode, g, b, st, a) }
        else { MX_DISPATCH_MULTI(true, false, false, mode, g, b, st, a) }
      }
    } else {
      if (fakequant) { MX_DISPATCH_MULTI(false, true, false, mode, g, b, st, a) }
      else { MX_DISPATCH_MULTI(false, false, false, mode, g, b, st, a) }
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
                                     double *tensor_sums, double *partial, int64_t partial_space,
                                     hipStream_t st) {
  const unsigned grid = error_grid(nitems, kFusedU, tensor_sums != nullptr, partial_space);
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
  if (tensor_sums) return sum_partials(partial, nitems > 0 ? grid : 0, tensor_sums, st);
  return hipSuccess;
}
