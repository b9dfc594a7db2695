// Shared device helpers for the gfx950 MoE kernels: vector types, exact
// format conversions, wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

namespace moe {

// bf16 bits -> f32: the bf16 pattern is the top half of the f32 pattern
// (dragon.c page, section 8 Round 3: bf16 -> f32 is a 16-bit left shift).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// UE8M0 byte -> the f32 power of two 2^(b-127) (b = 0 gives the subnormal
// 2^-127; b = 255 is not produced by the format's encoder).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Two OCP e4m3 codes (bytes 0,1 of w, or 2,3 with HI) -> two exact f32.
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Same pairs -> bf16 (exact: every e4m3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// Two e2m1 codes (byte `sel` of w: low nibble first) times a power-of-two
// scale -> bf16x2 / f32x2, exact while the result stays a normal number.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// One OCP e4m3 code (low byte of b) -> its exact f32 value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(b, false)[0];
}

// Two e2m1 codes (byte `sel` of w, low nibble first) times an e4m3 scale
// value -> bf16x2, exact.  The scaled conversion above applies only the
// exponent of its scale operand, so a non-power-of-two scale is applied here:
// decode at scale 1, multiply in f32 (e2m1 has at most 2 significant bits and
// e4m3 at most 4, so the product is exact and has at most 6), and keep the top
// 16 bits of each product, which for such a value is the bf16 value itself.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_times_to_bf16(uint32_t w, float scale) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  const uint32_t a = __float_as_uint(v.x * scale), b = __float_as_uint(v.y * scale);
  return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(b, a, 0x07060302u));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes, returned to every lane (uniform).  DPP moves sum
// each row of 16 lanes (quad swaps, then half-row and row mirrors); the four
// row sums are read out with v_readlane and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// Unsigned maximum over the 64 lanes, returned to every lane (uniform).
__device__ __forceinline__ uint32_t dpp_u32max(uint32_t v, uint32_t o) { return v > o ? v : o; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_u32max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = dpp_u32max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = dpp_u32max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = dpp_u32max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return dpp_u32max(dpp_u32max(a, b), dpp_u32max(c, d));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / WAVE; }

// silu(g) = g * sigma(g), the logistic by the hardware reciprocal (1 ulp; the
// result is rounded to bf16 next, 2^16 times coarser).  For g below about -88
// exp overflows, the reciprocal of infinity is 0 and silu is -0.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

}  // namespace moe
