// Device helpers shared by the gfx950 kernels: vector types, MXFP4 -> bf16
// conversion, bf16 rounding, wave-level bit tricks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

// E8M0 scale byte as the float operand of the gfx950 scaled converts.  The
// converts take only the exponent field of this operand, so s << 23 encodes
// 2^(s-127) for every byte 0..254 (byte 0 included); this was checked on all
// 16 codes x 255 finite scale bytes against the exact values.
__device__ __forceinline__ float e8m0_operand(uint32_t s) { return __uint_as_float(s << 23); }

// Two E2M1 codes (byte `SEL` of `packed`; low nibble -> low half) times the
// scale, rounded to bf16.  Exact for finite scales (the products have at most
// two significant bits and stay inside bf16's range or overflow to +-inf).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t packed, float scale) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight E2M1 codes (one dword, element 0 in the low nibble) -> eight bf16.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t packed, float scale) {
  u32x4 o;
  o[0] = fp4x2_to_bf16x2<0>(packed, scale);
  o[1] = fp4x2_to_bf16x2<1>(packed, scale);
  o[2] = fp4x2_to_bf16x2<2>(packed, scale);
  o[3] = fp4x2_to_bf16x2<3>(packed, scale);
  return o;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// float -> bf16 bits, round to nearest, ties to even; NaN -> 0x7FC0.
// FP8 E4M3 byte (OCP, finite-only: 4 exponent bits with bias 7, 3 mantissa
// bits, exponent field 0 subnormal, S.1111.111 NaN) -> float, exactly.  The
// NVFP4 block scale.
__device__ __forceinline__ float e4m3_operand(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  if ((b & 0x7fu) == 0x7fu) v = __builtin_nanf("");
  return (b & 0x80u) ? -v : v;
}

// Two floats -> two bf16 (round to nearest even) packed low/high, with the
// gfx950 conversion instruction (one v_cvt_pk_bf16_f32).
typedef __attribute__((ext_vector_type(2))) float f32x2v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// Eight E2M1 codes (one dword, low nibble first) times an arbitrary float
// scale -> eight bf16.  The scaled conversions above apply only the exponent
// of their float scale (a power of two, as an E8M0 scale is), so a scale with
// mantissa bits (an NVFP4 E4M3 block scale) is applied here in float32:
// codes -> exact floats, times the scale, then bf16 round to nearest even
// (exact when the product fits in 8 significant bits, as code x E4M3 does).
typedef __attribute__((ext_vector_type(2))) float f32x2e;
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8_any_scale(uint32_t packed, float scale) {
  u32x4 r;
  f32x2e v;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0);
  r[0] = pack_bf16x2_rne(v.x * scale, v.y * scale);
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1);
  r[1] = pack_bf16x2_rne(v.x * scale, v.y * scale);
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2);
  r[2] = pack_bf16x2_rne(v.x * scale, v.y * scale);
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3);
  r[3] = pack_bf16x2_rne(v.x * scale, v.y * scale);
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Number of set bits of `mask` below this lane (wave64).
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace mx
