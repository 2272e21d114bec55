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
// Two floats -> two bf16 (round to nearest even) packed low/high, with the
// gfx950 conversion instruction (one v_cvt_pk_bf16_f32).
typedef __attribute__((ext_vector_type(2))) float f32x2v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Number of set bits of `mask` below this lane (wave64).
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace mx
