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
// 16 codes x 255 finite scale bytes against the exact values.  Byte 0xFF
// (exponent field all ones) is the E8M0 NaN, and the converts follow that
// rule themselves: every code of such a group converts to NaN (checked on
// gfx950 hardware for all 16 codes, bf16 and f32 forms), so a NaN scale needs
// no handling of its own.
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

// Two FP8 E4M3 bytes (OCP, finite-only: 4 exponent bits with bias 7, 3
// mantissa bits, exponent field 0 subnormal, S.1111.111 NaN; bits 0-7 and
// 8-15 of `two`) -> two floats, exactly, in one v_cvt_pk_f32_fp8: the NVFP4
// block scales of a 32-code group.  gfx950's conversion follows the OCP
// encoding; it was checked on gfx950 hardware against the exact decode (sign,
// subnormals, NaN) for all 256 byte values.
typedef __attribute__((ext_vector_type(2))) float f32x2p;
__device__ __forceinline__ f32x2p e4m3x2_operands(uint32_t two) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
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
// Two codes (byte SEL of `packed`, low nibble -> low half) of the above.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2_any_scale(uint32_t packed, float scale) {
  const f32x2e v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
  return pack_bf16x2_rne(v.x * scale, v.y * scale);
}
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8_any_scale(uint32_t packed, float scale) {
  u32x4 r;
  r[0] = fp4x2_to_bf16x2_any_scale<0>(packed, scale);
  r[1] = fp4x2_to_bf16x2_any_scale<1>(packed, scale);
  r[2] = fp4x2_to_bf16x2_any_scale<2>(packed, scale);
  r[3] = fp4x2_to_bf16x2_any_scale<3>(packed, scale);
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// f16 forms, for NVFP4 weights: E2M1 x an E4M3 block scale has at most six
// significant bits and lies in [2^-10, 2688], so it is exact in f16.  The
// scaled convert applies the scale's power of two (only its exponent field
// counts, as for the bf16 convert), one packed f16 multiply its mantissa.
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2v;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t packed, float pow2) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, pow2, SEL));
}
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2v, a) * __builtin_bit_cast(f16x2v, b));
}
// Two floats -> two f16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_f16x2_rne(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v));
}
// An E4M3 scale as a float split into its power of two (the convert's scale
// operand) and its significand in [1, 2) with the sign, as an f16 pair (a NaN
// scale gives a NaN significand, so every product of its group is NaN).
__device__ __forceinline__ void split_scale_f16(float s, float& pow2, uint32_t& mant2) {
  const uint32_t b = __float_as_uint(s);
  pow2 = __uint_as_float(b & 0x7F800000u);
  const float m = s != s ? s : __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u);
  const f32x2v mm = {m, m};
  mant2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(mm, f16x2v));
}

// Number of set bits of `mask` below this lane (wave64).
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Cross-lane steps on the DPP datapath (GFX9 control encodings): a lane
// reads another lane's register inside one VALU instruction, without a trip
// through the LDS permute unit.  A wave is four rows of 16 lanes.  Every
// helper below expects all 64 lanes of the wave to be active.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

// The value of the lane the control selects; 0 where a row shift reaches
// past the start of the row.
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, kCtrl, 0xf, 0xf, true);
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)dpp_i32<kCtrl>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)dpp_i32<kCtrl>((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the 16 lanes of each row.
__device__ __forceinline__ int row_inclusive_sum(int x) {
  x += dpp_i32<kDppRowShr1>(x);
  x += dpp_i32<kDppRowShr2>(x);
  x += dpp_i32<kDppRowShr4>(x);
  x += dpp_i32<kDppRowShr8>(x);
  return x;
}

// Inclusive prefix sum over the wave: row scans, then the earlier rows'
// totals added from scalar reads of lanes 15, 31 and 47.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x = row_inclusive_sum(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane_id() >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest key of the wave, returned to every lane: butterfly inside each row
// (every lane then holds its row's largest), then the four rows' values.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = max_u64(k, dpp_u64<kDppQuadXor1>(k));
  k = max_u64(k, dpp_u64<kDppQuadXor2>(k));
  k = max_u64(k, dpp_u64<kDppRowRor4>(k));
  k = max_u64(k, dpp_u64<kDppRowRor8>(k));
  return max_u64(max_u64(readlane_u64(k, 0), readlane_u64(k, 16)), max_u64(readlane_u64(k, 32), readlane_u64(k, 48)));
}

// Sum over the wave in a fixed order (the same bits on every call with the
// same inputs), returned to every lane.
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += __int_as_float(dpp_i32<kDppQuadXor1>(__float_as_int(x)));
  x += __int_as_float(dpp_i32<kDppQuadXor2>(__float_as_int(x)));
  x += __int_as_float(dpp_i32<kDppRowRor4>(__float_as_int(x)));
  x += __int_as_float(dpp_i32<kDppRowRor8>(__float_as_int(x)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace mx
