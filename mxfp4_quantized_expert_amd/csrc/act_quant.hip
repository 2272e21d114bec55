// Block-scaled FP8 activations for the FP4 scaled-MFMA path (opt-in).
//
// Encodings of the OCP Microscaling Formats v1.0: MXFP8 E4M3 elements in
// blocks of 32 along K sharing one E8M0 scale.  The shared exponent is this
// implementation's own choice, floor(log2(max|v|)) - 7, one more than the
// specification's floor(log2(max|v|)) - emax (emax = 8 for E4M3): scaled
// magnitudes stay below 256, so no element needs clamping.  An all-zero block
// takes 127; elements round to nearest, ties to even.  "split"
// activations add the MXFP8 tensor of the residual v - hi, which brings the
// product within about 2^-8 of the block maximum of the exact bf16 value.
//
// Output layout, made for the GEMM's staging: per row, per 64-wide K chunk c,
// 128 bytes = the 64 high codes of K [64c, 64c+64) then the 64 residual
// codes; and 4 scale bytes = high scale of groups 2c and 2c+1, residual
// scale of groups 2c and 2c+1.  A chunk past K (K a multiple of 32 but not of
// 64) is padded with zero codes and scale 127.
#include "internal.h"
#include "mx_device.h"

namespace {

// E4M3 code of y (|y| < 256), round to nearest, ties to even.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(a * 0x1p9f);  // subnormal quantum 2^-9 (8 -> 2^-6, the first normal)
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 255u) - 127;      // binade, -6 .. 7
    const uint32_t m = (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));    // 8 .. 16
    code = ((uint32_t)(e + 7) << 3) + (m - 8);                         // m == 16 carries into the exponent
  }
  return code | (y < 0.f || (y == 0.f && __builtin_signbit(y)) ? 0x80u : 0u);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -v : v;
}

// Scale byte of a block with maximum magnitude amax.
__device__ __forceinline__ int mx_scale_byte(float amax) {
  if (amax == 0.f) return 127;
  const int x = ilogbf(amax) - 7;
  return min(max(x + 127, 0), 254);
}

// Quantizes the 32 values v (in place: returns the codes packed 4 per dword in
// q) and returns the scale byte; r receives v - dequantized value.
__device__ __forceinline__ int quantize32(const float (&v)[32], uint32_t (&q)[8], float (&r)[32]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int sb = mx_scale_byte(amax);
  const int x = sb - 127;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * d + k;
      const uint32_t c = e4m3_rne(ldexpf(v[i], -x));
      r[i] = v[i] - ldexpf(e4m3_value(c), x);  // exact in fp32
      w |= c << (8 * k);
    }
    q[d] = w;
  }
  return sb;
}

// One thread per (row, 32-wide group); groups past K write the padding.
template <bool kSplit>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ src, int rows, int K,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int ngroups = 2 * ((K + 63) >> 6);  // padded to whole chunks
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)rows * ngroups) return;
  const int row = (int)(idx / ngroups);
  const int g = (int)(idx - (long)row * ngroups);
  const int c = g >> 1, h = g & 1;
  const size_t row_bytes = (size_t)64 * ngroups;  // 128 per chunk
  uint8_t* dst = codes + (size_t)row * row_bytes + (size_t)c * 128 + 32 * h;
  uint8_t* sdst = scales + (size_t)row * (2 * ngroups) + (size_t)c * 4 + h;
  uint32_t hq[8], lq[8];
  int hs = 127, ls = 127;
  if (32 * g < K) {
    float v[32], r[32], r2[32];
    const mx::u32x4* p = reinterpret_cast<const mx::u32x4*>(src + (size_t)row * K + 32 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const mx::u32x4 w = p[j];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * j + 2 * k] = mx::bf16_to_f32(w[k] & 0xffffu);
        v[8 * j + 2 * k + 1] = mx::bf16_to_f32(w[k] >> 16);
      }
    }
    hs = quantize32(v, hq, r);
    if (kSplit) ls = quantize32(r, lq, r2);
  }
  if (32 * g >= K) {
#pragma unroll
    for (int d = 0; d < 8; ++d) hq[d] = 0u;
  }
  if (!kSplit || 32 * g >= K) {
#pragma unroll
    for (int d = 0; d < 8; ++d) lq[d] = 0u;
  }
  mx::u32x4* o = reinterpret_cast<mx::u32x4*>(dst);
  o[0] = mx::u32x4{hq[0], hq[1], hq[2], hq[3]};
  o[1] = mx::u32x4{hq[4], hq[5], hq[6], hq[7]};
  o[4] = mx::u32x4{lq[0], lq[1], lq[2], lq[3]};  // +64 bytes: the residual half of the chunk
  o[5] = mx::u32x4{lq[4], lq[5], lq[6], lq[7]};
  sdst[0] = (uint8_t)hs;
  sdst[2] = (uint8_t)ls;
}

}  // namespace

namespace mxfp4moe {

size_t act_quant_row_bytes(int K) { return (size_t)128 * ((K + 63) / 64); }
size_t act_quant_scale_row_bytes(int K) { return (size_t)4 * ((K + 63) / 64); }

hipError_t launch_act_quant(const uint16_t* src, int rows, int K, bool split, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  const long n = (long)rows * 2 * ((K + 63) / 64);
  if (n == 0) return hipSuccess;
  ProfileScope prof(kStageActQuant, stream);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (split)
    act_quant_kernel<true><<<grid, 256, 0, stream>>>(src, rows, K, codes, scales);
  else
    act_quant_kernel<false><<<grid, 256, 0, stream>>>(src, rows, K, codes, scales);
  return hipGetLastError();
}

}  // namespace mxfp4moe
