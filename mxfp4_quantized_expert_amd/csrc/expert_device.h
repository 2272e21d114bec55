// Device helpers of the expert GEMM kernels (prefill tiles and the decode
// path): the clamped SwiGLU of the gpt-oss experts, the gate/up row layouts of
// w13, bias reads, MXFP4 / NVFP4 group conversion, and scale-row staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.h"

namespace mxgemm {

using mx::f32x4;
using mx::u32x4;

__device__ __forceinline__ float swiglu_clamped(float gate, float up) {
  // gpt-oss family constants: alpha 1.702, limit 7; gate clamped from above,
  // up clamped on both sides, +1 after the clamp.  The clamps are IEEE 754-2019
  // minimum / maximum (gfx950's v_minimum3_f32 / v_maximum3_f32), which keep a
  // NaN input (a weight group with a NaN scale) NaN instead of turning it into
  // the limit, and equal the plain clamp for every other input (+-inf
  // included): one instruction each instead of a compare and a select.
  const float g = __builtin_elementwise_minimum(gate, 7.0f);
  const float u = __builtin_elementwise_maximum(__builtin_elementwise_minimum(up, 7.0f), -7.0f);
  // sigmoid(alpha g) = 1 / (1 + 2^(-alpha log2(e) g)) through the hardware
  // exp2 and reciprocal (about 1 ulp each; the result is rounded to bf16).
  // g * sigmoid first (a very negative gate gives -0, not an overflow), then
  // times (u + 1) as one fused multiply-add.
  constexpr float kNegAlphaLog2e = -1.702f * 1.4426950408889634f;
  const float gs = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(kNegAlphaLog2e * g));
  return __builtin_fmaf(gs, u, gs);
}

// gate/up row layout of w13.  Logical row 2i is gate i and 2i+1 is up i (the
// order every kernel computes in).  Interleaved checkpoints store them so;
// split ones ("feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss",
// FreeToken PR #838, "What it does": swigluoai is the uninterleaved spelling
// of the same activation) store the I gate rows first, then the I up rows.
__device__ __forceinline__ int w13_row(int r, int N, bool split) {
  return split ? ((r & 1) ? (N >> 1) + (r >> 1) : (r >> 1)) : r;
}
// LDS row of block-local logical row rl after stage_scales (split: the block's
// gate rows, then its up rows).
__device__ __forceinline__ int staged_row(int rl, int nv, bool split) {
  return split ? ((rl & 1) ? (nv >> 1) + (rl >> 1) : (rl >> 1)) : rl;
}
// The two dwords of bf16 biases that hold logical rows n..n+3 (n a multiple
// of 4, below N), as loaded: interleaved rows n, n+1 | n+2, n+3; split: gate
// n/2, n/2+1 | up n/2, n/2+1.  Branch-free (the same two loads either way),
// so a caller can issue many of them before the first use.
__device__ __forceinline__ uint2 load_bias4_raw(const uint16_t* bias, int n, int N, bool split) {
  const int a0 = split ? (n >> 1) : n;
  const int a1 = split ? (N >> 1) + (n >> 1) : n + 2;
  return uint2{*reinterpret_cast<const uint32_t*>(bias + a0), *reinterpret_cast<const uint32_t*>(bias + a1)};
}
// ... and the four biases of rows n..n+3 in order.
__device__ __forceinline__ f32x4 bias4_of(uint2 d, bool split) {
  const uint32_t lo = split ? (d.x & 0xffffu) | (d.y << 16) : d.x;
  const uint32_t hi = split ? (d.x >> 16) | (d.y & 0xffff0000u) : d.y;
  return f32x4{mx::bf16_to_f32(lo & 0xffffu), mx::bf16_to_f32(lo >> 16), mx::bf16_to_f32(hi & 0xffffu),
               mx::bf16_to_f32(hi >> 16)};
}
// Biases of logical rows n..n+3 (n a multiple of 4, below N).
__device__ __forceinline__ f32x4 load_bias4(const uint16_t* bias, int n, int N, bool split) {
  return bias4_of(load_bias4_raw(bias, n, N, split), split);
}

// Scale operands of the 32 codes a lane converts at once (one 16-byte piece).
// MXFP4: one E8M0 byte for all 32.  NVFP4: two E4M3 block scales, the first
// for the codes of steps 0 and 1, the second for steps 2 and 3; the result is
// exact in bf16 (a code has at most 2 significant bits, an E4M3 value 4).
// A NaN scale (E8M0 0xFF, E4M3 S.1111.111) makes every weight of its group
// NaN through the conversion itself (see e8m0_operand).
template <bool kNv>
struct GroupScale {
  float lo, hi;
  __device__ __forceinline__ GroupScale(const uint8_t* srow, int g) : GroupScale(kNv ? srow[2 * g] : srow[g],
                                                                                   kNv ? srow[2 * g + 1] : 0u) {}
  // from the group's scale byte(s) already read (b1 only for NVFP4)
  __device__ __forceinline__ GroupScale(uint32_t b0, uint32_t b1) {
    if (kNv) {
      const mx::f32x2p v = mx::e4m3x2_operands(b0 | (b1 << 8));
      lo = v.x;
      hi = v.y;
    } else {
      lo = hi = mx::e8m0_operand(b0);
    }
  }
  __device__ __forceinline__ float step(int s) const { return s < 2 ? lo : hi; }
  // eight codes of step s as bf16
  __device__ __forceinline__ u32x4 convert(uint32_t packed, int s) const {
    return kNv ? mx::fp4x8_to_bf16x8_any_scale(packed, step(s)) : mx::fp4x8_to_bf16x8(packed, step(s));
  }
};

// 16 bytes per lane from global memory straight into LDS (the load unit
// writes lane l's bytes at lds + 16 * l; lds is the same for the whole wave).
__device__ __forceinline__ void load_lds16(const void* src, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// 4 bytes per lane from global memory straight into LDS (lane l's word at lds + 4 * l).
__device__ __forceinline__ void load_lds4(const void* src, uint32_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// Scale bytes of a block's BN weight rows, row-major as in memory: the rows
// are one contiguous, 32-byte aligned range (row counts and tile starts are
// multiples of 32), copied with 16-byte loads.  Rows past N are not copied
// (their outputs are dropped).  kDma: the load unit writes LDS itself
// (global_load_lds, lane l of a wave at the wave's slot + 16 * l), so the
// copy flies with the first operand loads instead of waiting to be stored;
// the caller waits for it (vmcnt) before the first barrier.
template <int BN, int kThreads, bool kDma = false>
__device__ __forceinline__ void stage_scales(uint8_t* sst, const uint8_t* wscales, int N, int e, int ntile,
                                             int kgroups, int t, bool split = false) {
  // wscales [E, N, kgroups]; kgroups: scale bytes per weight row (K/32 for
  // MXFP4, K/16 for NVFP4)
  const int nv = min(BN, N - ntile * BN);
  u32x4* dst = reinterpret_cast<u32x4*>(sst);
  // the block's rows (split layout: its gate rows, then its up rows; each
  // range contiguous and 16-byte aligned)
  const int n16 = (nv * kgroups) >> 4;
  const int h = split ? ((nv >> 1) * kgroups) >> 4 : n16;
  const u32x4* g = reinterpret_cast<const u32x4*>(
      wscales + ((size_t)e * N + (split ? ntile * BN >> 1 : ntile * BN)) * (size_t)kgroups);
  const u32x4* u =
      reinterpret_cast<const u32x4*>(wscales + ((size_t)e * N + (N >> 1) + (ntile * BN >> 1)) * (size_t)kgroups);
  if (kDma) {
    for (int i0 = 0; i0 < n16; i0 += kThreads) {  // the same trip count in every wave
      const int i = i0 + t;
      if (i < n16) load_lds16(i < h ? g + i : u + (i - h), dst + i0 + (t & ~63));
    }
  } else {
    for (int i = t; i < n16; i += kThreads) dst[i] = i < h ? g[i] : u[i - h];
  }
}

// Four fp32 values as four bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint2 pack_bf16x4(const f32x4& v) {
  return uint2{mx::pack_bf16x2_rne(v[0], v[1]), mx::pack_bf16x2_rne(v[2], v[3])};
}


// Waits until at most kVm of this wave's vector-memory loads are in flight
// and its LDS operations are done, then joins the block barrier.  The empty
// asm statements keep the compiler from moving memory accesses across it
// (the barrier builtin alone is not a memory fence to the compiler).
template <int kVm>
__device__ __forceinline__ void wait_loads_then_barrier() {
  static_assert(kVm >= 0 && kVm < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);  // nothing (MFMAs included) is scheduled across the wait
  asm volatile("" ::: "memory");
  // s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt 11:8 (0)
  __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Waits until this wave's LDS reads are done (vector-memory loads may stay in
// flight), then joins the block barrier: after it no wave still reads what a
// load issued afterwards will overwrite.
__device__ __forceinline__ void lds_reads_then_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  // s_waitcnt fields: vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace mxgemm
