// Standalone MXFP4 -> bf16 dequant ("dequant-on-copy", MoE-Infinity PR #152,
// Changes): a pure HBM streaming kernel.
//
// The packed rows [N, K/2] and their scales [N, K/32] are one flat stream of
// 32-element groups: group g owns block bytes [16g, 16g+16), scale byte g and
// output elements [32g, 32g+32).  A thread converts one dword of blocks (eight
// codes, a quarter group) into four dwords of bf16.  Consecutive lanes take
// consecutive dwords, so every load instruction of a wave reads 256 contiguous
// bytes and every store instruction writes 1 KiB contiguous bytes.
#include "internal.h"
#include "mx_device.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // dwords per thread per iteration, kThreads apart

__global__ __launch_bounds__(kThreads) void mxfp4_dequant_kernel(const uint32_t* __restrict__ blocks,
                                                                 const uint8_t* __restrict__ scales,
                                                                 mx::u32x4* __restrict__ out,
                                                                 uint64_t n_dwords) {
  const uint64_t per_iter = (uint64_t)gridDim.x * kThreads * kUnroll;
  for (uint64_t base = (uint64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n_dwords;
       base += per_iter) {
    uint32_t w[kUnroll];
    uint32_t s[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t d = base + (uint64_t)u * kThreads;
      if (d < n_dwords) {
        w[u] = __builtin_nontemporal_load(blocks + d);
        s[u] = scales[d >> 2];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t d = base + (uint64_t)u * kThreads;
      if (d < n_dwords) {
        mx::u32x4 o = mx::fp4x8_to_bf16x8(w[u], mx::e8m0_operand(s[u]));
        if (s[u] == 255u) o = mx::u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
        __builtin_nontemporal_store(o, out + d);
      }
    }
  }
}

}  // namespace

namespace mxfp4moe {

hipError_t launch_dequant(const uint8_t* blocks, const uint8_t* scales, uint16_t* out, int64_t N, int64_t K,
                          hipStream_t stream) {
  const uint64_t n_dwords = (uint64_t)N * (uint64_t)K / 8;
  if (n_dwords == 0) return hipSuccess;
  const uint64_t per_block = (uint64_t)kThreads * kUnroll;
  uint64_t blocks_needed = (n_dwords + per_block - 1) / per_block;
  const uint64_t cap = (uint64_t)device_cu_count() * 32;
  const unsigned grid = (unsigned)(blocks_needed < cap ? blocks_needed : cap);
  ProfileScope prof(kStageDequant, stream);
  mxfp4_dequant_kernel<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint32_t*>(blocks), scales,
                                                      reinterpret_cast<mx::u32x4*>(out), n_dwords);
  return hipGetLastError();
}

}  // namespace mxfp4moe
