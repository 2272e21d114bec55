// Grouped expert GEMMs over packed MXFP4 weights with fused epilogues, and
// the routing-weighted combine.
//
// The MoE expert FFN of gpt-oss ("feat(gguf): serve gpt-oss gguf checkpoints
// on gpt_oss", FreeToken PR #838, "What it does"; numerical review of
// "expert offloading Phase 2", MoE-Infinity PR #152):
//   gate_up: h = x W13_e^T + b13_e, a = clamped SwiGLU(h[0::2], h[1::2])
//   down:    z = a W2_e^T + b2_e, weighted by the routing weight of the pair
//   combine: y_t = sum_j w_tj z_(t,j)
//
// Each GEMM computes C[n, m] = sum_k W[n, k] X[m, k] with n = weight rows
// (output features) and m = the tokens of one expert.  Weights are the MFMA A
// operand, tokens the B operand, so the output layout of
// v_mfma_f32_32x32x16_bf16 gives every lane four consecutive output features
// of one token: a gate/up pair sits in one lane (SwiGLU without shuffles) and
// the down outputs leave as 16-byte stores.
//
// In the full-tile kernels K runs in chunks of 64 = two E8M0 groups.  Within
// a chunk lane half h (lane / 32) takes group h: it reads that group's 16
// packed bytes of its weight row (staged in LDS with the chunk) with one
// 128-bit read and converts dword s (eight codes) to the eight bf16 it feeds
// to MFMA step s; the tokens' bf16 rows of the chunk are staged beside them
// and each lane reads the eight values matching its weight codes.  (The mid
// and streaming kernels use the 16x16x32 MFMA with a lane layout of their
// own, described with them.)  Any consistent assignment of k to (lane half,
// step, element) yields the same dot products, and this one needs no
// reshuffle of the checkpoint layout.  Weights are dequantized exactly
// (E2M1 x 2^(s-127) is a bf16 value) and MFMA accumulates in fp32.
#include "internal.h"
#include "mx_device.h"

namespace {

using mx::bf16x8;
using mx::f32x16;
using mx::f32x4;
using mx::u32x4;

// Staged token chunks are [BM][8] slots of 16 bytes with an XOR swizzle of the
// slot column, so the 128-bit LDS reads of 8 (or 16) consecutive token rows at
// one logical column hit distinct banks.  The swizzle depends only on the row
// within its 32-row block, so a lane's addresses for different 32-row blocks
// and ring stages differ by constants.
__device__ __forceinline__ int slot_col(int row, int part) {
  const int r = row & 31;  // depends only on the row within its 32-row block
  return part ^ ((r ^ (r >> 3)) & 7);
}

__device__ __forceinline__ float swiglu_clamped(float gate, float up) {
  // gpt-oss family constants: alpha 1.702, limit 7; gate clamped from above,
  // up clamped on both sides, +1 after the clamp.
  const float g = fminf(gate, 7.0f);
  const float u = fminf(fmaxf(up, -7.0f), 7.0f);
  // sigmoid through the hardware reciprocal (about 1 ulp; the result is
  // rounded to bf16)
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * g)) * (u + 1.0f);
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
// Biases of logical rows n..n+3 (n a multiple of 4, below N).
__device__ __forceinline__ f32x4 load_bias4(const uint16_t* bias, int n, int N, bool split) {
  uint32_t lo, hi;
  if (split) {  // gate n/2, up n/2, gate n/2+1, up n/2+1
    const uint32_t g = *reinterpret_cast<const uint32_t*>(bias + (n >> 1));
    const uint32_t u = *reinterpret_cast<const uint32_t*>(bias + (N >> 1) + (n >> 1));
    lo = (g & 0xffffu) | (u << 16);
    hi = (g >> 16) | (u & 0xffff0000u);
  } else {
    const uint2 b = *reinterpret_cast<const uint2*>(bias + n);
    lo = b.x;
    hi = b.y;
  }
  return f32x4{mx::bf16_to_f32(lo & 0xffffu), mx::bf16_to_f32(lo >> 16), mx::bf16_to_f32(hi & 0xffffu),
               mx::bf16_to_f32(hi >> 16)};
}

// Scale operands of the 32 codes a lane converts at once (one 16-byte piece).
// MXFP4: one E8M0 byte for all 32.  NVFP4: two E4M3 block scales, the first
// for the codes of steps 0 and 1, the second for steps 2 and 3; the result is
// exact in bf16 (a code has at most 2 significant bits, an E4M3 value 4).
template <bool kNv>
struct GroupScale {
  float lo, hi;
  __device__ __forceinline__ GroupScale(const uint8_t* srow, int g) {
    if (kNv) {
      lo = mx::e4m3_operand(srow[2 * g]);
      hi = mx::e4m3_operand(srow[2 * g + 1]);
    } else {
      lo = hi = mx::e8m0_operand(srow[g]);
    }
  }
  // from the group's scale byte(s) already read (b1 only for NVFP4)
  __device__ __forceinline__ GroupScale(uint32_t b0, uint32_t b1) {
    if (kNv) {
      lo = mx::e4m3_operand(b0);
      hi = mx::e4m3_operand(b1);
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

// Block -> (tile, weight-row tile).  Blocks are dealt to the 8 XCDs round
// robin (block b runs on XCD b % 8), so the id is first remapped so that each
// XCD owns a contiguous range of the work, then walked in groups of kGroup
// token tiles with the token tile fastest: blocks running together on one XCD
// share the weight rows of one expert (and the staged tokens of a few tiles)
// through that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroup = 4;

__device__ __forceinline__ bool map_block(int num_tiles, int n_tiles, int& tile, int& ntile) {
  const int b = blockIdx.x;
  const int total = num_tiles * n_tiles;
  const int per = (total + kXcds - 1) / kXcds;
  const int local = b / kXcds;
  if (local >= per) return false;
  const int pid = (b % kXcds) * per + local;
  if (pid >= total) return false;
  const int gsz = kGroup * n_tiles;
  const int g = pid / gsz;
  const int rem = pid - g * gsz;
  const int gm = min(kGroup, num_tiles - g * kGroup);
  tile = g * kGroup + rem % gm;
  ntile = rem / gm;
  return true;
}

// One 64-wide K chunk of MFMA work for a wave from operands in registers:
// for each of the four K steps, RN x RM MFMAs over the token fragments b
// (step s, token block cb).  The converts producing step s+1's weight
// fragments, written to the other half of a double buffer, are interleaved
// with step s's MFMAs so the matrix core does not wait for a burst of
// conversions.
struct NoExtra {
  __device__ void operator()(int) const {}
};

// `extra(k)` runs right after the k-th MFMA of the chunk (k = 0 .. 4*RN*RM-1),
// so a caller can spread other instructions between the MFMAs.
template <int RN, int RM, typename Extra = NoExtra>
__device__ __forceinline__ void chunk_mma_regs(f32x16 (&acc)[RN][RM], const bf16x8 (&b)[4][RM],
                                               const u32x4 (&w)[RN], const float (&sc)[RN],
                                               Extra extra = Extra()) {
  u32x4 a[2][RN];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) a[0][rb] = mx::fp4x8_to_bf16x8(w[rb][0], sc[rb]);
  auto convert = [&](int s, int i) {  // converts pair i%4 of fragment i/4 for step s
    const int rb = i / 4, sel = i % 4;
    const uint32_t packed = w[rb][s];
    uint32_t v;
    if (sel == 0) v = mx::fp4x2_to_bf16x2<0>(packed, sc[rb]);
    else if (sel == 1) v = mx::fp4x2_to_bf16x2<1>(packed, sc[rb]);
    else if (sel == 2) v = mx::fp4x2_to_bf16x2<2>(packed, sc[rb]);
    else v = mx::fp4x2_to_bf16x2<3>(packed, sc[rb]);
    a[s & 1][rb][sel] = v;
  };
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < RN * RM; ++i) {
      const int rb = i % RN, cb = i / RN;
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mx::as_bf16x8(a[s & 1][rb]), b[s][cb], acc[rb][cb], 0, 0, 0);
      if (s + 1 < 4 && i < 4 * RN) convert(s + 1, i);
      extra(s * RN * RM + i);
    }
    if (s + 1 < 4) {
#pragma unroll
      for (int i = RN * RM; i < 4 * RN; ++i) convert(s + 1, i);
    }
  }
}

// The token fragments of one chunk from a staged token slab xb (RM blocks of
// 32 rows, 128 bytes each): lane (r, h) takes row r of block cb, 16-byte slot
// 4h + s for step s.
template <int RM>
__device__ __forceinline__ void read_token_frags(bf16x8 (&b)[4][RM], const u32x4* __restrict__ xb, int lrow,
                                                 int half) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int cb = 0; cb < RM; ++cb) {
      const int row = cb * 32 + lrow;
      b[s][cb] = __builtin_bit_cast(bf16x8, xb[row * 8 + slot_col(row, half * 4 + s)]);
    }
  }
}

// Full tiles (the wide kernel): one wave per SIMD, each computing a
// (32*RN) x (32*RM) tile with its accumulators in registers; WN waves stack
// along the weight rows, so a block covers (32*RN*WN) weight rows x (32*RM)
// tokens and every staged token chunk feeds WN waves.  Per 64-wide K chunk a
// block moves BM*128 bytes of tokens and BN*32 bytes of packed weights from
// global memory.  The scale bytes of the block's weight rows are staged once.
constexpr int kWideMaxGroups = 128;  // K <= 4096
constexpr int kFp4StageBytes = (128 * 8 + 512 * 2) * 16 + 256 * 4;  // one LDS stage of the FP4 kernel
constexpr int kFp4MaxLds = 160 * 1024;                              // LDS per workgroup on gfx950

// 16 bytes per lane from global memory straight into LDS (the load unit
// writes lane l's bytes at lds + 16 * l; lds is the same for the whole wave).
__device__ __forceinline__ void load_lds16(const void* src, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Scale bytes of a block's BN weight rows, row-major as in memory: the rows
// are one contiguous, 32-byte aligned range (row counts and tile starts are
// multiples of 32), copied with 16-byte loads.  Rows past N are not copied
// (their outputs are dropped).  kDma: the load unit writes LDS itself
// (global_load_lds, lane l of a wave at the wave's slot + 16 * l), so the
// copy flies with the first operand loads instead of waiting to be stored;
// the caller waits for it (vmcnt) before the first barrier.
template <int BN, int kThreads, bool kDma = false>
__device__ __forceinline__ void stage_scales(uint8_t* sst, const mxfp4moe::GemmArgs& args, int e, int ntile,
                                             int kgroups, int t, bool split = false) {
  // kgroups: scale bytes per weight row (K/32 for MXFP4, K/16 for NVFP4)
  const int N = args.N;
  const int nv = min(BN, N - ntile * BN);
  u32x4* dst = reinterpret_cast<u32x4*>(sst);
  // the block's rows (split layout: its gate rows, then its up rows; each
  // range contiguous and 16-byte aligned)
  const int n16 = (nv * kgroups) >> 4;
  const int h = split ? ((nv >> 1) * kgroups) >> 4 : n16;
  const u32x4* g = reinterpret_cast<const u32x4*>(
      args.wscales + ((size_t)e * N + (split ? ntile * BN >> 1 : ntile * BN)) * (size_t)kgroups);
  const u32x4* u =
      reinterpret_cast<const u32x4*>(args.wscales + ((size_t)e * N + (N >> 1) + (ntile * BN >> 1)) * (size_t)kgroups);
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

// Epilogue, staged through an LDS region of RM*32*128 bytes per wave so
// that every token's outputs leave as full 128-byte rows: the lane layout of
// the MFMA results (four consecutive features of one token per lane) is
// written to LDS as [token][features] (16-byte chunks XOR-swizzled by token),
// then read back along the features and stored as whole rows.
// gate_up: bias, clamped SwiGLU, bf16 -> a[pair row][I] (16*RN activations,
// 32*RN bytes, per token per wave).  down: bias and routing weight in fp32,
// rounded to bf16 -> zw[pair][H], one 32-feature slab (staged as 128 bytes,
// stored as 64 per token) per pass.
template <int RN, int RM, bool kGateUp>
__device__ __forceinline__ void store_epilogue(const mxfp4moe::GemmArgs& args, const f32x16 (&acc)[RN][RM], int e,
                                              int row0, int count, int n_wave, int lane, uint8_t* region) {
  const int N = args.N;
  const int half = lane >> 5, lrow = lane & 31;
  const uint16_t* bias = args.bias + (size_t)e * N;
  auto chunk_addr = [](int m, int chunk) { return m * 128 + ((chunk ^ (m & 7)) << 4); };
  if (kGateUp) {
    // stage a[m][q_local], q_local = 0..16*RN-1 for this wave's 32*RN rows of w13
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = n_wave + rb * 32 + 8 * i + 4 * half;
        const f32x4 bv = load_bias4(bias, n < N ? n : N - 4, N, args.split_gate_up != 0);
        const float b0 = bv[0], b1 = bv[1], b2 = bv[2], b3 = bv[3];
        const int byte = rb * 32 + 8 * i + 4 * half;  // 2 * q_local
#pragma unroll
        for (int cb = 0; cb < RM; ++cb) {
          const int m = cb * 32 + lrow;
          const float a0 = swiglu_clamped(acc[rb][cb][4 * i + 0] + b0, acc[rb][cb][4 * i + 1] + b1);
          const float a1 = swiglu_clamped(acc[rb][cb][4 * i + 2] + b2, acc[rb][cb][4 * i + 3] + b3);
          *reinterpret_cast<uint32_t*>(region + chunk_addr(m, byte >> 4) + (byte & 15)) = mx::pack_bf16x2_rne(a0, a1);
        }
      }
    }
    const int I = N >> 1;
    const int q0 = n_wave >> 1;
    constexpr int kChunks = 2 * RN;  // 16-byte chunks of a per token (RN*16 activations)
#pragma unroll 4
    for (int j = 0; j < RM * 32 * kChunks / 64; ++j) {
      const int idx = j * 64 + lane;
      const int m = idx / kChunks, chunk = idx % kChunks;
      const int q = q0 + chunk * 8;
      if (m < count && q < I) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(region + chunk_addr(m, chunk));
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(args.out) + (size_t)(row0 + m) * I + q) = v;
      }
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      // stage zw[m][32 features of block rb]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = n_wave + rb * 32 + 8 * i + 4 * half;
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + (n < N ? n : N - 4));
        const float b0 = mx::bf16_to_f32(bb.x & 0xffffu), b1 = mx::bf16_to_f32(bb.x >> 16);
        const float b2 = mx::bf16_to_f32(bb.y & 0xffffu), b3 = mx::bf16_to_f32(bb.y >> 16);
#pragma unroll
        for (int cb = 0; cb < RM; ++cb) {
          const int m = cb * 32 + lrow;
          const float w = m < count ? args.topk_weights[args.sorted_pairs[row0 + m]] : 0.f;
          f32x4 v;
          v[0] = w * (acc[rb][cb][4 * i + 0] + b0);
          v[1] = w * (acc[rb][cb][4 * i + 1] + b1);
          v[2] = w * (acc[rb][cb][4 * i + 2] + b2);
          v[3] = w * (acc[rb][cb][4 * i + 3] + b3);
          *reinterpret_cast<f32x4*>(region + chunk_addr(m, 2 * i + half)) = v;
        }
      }
#pragma unroll 4
      for (int j = 0; j < RM * 32 * 8 / 64; ++j) {
        const int idx = j * 64 + lane;
        const int m = idx >> 3, chunk = idx & 7;
        const int n = n_wave + rb * 32 + chunk * 4;
        if (m < count && n < N) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(region + chunk_addr(m, chunk));
          const int p = args.sorted_pairs[row0 + m];
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(args.out) + (size_t)p * N + n) = pack_bf16x4(v);
        }
      }
    }
  }
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

// The wide kernel.  Operand chunks move from global memory to LDS by the
// load unit itself (global_load_lds_dwordx4: 16 bytes per lane, written at
// the wave's LDS address + 16 * lane; no staging registers, no LDS stores in
// the wave's stream), three LDS stages deep, and each wave reads its
// operands of chunk c+1 (weight groups, scale bytes, token fragments) from
// LDS into a second register set while chunk c runs on the matrix core.
// Per chunk c: wait for this wave's loads of chunk c+1 (those of chunk c+2
// stay in flight) and for its reads of chunk c, barrier (every wave's share
// of chunk c+1 is in LDS; every wave is done with chunk c's stage), then
// the 64 MFMAs of chunk c from registers, with the loads of chunk c+3 into
// chunk c's stage and the reads of chunk c+1 spread between them, one after
// every other MFMA.  Issued as a burst, 32 memory instructions would stall
// the wave (and leave the matrix core idle) until the LDS queue drains;
// spread out, they issue while earlier MFMAs run.  All waits sit at the
// barrier and cover work issued a whole chunk earlier.  While LDS-DMA loads
// are in flight the compiler only waits for all LDS reads at once, which
// this order makes free.
// kAhead = false: one operand set per wave, read right after the barrier
// that makes the chunk visible; meant for two waves per SIMD (WM = 2), where
// the other wave's MFMAs cover that wait.  Two chunks in flight.
template <int WN, int WM, int RN, int RM, bool kGateUp, bool kAhead = true>
__global__ __launch_bounds__(WN * WM * 64, 1) void expert_wide_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kThreads = WN * WM * 64;
  constexpr int BN = WN * RN * 32;
  constexpr int BM = WM * RM * 32;
  constexpr int kXSlots = BM * 8;
  constexpr int kWSlots = BN * 2;
  constexpr int kXPer = kXSlots / kThreads;
  constexpr int kWPer = kWSlots / kThreads;
  static_assert(kXSlots % kThreads == 0 && kWSlots % kThreads == 0, "tile / thread mismatch");
  constexpr int kStages = 3;              // LDS stages: chunk c+3 loads while c+1 is read and c runs
  constexpr int kLoads = kXPer + kWPer;  // loads per thread per chunk
  constexpr int kStage = kXSlots + kWSlots;  // 16-byte slots per stage
  constexpr int kArena = kStages * kStage * 16 + BN * kWideMaxGroups;
  static_assert(WN * WM * RM * 32 * 128 <= kArena, "epilogue regions fit in the arena");
  __shared__ __attribute__((aligned(16))) u32x4 arena[kArena / 16];
  uint8_t* const sst = reinterpret_cast<uint8_t*>(arena + kStages * kStage);

  const int N = args.N, K = args.K;
  const int n_tiles = (N + BN - 1) / BN;
  int tile, ntile;
  if (!map_block(*args.num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
  const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  const int e = __builtin_amdgcn_readfirstlane(tl.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tl.y);
  const int count = __builtin_amdgcn_readfirstlane(tl.z);
  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 1) >> 1;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int lane = t & 63;
  const int half = lane >> 5;
  const int lrow = lane & 31;

  const bool split = kGateUp && args.split_gate_up;  // uniform
  stage_scales<BN, kThreads, true>(sst, args, e, ntile, kgroups, t, split);

  // token slot p = t + i*threads -> row p/8, logical column slot_col(row, p%8);
  // rows past `count` re-read the tile's first row (their columns are never stored)
  const uint16_t* xsrc[kXPer];
  int xcol[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int p = t + i * kThreads;
    const int r = p >> 3;
    const int part = slot_col(r, p & 7);
    const int rr = r < count ? r : 0;
    const size_t src_row = kGateUp ? (size_t)(args.sorted_pairs[row0 + rr] / args.top_k) : (size_t)(row0 + rr);
    xsrc[i] = args.act + src_row * (size_t)K + part * 8;
    xcol[i] = part * 8;
  }
  // weight slot q = t + j*threads: row q/2 of the block, group 2c + (q&1) of chunk c
  const uint8_t* wsrc[kWPer];
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    int wr = ntile * BN + ((t + j * kThreads) >> 1);
    wr = w13_row(wr < N ? wr : N - 1, N, split);
    wsrc[j] = args.wblocks + ((size_t)e * N + wr) * (size_t)(K >> 1);
  }
  const int wh = t & 1;

  // chunk c (the last chunk again past the end) into stage st; lane l of the
  // wave lands in slot wave*64 + l (+ i*threads), as the register path stores it
  auto issue = [&](int c, int st) {
    c = c < nchunks ? c : nchunks - 1;
    u32x4* xs = arena + st * kStage + wave * 64;
    u32x4* ws = xs + kXSlots;
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      // K tail: the missing half chunk re-reads the first half (its weights are zero)
      const int koff = (c * 64 + xcol[i] < K) ? c * 64 : c * 64 - 32;
      load_lds16(xsrc[i] + koff, xs + i * kThreads);
    }
    int g = 2 * c + wh;
    g = g < kgroups ? g : g - 1;
#pragma unroll
    for (int j = 0; j < kWPer; ++j) load_lds16(wsrc[j] + (size_t)g * 16, ws + j * kThreads);
  };

  const int wslot0 = (wn * RN * 32 + lrow) * 2 + half;
  const uint8_t* srow = sst + staged_row(wn * RN * 32 + lrow, min(BN, N - ntile * BN), split) * kgroups;
  const int n_wave = ntile * BN + wn * RN * 32;
  const int m_wave = wm * RM * 32;
  const bool live = WM == 1 || m_wave < count;  // wave-uniform; a tile holds at least one pair
  const int rb_stride = (split ? 16 : 32) * kgroups;

  f32x16 acc[RN][RM];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int cb = 0; cb < RM; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  // the operands of one chunk in registers, as read (nothing computed from
  // them until the chunk runs, a chunk later)
  struct Ops {
    u32x4 w[RN];
    uint32_t sb[RN];  // E8M0 scale bytes
    bf16x8 b[4][RM];
  };
  auto read_ops = [&](Ops& o, int c, int st) {
    c = c < nchunks ? c : nchunks - 1;  // past the end: a harmless re-read
    const u32x4* xs = arena + st * kStage;
    const u32x4* wsm = xs + kXSlots;
    const int g = 2 * c + half;
    const int gg = g < kgroups ? g : g - 1;
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      o.w[rb] = wsm[wslot0 + rb * 64];
      o.sb[rb] = srow[rb * rb_stride + gg];
    }
    read_token_frags<RM>(o.b, xs + m_wave * 8, lrow, half);
  };
  // load k (0 .. kLoads-1) of chunk c into stage st
  auto issue_one = [&](int c, int st, int k) {
    c = c < nchunks ? c : nchunks - 1;
    u32x4* xs = arena + st * kStage + wave * 64;
    if (k < kXPer) {
      const int koff = (c * 64 + xcol[k] < K) ? c * 64 : c * 64 - 32;
      load_lds16(xsrc[k] + koff, xs + k * kThreads);
    } else {
      int g = 2 * c + wh;
      g = g < kgroups ? g : g - 1;
      load_lds16(wsrc[k - kXPer] + (size_t)g * 16, xs + kXSlots + (k - kXPer) * kThreads);
    }
  };
  // LDS read j of chunk c's operands (weights, scale bytes, token fragments) from stage st
  constexpr int kReads = 2 * RN + 4 * RM;
  auto read_one = [&](Ops& o, int c, int st, int j) {
    c = c < nchunks ? c : nchunks - 1;
    const u32x4* xs = arena + st * kStage;
    const int g = 2 * c + half;
    const int gg = g < kgroups ? g : g - 1;
    if (j < RN) {
      o.w[j] = xs[kXSlots + wslot0 + j * 64];
    } else if (j < 2 * RN) {
      o.sb[j - RN] = srow[(j - RN) * rb_stride + gg];
    } else {
      const int s = (j - 2 * RN) / RM, cb = (j - 2 * RN) % RM;
      const int row = cb * 32 + lrow;
      o.b[s][cb] = __builtin_bit_cast(bf16x8, xs[m_wave * 8 + row * 8 + slot_col(row, half * 4 + s)]);
    }
  };
  // chunk c from registers `cur` (stage st = c % kStages, a constant at every
  // call site); chunk c+1's operands into `nxt`; chunk c+kStages into
  // chunk c's stage.  The loads and reads are spread through the chunk's
  // MFMAs, one after every other MFMA, so the wave never stalls on a burst of
  // memory instructions while the matrix core idles.
  auto step = [&](int c, int st, const Ops& cur, Ops& nxt) {
    // this wave's loads of chunk c+1 are done once at most the loads of the
    // chunks after it are in flight
    wait_loads_then_barrier<(kStages - 2) * kLoads>();
    if (live) {
      static_assert(!kAhead || 2 * (kLoads + kReads) <= 4 * RN * RM, "room between the MFMAs");
      auto extra = [&](int k) {
        if (k % 2 != 0) return;
        const int op = k / 2;
        if (op < kLoads) issue_one(c + kStages, st, op);
        else if (op < kLoads + kReads) read_one(nxt, c + 1, (st + 1) % kStages, op - kLoads);
        else return;
        __builtin_amdgcn_sched_barrier(0);  // keep the order: the compiler would bunch the MFMAs
      };
      // K tail: the group past K multiplies zero weights
      const bool glive = 2 * c + half < kgroups;
      u32x4 w[RN];
      float sc[RN];
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
        w[rb] = glive ? cur.w[rb] : u32x4{0u, 0u, 0u, 0u};
        sc[rb] = mx::e8m0_operand(cur.sb[rb]);
      }
      chunk_mma_regs<RN, RM>(acc, cur.b, w, sc, extra);
    } else {
      issue(c + kStages, st);
    }
  };
  if constexpr (kAhead) {
    Ops ops0, ops1;
  #pragma unroll
    for (int c = 0; c < kStages; ++c) issue(c, c);
    wait_loads_then_barrier<(kStages - 1) * kLoads>();  // chunk 0 (and the scale table) landed
    if (live) read_ops(ops0, 0, 0);
    // trips of 2*kStages chunks: the register set and the stage of every step
    // are constants; then the remaining steps one by one
    constexpr int kTrip = 2 * kStages;
    const int nfull = nchunks / kTrip * kTrip;
    for (int c0 = 0; c0 < nfull; c0 += kTrip) {
  #pragma unroll
      for (int u = 0; u < kTrip; u += 2) {
        step(c0 + u, u % kStages, ops0, ops1);
        step(c0 + u + 1, (u + 1) % kStages, ops1, ops0);
      }
    }
  #pragma unroll
    for (int u = 0; u < kTrip - 1; u += 2) {
      if (nfull + u < nchunks) step(nfull + u, u % kStages, ops0, ops1);
      if (nfull + u + 1 < nchunks) step(nfull + u + 1, (u + 1) % kStages, ops1, ops0);
    }
  } else {
    // one operand set: chunk c is read after the barrier that makes it
    // visible (the other wave on the SIMD covers the wait), chunk c+2 goes
    // to the stage of chunk c-1, its loads spread between the MFMAs
    auto step1 = [&](int c, int st) {
      wait_loads_then_barrier<kLoads>();  // chunk c landed; chunk c+1 may be in flight
      Ops cur;
      if (live) {
#pragma unroll
        for (int j = 0; j < kReads; ++j) read_one(cur, c, st, j);
        constexpr int kMfma = 4 * RN * RM;
        constexpr int kEvery = kMfma / kLoads >= 2 ? 2 : 1;
        static_assert(kEvery * kLoads <= kMfma, "room between the MFMAs");
        auto extra = [&](int k) {
          if (k % kEvery != 0 || k / kEvery >= kLoads) return;
          issue_one(c + 2, (st + 2) % kStages, k / kEvery);
          __builtin_amdgcn_sched_barrier(0);
        };
        const bool glive = 2 * c + half < kgroups;
        u32x4 w[RN];
        float sc[RN];
#pragma unroll
        for (int rb = 0; rb < RN; ++rb) {
          w[rb] = glive ? cur.w[rb] : u32x4{0u, 0u, 0u, 0u};
          sc[rb] = mx::e8m0_operand(cur.sb[rb]);
        }
        chunk_mma_regs<RN, RM>(acc, cur.b, w, sc, extra);
      } else {
        issue(c + 2, (st + 2) % kStages);
      }
    };
    issue(0, 0);
    issue(1, 1);
    const int nfull = nchunks / kStages * kStages;
    for (int c0 = 0; c0 < nfull; c0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) step1(c0 + u, u);
    }
    if (nfull < nchunks) step1(nfull, 0);
    if (nfull + 1 < nchunks) step1(nfull + 1, 1);
  }
  // the chunks issued past the end land before the arena is reused
  wait_loads_then_barrier<0>();
  uint8_t* region = reinterpret_cast<uint8_t*>(arena) + wave * (RM * 32 * 128);
  if (live) store_epilogue<RN, RM, kGateUp>(args, acc, e, row0 + m_wave, count - m_wave, n_wave, lane, region);
}

template <int WN, int WM, int RN, int RM, bool kGateUp, bool kAhead = true>
hipError_t launch_wide(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  constexpr int BN = WN * RN * 32;
  const long n_tiles = (a.N + BN - 1) / BN;
  const long blocks = n_tiles * a.max_tiles;
  if (blocks == 0) return hipSuccess;
  const long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  expert_wide_kernel<WN, WM, RN, RM, kGateUp, kAhead><<<(unsigned)grid, WN * WM * 64, 0, stream>>>(a);
  return hipGetLastError();
}

// 4 bytes per lane from global memory straight into LDS (lane l's word at lds + 4 * l).
__device__ __forceinline__ void load_lds4(const void* src, uint32_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// FP4 scaled-MFMA variant of the wide kernel (opt-in): the same 512-row x
// 128-token tiles, staging, read-ahead and epilogue, with
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplying the packed E2M1 weights,
// scaled by their E8M0 bytes, with the tokens as MXFP8 E4M3 codes scaled by
// their own block bytes (the quantizer's chunk-interleaved rows; kSplit adds a
// second MFMA for the residual codes).  No weight is converted: the
// checkpoint's 16-byte group is the A operand.  Operand layouts of the
// 32x32x64 instruction (measured on gfx950): A lane (r, h) holds row r, K
// [32h, 32h + 32) of the chunk as 32 nibbles, low nibble first, with its
// scale byte; B lane (n, h) holds token n, K [16h, 16h + 16) in bytes 0..15
// and K [32 + 16h, 48 + 16h) in bytes 16..31, with the scale of group h; D as
// the bf16 32x32 MFMA.
// A stage holds the chunk's token codes, weight groups and the tokens' four
// scale bytes (one word per token).  kStages
// LDS stages (dynamic LDS: three when they and the scale table fit, else two);
// two memory instructions follow each MFMA (the MFMAs are twice as long as
// the bf16 ones and there are no conversions).
template <bool kGateUp, bool kSplit, int kStages>
__global__ __launch_bounds__(256, 1) void expert_fp4_kernel(mxfp4moe::GemmArgs args) {
  constexpr int WN = 4, RN = 4, RM = 4;
  constexpr int kThreads = 256;
  constexpr int BN = WN * RN * 32;
  constexpr int BM = RM * 32;
  constexpr int kXSlots = BM * 8;  // 16-byte token slots per chunk (64 high + 64 residual codes per token)
  constexpr int kWSlots = BN * 2;  // 16-byte weight slots per chunk
  constexpr int kXPer = kXSlots / kThreads;
  constexpr int kWPer = kWSlots / kThreads;
  constexpr int kLoads = kXPer + kWPer + 1;      // per thread per chunk: token slots, weight slots, a scale word
  constexpr int kStageBytes = (kXSlots + kWSlots) * 16 + kThreads * 4;
  static_assert(kStageBytes % 16 == 0 && kThreads % BM == 0, "stage layout");
  static_assert(kStages * kStageBytes >= 4 * RM * 32 * 128, "epilogue regions fit in the stages");
  extern __shared__ __attribute__((aligned(16))) u32x4 fp4_arena[];
  uint8_t* const base = reinterpret_cast<uint8_t*>(fp4_arena);
  uint8_t* const sst = base + kStages * kStageBytes;
  auto xs_of = [&](int st) { return reinterpret_cast<u32x4*>(base + st * kStageBytes); };
  auto xsc_of = [&](int st) { return reinterpret_cast<uint32_t*>(base + st * kStageBytes + (kXSlots + kWSlots) * 16); };

  const int N = args.N, K = args.K;
  const int n_tiles = (N + BN - 1) / BN;
  int tile, ntile;
  if (!map_block(*args.num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
  const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  const int e = __builtin_amdgcn_readfirstlane(tl.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tl.y);
  const int count = __builtin_amdgcn_readfirstlane(tl.z);
  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 1) >> 1;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int half = lane >> 5;
  const int lrow = lane & 31;

  const bool split = kGateUp && args.split_gate_up;  // uniform
  stage_scales<BN, kThreads, true>(sst, args, e, ntile, kgroups, t, split);

  // token slot p = t + i*threads -> row p/8, logical column slot_col(row, p%8);
  // rows past `count` re-read the tile's first row (their columns are never stored)
  const size_t qrow = (size_t)128 * nchunks;  // code bytes per quantized row
  const uint8_t* const q = reinterpret_cast<const uint8_t*>(args.act);
  const uint8_t* xsrc[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int p = t + i * kThreads;
    const int r = p >> 3;
    const int rr = r < count ? r : 0;
    const size_t src_row = kGateUp ? (size_t)(args.sorted_pairs[row0 + rr] / args.top_k) : (size_t)(row0 + rr);
    xsrc[i] = q + src_row * qrow + slot_col(r, p & 7) * 16;
  }
  // the 4 scale bytes of token t % BM per chunk (threads past BM load copies,
  // into words nobody reads, so every wave issues the same loads)
  const int st_rr = (t & (BM - 1)) < count ? (t & (BM - 1)) : 0;
  const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(args.act_scales) +
                         (kGateUp ? (size_t)(args.sorted_pairs[row0 + st_rr] / args.top_k) : (size_t)(row0 + st_rr)) *
                             nchunks;
  const uint8_t* wsrc[kWPer];
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    int wr = ntile * BN + ((t + j * kThreads) >> 1);
    wr = w13_row(wr < N ? wr : N - 1, N, split);
    wsrc[j] = args.wblocks + ((size_t)e * N + wr) * (size_t)(K >> 1);
  }
  const int wh = t & 1;

  // load o of chunk c into stage st: o = 0 the scale word, 1..kXPer token
  // slots, then the weight slots; lane l of the wave lands in slot
  // wave*64 + l (+ i*threads)
  constexpr int kLoadOps = kLoads;
  auto issue_one = [&](int c, int st, int o) {
    c = c < nchunks ? c : nchunks - 1;  // past the end: the last chunk again
    u32x4* xs = xs_of(st) + wave * 64;
    if (o == 0) {
      load_lds4(ssrc + c, xsc_of(st) + wave * 64);
    } else if (o <= kXPer) {
      load_lds16(xsrc[o - 1] + (size_t)c * 128, xs + (o - 1) * kThreads);
    } else {
      int g = 2 * c + wh;
      g = g < kgroups ? g : g - 1;
      load_lds16(wsrc[o - 1 - kXPer] + (size_t)g * 16, xs + kXSlots + (o - 1 - kXPer) * kThreads);
    }
  };
  auto issue = [&](int c, int st) {
#pragma unroll
    for (int o = 0; o < kLoadOps; ++o) issue_one(c, st, o);
  };

  const int n_wave = ntile * BN + wave * RN * 32;
  const int wslot0 = (wave * RN * 32 + lrow) * 2 + half;
  const uint8_t* srow = sst + staged_row(wave * RN * 32 + lrow, min(BN, N - ntile * BN), split) * kgroups;
  const int rb_stride = (split ? 16 : 32) * kgroups;

  f32x16 acc[RN][RM];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int cb = 0; cb < RM; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  // the operands of one chunk in registers, as read
  constexpr int kHalves = kSplit ? 2 : 1;  // high codes, and the residual's
  struct Ops {
    u32x4 w[RN];
    uint32_t sa[RN];               // weight E8M0 bytes
    uint32_t sw[RM];               // token scale words
    mx::i32x8 x[RM][kHalves];      // token code fragments, as the MFMA's B operand
  };
  constexpr int kPerBlock = 1 + 2 * kHalves;  // reads per token block: scale word, code fragments
  constexpr int kReads = 2 * RN + RM * kPerBlock;
  // LDS read j of chunk c's operands from stage st
  auto read_one = [&](Ops& o, int c, int st, int j) {
    c = c < nchunks ? c : nchunks - 1;
    const u32x4* xs = xs_of(st);
    const int g = 2 * c + half;
    const int gg = g < kgroups ? g : g - 1;
    if (j < RN) {
      o.w[j] = xs[kXSlots + wslot0 + j * 64];
    } else if (j < 2 * RN) {
      o.sa[j - RN] = srow[(j - RN) * rb_stride + gg];
    } else {
      const int cb = (j - 2 * RN) / kPerBlock, k = (j - 2 * RN) % kPerBlock;
      const int row = cb * 32 + lrow;
      if (k == 0) {
        o.sw[cb] = xsc_of(st)[row];
      } else {
        const int hh = (k - 1) / 2, f = (k - 1) % 2;  // code half (high / residual), fragment
        const u32x4 v = xs[row * 8 + slot_col(row, 4 * hh + 2 * f + half)];
#pragma unroll
        for (int i = 0; i < 4; ++i) o.x[cb][hh][4 * f + i] = (int)v[i];
      }
    }
  };
  auto read_ops = [&](Ops& o, int c, int st) {
#pragma unroll
    for (int j = 0; j < kReads; ++j) read_one(o, c, st, j);
  };
  constexpr int kMfma = RN * RM * kHalves;
  static_assert(2 * kMfma >= kLoadOps + kReads, "room between the MFMAs");
  // chunk c from registers `cur` (stage st = c % kStages, a constant at every
  // call site); chunk c+1's operands into `nxt`; chunk c+kStages into chunk
  // c's stage; two memory instructions after each MFMA
  auto step = [&](int c, int st, const Ops& cur, Ops& nxt) {
    wait_loads_then_barrier<(kStages - 2) * kLoads>();
    auto extra = [&](int o) {
      if (o < kLoadOps) issue_one(c + kStages, st, o);
      else if (o < kLoadOps + kReads) read_one(nxt, c + 1, (st + 1) % kStages, o - kLoadOps);
      else return;
      __builtin_amdgcn_sched_barrier(0);  // keep the order: the compiler would bunch the MFMAs
    };
    const bool glive = 2 * c + half < kgroups;  // K tail: the group past K multiplies zero weights
    mx::i32x8 a[RN];
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      const u32x4 w = glive ? cur.w[rb] : u32x4{0u, 0u, 0u, 0u};
      a[rb] = mx::i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
    }
    int k = 0;
#pragma unroll
    for (int cb = 0; cb < RM; ++cb) {
#pragma unroll
      for (int hh = 0; hh < kHalves; ++hh) {
        const mx::i32x8 bx = cur.x[cb][hh];
        const int sb = (int)((cur.sw[cb] >> (16 * hh + 8 * half)) & 255u);
#pragma unroll
        for (int rb = 0; rb < RN; ++rb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[rb], bx, acc[rb][cb], 4, 0, 0,
                                                                        (int)cur.sa[rb], 0, sb);
          extra(2 * k);
          extra(2 * k + 1);
          ++k;
        }
      }
    }
  };
  Ops ops0, ops1;
#pragma unroll
  for (int c = 0; c < kStages; ++c) issue(c, c);
  wait_loads_then_barrier<(kStages - 1) * kLoads>();  // chunk 0 (and the scale table) landed
  read_ops(ops0, 0, 0);
  constexpr int kTrip = 2 * kStages;
  const int nfull = nchunks / kTrip * kTrip;
  for (int c0 = 0; c0 < nfull; c0 += kTrip) {
#pragma unroll
    for (int u = 0; u < kTrip; u += 2) {
      step(c0 + u, u % kStages, ops0, ops1);
      step(c0 + u + 1, (u + 1) % kStages, ops1, ops0);
    }
  }
#pragma unroll
  for (int u = 0; u < kTrip - 1; u += 2) {
    if (nfull + u < nchunks) step(nfull + u, u % kStages, ops0, ops1);
    if (nfull + u + 1 < nchunks) step(nfull + u + 1, (u + 1) % kStages, ops1, ops0);
  }
  // the chunks issued past the end land before the stages are reused
  wait_loads_then_barrier<0>();
  uint8_t* region = base + wave * (RM * 32 * 128);
  store_epilogue<RN, RM, kGateUp>(args, acc, e, row0, count, n_wave, lane, region);
}

template <bool kGateUp, bool kSplit, int kStages>
hipError_t launch_fp4_cfg(const mxfp4moe::GemmArgs& a, unsigned grid, size_t lds, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&expert_fp4_kernel<kGateUp, kSplit, kStages>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kFp4MaxLds);
  if (attr != hipSuccess) return attr;
  expert_fp4_kernel<kGateUp, kSplit, kStages><<<grid, 256, lds, stream>>>(a);
  return hipGetLastError();
}

template <bool kGateUp>
hipError_t launch_fp4(const mxfp4moe::GemmArgs& a, bool split_act, hipStream_t stream) {
  constexpr int BN = 512;
  const long n_tiles = (a.N + BN - 1) / BN;
  const long blocks = n_tiles * a.max_tiles;
  if (blocks == 0) return hipSuccess;
  const unsigned grid = (unsigned)((blocks + kXcds - 1) / kXcds * kXcds);
  const size_t table = (size_t)BN * (a.K >> 5);
  // three stages when they fit, except for the split down GEMM, whose
  // three-stage build runs out of registers (reloads from scratch in the
  // loop; measured 312 against 293 us at the 120b prefill shape)
  const bool three = 3 * kFp4StageBytes + table <= (size_t)kFp4MaxLds && (kGateUp || !split_act);
  const size_t lds = (three ? 3 : 2) * kFp4StageBytes + table;
  if (split_act)
    return three ? launch_fp4_cfg<kGateUp, true, 3>(a, grid, lds, stream)
                 : launch_fp4_cfg<kGateUp, true, 2>(a, grid, lds, stream);
  return three ? launch_fp4_cfg<kGateUp, false, 3>(a, grid, lds, stream)
               : launch_fp4_cfg<kGateUp, false, 2>(a, grid, lds, stream);
}

// Streaming kernel for tiles of at most kStreamTokens pairs: decode batches
// and the smallest per-expert remainders of prefill.  It runs on the 16x16x32
// bf16 MFMA, whose A operand gives lane l row l%16 and the eight K values of
// quarter q = l/16: so lane (r, q) can take one whole E8M0 group (16 bytes,
// 32 codes, four MFMA steps) and the four lanes of a row read 64 contiguous
// bytes of it per load instruction, the pattern that lets HBM stream at full
// rate (a 32-byte piece per row per instruction does not).  Chunk j holds K
// [128j, 128j+128): lane (r, q) supplies group 4j+q, and step s uses its codes
// [8s, 8s+8), i.e. K = 128j + 32q + 8s + i; the B operand (token l%16) holds
// the same K values of its token.  Sixteen token columns instead of 32 halve
// the MFMA work of a few-token tile.
//
// A block owns 64*RN weight rows of one expert; it copies the tile's token
// rows and the rows' scale bytes into LDS, then each wave streams its own
// 16*RN rows from global memory straight into registers, kBatch chunks per
// batch (every load of a batch issued before its first MFMA; the batches of
// the several waves per SIMD overlap).  Token columns past the tile's pairs
// read its first pair (their outputs are dropped).  Even and odd steps
// accumulate separately.  Outputs: lane (n, q) holds rows 4q..4q+3 of each
// 16-row block for token n, i.e. two gate/up pairs (gate_up) or four
// consecutive features (down), stored directly.
//
// With kKSplit = 2 the two waves of a row group take the two halves of K
// (the first half rounded up to whole batches) and the second wave's sums
// reach the first through LDS after a barrier, added in that fixed order:
// twice the blocks for a launch with few weight rows (the down GEMM of a
// decode batch), and half the serial batches per wave.
//
// Dynamic LDS: tokens [kStreamTokens][K] bf16 | scales [BN][K/32] |
// (kKSplit = 2) the second halves' sums [BN/16 row groups][RN][64 lanes] f32x4.
template <int RN, bool kNv = false, int kKSplit = 1>
__host__ __device__ constexpr size_t stream_lds_bytes(int K) {
  return (size_t)mxfp4moe::kStreamTokens * K * 2 + (size_t)(64 / kKSplit) * RN * (K / (kNv ? 16 : 32)) +
         (kKSplit == 2 ? (size_t)2 * RN * 64 * 16 : 0);
}

template <int RN, int kBatch, bool kGateUp, bool kNv, int kKSplit = 1>
__global__ __launch_bounds__(256, 5) void expert_stream_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kThreads = 256;
  constexpr int BN = 64 * RN / kKSplit;
  static_assert(kKSplit == 1 || kKSplit == 2, "one or two K parts");
  extern __shared__ u32x4 dyn[];
  uint8_t* const lds = reinterpret_cast<uint8_t*>(dyn);

  const int N = args.N, K = args.K;
  const int n_tiles = (N + BN - 1) / BN;
  int tile, ntile;
  if (!map_block(*args.num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
  const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  const int e = __builtin_amdgcn_readfirstlane(tl.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tl.y);
  const int count = __builtin_amdgcn_readfirstlane(tl.z);
  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 3) >> 2;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int q = lane >> 4;
  const int lr = lane & 15;
  const int rgrp = wave / kKSplit, kpart = wave % kKSplit;  // row group, K part
  // this wave's chunks [c_begin, c_end)
  const int half = min(nchunks, ((nchunks + 1) / 2 + kBatch - 1) / kBatch * kBatch);
  const int c_begin = kKSplit == 1 || kpart == 0 ? 0 : half;
  const int c_end = kKSplit == 1 || kpart == 1 ? nchunks : half;
  const bool has_work = c_begin < c_end;  // wave-uniform

  const bool split = kGateUp && args.split_gate_up;  // uniform
  const int n_wave = ntile * BN + rgrp * 16 * RN;
  const uint8_t* wrow[RN];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) {
    const int r = w13_row(min(n_wave + rb * 16 + lr, N - 1), N, split);  // rows past N: outputs dropped
    wrow[rb] = args.wblocks + ((size_t)e * N + r) * (size_t)(K >> 1);
  }
  // A group past the wave's last one (K tail, or a padding chunk of its last
  // batch) re-reads its last chunk's group, whose weights, scale and token
  // values are finite, and multiplies zero weights.
  auto load_batch = [&](int c0, u32x4 (&w)[kBatch][RN]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int g = min(4 * min(c0 + j, c_end - 1) + q, kgroups - 1);
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) w[j][rb] = *reinterpret_cast<const u32x4*>(wrow[rb] + (size_t)g * 16);
    }
  };
  // The first batch's weight loads go out before the staging below, so the
  // two round trips to memory overlap.
  u32x4 w_first[kBatch][RN];
  if (has_work) load_batch(c_begin, w_first);

  uint16_t* const xl = reinterpret_cast<uint16_t*>(lds);
  uint8_t* const sl = lds + (size_t)mxfp4moe::kStreamTokens * K * 2;
  {
    // token rows: at most 4 x K/8 <= 2048 pieces of 16 bytes, all loads issued
    // before the first store
    static_assert(mxfp4moe::kStreamTokens == 4 && mxfp4moe::kMaxHidden * 4 / 8 <= 8 * kThreads, "copy bounds");
    size_t xsrc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = r < count ? r : 0;
      xsrc[r] = (kGateUp ? (size_t)(args.sorted_pairs[row0 + rr] / args.top_k) : (size_t)(row0 + rr)) * (size_t)K;
    }
    const int k16 = K >> 3;
    const int nx16 = count * k16;
    u32x4 xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = min(t + j * kThreads, nx16 - 1);
      const int r = i / k16, p = i - r * k16;
      const size_t base = r == 0 ? xsrc[0] : r == 1 ? xsrc[1] : r == 2 ? xsrc[2] : xsrc[3];
      if (j * kThreads < nx16) xv[j] = reinterpret_cast<const u32x4*>(args.act + base)[p];
    }
    stage_scales<BN, kThreads>(sl, args, e, ntile, kNv ? 2 * kgroups : kgroups, t, split);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (t + j * kThreads < nx16) reinterpret_cast<u32x4*>(xl)[t + j * kThreads] = xv[j];
  }
  __syncthreads();

  const bool wave_live = n_wave < N && has_work;  // wave-uniform
  if (kKSplit == 1 && !wave_live) return;          // no barrier follows
  f32x4 acc[RN][2];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* srow[RN];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
    srow[rb] = sl + staged_row(rgrp * 16 * RN + rb * 16 + lr, min(BN, N - ntile * BN), split) * (kNv ? 2 : 1) *
                        kgroups;
  const uint16_t* xrow = xl + (lr < count ? lr : 0) * K;
  auto compute_batch = [&](int c0, const u32x4 (&w)[kBatch][RN]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int g0 = 4 * (c0 + j) + q;
      const bool glive = c0 + j < c_end && g0 < kgroups;
      const int g = min(4 * min(c0 + j, c_end - 1) + q, kgroups - 1);
      bf16x8 b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        b[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xrow + g * 32 + 8 * s));
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
        const GroupScale<kNv> sc(srow[rb], g);
        const u32x4 wj = glive ? w[j][rb] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = mx::as_bf16x8(sc.convert(wj[s], s));
          acc[rb][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[s], acc[rb][s & 1], 0, 0, 0);
        }
      }
    }
  };
  if (wave_live) {
    compute_batch(c_begin, w_first);
    for (int c0 = c_begin + kBatch; c0 < c_end; c0 += kBatch) {
      u32x4 w[kBatch][RN];
      load_batch(c0, w);
      // the whole batch in flight before its first use: left alone, the
      // scheduler sinks each load next to its MFMAs and only about two of a
      // wave's loads are ever outstanding
      __builtin_amdgcn_sched_barrier(0);
      compute_batch(c0, w);
    }
  }
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) acc[rb][0] = acc[rb][0] + acc[rb][1];  // (even + odd steps) of this K part
  if (kKSplit == 2) {
    f32x4* red = reinterpret_cast<f32x4*>(sl + (size_t)BN * (kNv ? 2 : 1) * kgroups);
    if (kpart == 1) {
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) red[(rgrp * RN + rb) * 64 + lane] = acc[rb][0];
    }
    __syncthreads();
    if (kpart == 1 || n_wave >= N) return;
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      acc[rb][0] = acc[rb][0] + red[(rgrp * RN + rb) * 64 + lane];  // first half, then second half
    }
  }

  if (lr >= count) return;
  const uint16_t* bias = args.bias + (size_t)e * N;
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) {
    const int n = n_wave + rb * 16 + 4 * q;  // first of this lane's four rows
    if (n >= N) continue;
    const f32x4 bv = load_bias4(bias, n, N, split);
    const float s2 = kNv ? args.scale2[e] : 1.0f;  // second-level scale, before the bias
    f32x4 v;
    v[0] = s2 * acc[rb][0][0] + bv[0];
    v[1] = s2 * acc[rb][0][1] + bv[1];
    v[2] = s2 * acc[rb][0][2] + bv[2];
    v[3] = s2 * acc[rb][0][3] + bv[3];
    if (kGateUp) {
      const int I = N >> 1;
      const uint32_t packed = mx::pack_bf16x2_rne(swiglu_clamped(v[0], v[1]), swiglu_clamped(v[2], v[3]));
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(args.out) + (size_t)(row0 + lr) * I + (n >> 1)) = packed;
    } else {
      const int p = args.sorted_pairs[row0 + lr];
      const float wt = args.topk_weights[p];
      v[0] *= wt;
      v[1] *= wt;
      v[2] *= wt;
      v[3] *= wt;
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(args.out) + (size_t)p * N + n) = pack_bf16x4(v);
    }
  }
}

#ifndef MX_STREAM_RN
#define MX_STREAM_RN 1
#endif
#ifndef MX_STREAM_BATCH
#define MX_STREAM_BATCH 6
#endif

#ifndef MX_STREAM_KSPLIT_UP
#define MX_STREAM_KSPLIT_UP 1
#endif
#ifndef MX_STREAM_KSPLIT_DOWN
#define MX_STREAM_KSPLIT_DOWN 2
#endif

template <bool kGateUp, bool kNv>
hipError_t launch_stream(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  constexpr int RN = MX_STREAM_RN;
  constexpr int kBatch = MX_STREAM_BATCH;
  constexpr int kKSplit = kGateUp ? MX_STREAM_KSPLIT_UP : MX_STREAM_KSPLIT_DOWN;
  constexpr int BN = 64 * RN / kKSplit;
  const long n_tiles = (a.N + BN - 1) / BN;
  const long blocks = n_tiles * a.max_tiles;
  if (blocks == 0) return hipSuccess;
  const long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  const size_t lds = stream_lds_bytes<RN, kNv, kKSplit>(a.K);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&expert_stream_kernel<RN, kBatch, kGateUp, kNv, kKSplit>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)stream_lds_bytes<RN, kNv, kKSplit>(mxfp4moe::kMaxHidden));
  if (attr != hipSuccess) return attr;
  expert_stream_kernel<RN, kBatch, kGateUp, kNv, kKSplit><<<(unsigned)grid, 256, lds, stream>>>(a);
  return hipGetLastError();
}

// Mid-size tiles (kStreamTokens < pairs <= kMidTokens): the per-expert
// remainders of prefill.  16x16x32 MFMA (A: lane (r, q) takes group 4c+q of
// row r, step s its codes [8s, 8s+8), so K = 128c + 32q + 8s + i; B: the same
// K values of token l%16).  A block owns 128 weight rows (four waves of
// 2 x 16 rows) and up to 64 tokens (four 16-token column blocks).  K runs in
// panels of kP chunks (128 K each); both operands of a panel are staged in
// LDS: the block's 128 weight rows as kP*64 contiguous bytes per row (eight
// lanes per row, 128 bytes per row per load: the pattern HBM streams at full
// rate) and the tile's token rows as kP*256 bytes each.  The loads of panel
// p+1 are issued before the MFMAs of panel p and stored after them (single
// LDS buffer, two barriers per panel); with panels of one chunk a block
// needs about 39 KB of LDS and 160 registers per lane at K = 2880, so three
// blocks share a CU and overlap further (panels of two chunks, two blocks
// per CU: 9 % slower at the 20b prefill shape, 17 % with NVFP4 weights).
// Token columns past the tile's pairs read its first pair (their outputs are
// dropped).
//
// Dynamic LDS: tokens [64][kP*256 + 16] | weights [128][kP*64 + 16] |
// scales [128][K/32]  (the 16-byte row pads make the 16-lane column reads
// conflict-free).
template <int kP, bool kNv = false>
__host__ __device__ constexpr size_t mid_lds_bytes(int K) {
  return (size_t)64 * (kP * 256 + 16) + (size_t)128 * (kP * 64 + 16) + (size_t)128 * (K / (kNv ? 16 : 32));
}

template <int kP, bool kGateUp, bool kNv>
__global__ __launch_bounds__(256, 2) void expert_mid_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kThreads = 256;
  constexpr int BN = 128;
  constexpr int kXRow = kP * 256 + 16;      // LDS bytes per token row of a panel
  constexpr int kWRow = kP * 64 + 16;       // LDS bytes per weight row of a panel
  constexpr int kXPieces = kP * 16;         // 16-byte pieces per token row of a panel
  constexpr int kWPieces = kP * 4;          // 16-byte pieces per weight row of a panel
  constexpr int kXPer = 64 * kXPieces / kThreads;
  constexpr int kWPer = BN * kWPieces / kThreads;
  static_assert(64 * kXPieces % kThreads == 0 && BN * kWPieces % kThreads == 0, "panel / thread mismatch");
  extern __shared__ u32x4 dyn[];
  uint8_t* const lds = reinterpret_cast<uint8_t*>(dyn);

  const int N = args.N, K = args.K;
  const int n_tiles = (N + BN - 1) / BN;
  int tile, ntile;
  if (!map_block(*args.num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
  const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  const int e = __builtin_amdgcn_readfirstlane(tl.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tl.y);
  const int count = __builtin_amdgcn_readfirstlane(tl.z);
  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 3) >> 2;
  const int npanels = (nchunks + kP - 1) / kP;
  const int k16 = K >> 3;   // 16-byte pieces of a token row
  const int kg16 = K >> 5;  // 16-byte pieces (groups) of a weight row
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int q = lane >> 4;
  const int lr = lane & 15;

  uint8_t* const xs = lds;
  uint8_t* const ws = lds + 64 * kXRow;
  uint8_t* const sl = ws + BN * kWRow;
  const bool split = kGateUp && args.split_gate_up;  // uniform
  stage_scales<BN, kThreads>(sl, args, e, ntile, kNv ? 2 * kgroups : kgroups, t, split);

  // load slots: token piece i = t + j*256 -> token i / kXPieces; weight piece
  // i = t + j*256 -> row i / kWPieces (rows past N re-read row N-1)
  const u32x4* xsrc[kXPer];
  int xpiece[kXPer], xdst[kXPer];
#pragma unroll
  for (int j = 0; j < kXPer; ++j) {
    const int i = t + j * kThreads;
    const int r = i / kXPieces;
    const int rr = r < count ? r : 0;
    const size_t src_row = kGateUp ? (size_t)(args.sorted_pairs[row0 + rr] / args.top_k) : (size_t)(row0 + rr);
    xsrc[j] = reinterpret_cast<const u32x4*>(args.act + src_row * (size_t)K);
    xpiece[j] = i - r * kXPieces;
    xdst[j] = r * kXRow + xpiece[j] * 16;
  }
  const u32x4* wsrc[kWPer];
  int wpiece[kWPer], wdst[kWPer];
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int i = t + j * kThreads;
    const int r = i / kWPieces;
    const int gr = w13_row(min(ntile * BN + r, N - 1), N, split);
    wsrc[j] = reinterpret_cast<const u32x4*>(args.wblocks + ((size_t)e * N + gr) * (size_t)(K >> 1));
    wpiece[j] = i - r * kWPieces;
    wdst[j] = r * kWRow + wpiece[j] * 16;
  }
  // Two register slots hold the next two panels in flight.  Groups / pieces
  // past the end re-read the last one (finite; the weights of a missing group
  // are zeroed at use); panels past the last re-read the last panel.
  u32x4 xv[2][kXPer], wv[2][kWPer];
  auto issue = [&](int p, int sl2) {
    p = min(p, npanels - 1);
#pragma unroll
    for (int j = 0; j < kWPer; ++j) wv[sl2][j] = wsrc[j][min(p * kWPieces + wpiece[j], kg16 - 1)];
#pragma unroll
    for (int j = 0; j < kXPer; ++j) xv[sl2][j] = xsrc[j][min(p * kXPieces + xpiece[j], k16 - 1)];
  };
  auto commit = [&](int sl2) {
#pragma unroll
    for (int j = 0; j < kWPer; ++j) *reinterpret_cast<u32x4*>(ws + wdst[j]) = wv[sl2][j];
#pragma unroll
    for (int j = 0; j < kXPer; ++j)
      if (t + j * kThreads < count * kXPieces) *reinterpret_cast<u32x4*>(xs + xdst[j]) = xv[sl2][j];
  };

  const int n_wave = ntile * BN + wave * 32;
  const uint8_t* srow[2];
  int wrd[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    srow[rb] = sl + staged_row(wave * 32 + rb * 16 + lr, min(BN, N - ntile * BN), split) * (kNv ? 2 : 1) * kgroups;
    wrd[rb] = (wave * 32 + rb * 16 + lr) * kWRow + 16 * q;
  }
  const int ncb = (count + 15) >> 4;  // live 16-token column blocks
  int xrd[4];  // LDS byte offset of this lane's token row for each column block
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int m = cb * 16 + lr;
    xrd[cb] = (m < count ? m : 0) * kXRow + 64 * q;
  }
  f32x4 acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  issue(1, 1);
  commit(0);
  __syncthreads();  // panel 0 and the scale rows staged
  issue(2, 0);
  // iteration p: panel p is in LDS, slot (p+1)&1 holds panel p+1 and slot p&1
  // panel p+2; after the MFMAs, panel p+1 goes to LDS and its slot is refilled
  // with panel p+3.  Unrolled by two so the slots are static.
  auto compute = [&](int p) {
#pragma unroll
    for (int jj = 0; jj < kP; ++jj) {
      const int g0 = 4 * (p * kP + jj) + q;
      const bool glive = g0 < kgroups;
      const int g = glive ? g0 : kgroups - 1;
      u32x4 a[2][4];  // [rb][step] converted A fragments
      // both row blocks' weight fragments and scale bytes read together
      u32x4 wr[2];
      uint32_t sb[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        wr[rb] = *reinterpret_cast<const u32x4*>(ws + wrd[rb] + jj * 64);
        sb[rb][0] = kNv ? srow[rb][2 * g] : srow[rb][g];
        sb[rb][1] = kNv ? srow[rb][2 * g + 1] : 0u;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const GroupScale<kNv> sc(sb[rb][0], sb[rb][1]);
        const u32x4 wj = glive ? wr[rb] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int st = 0; st < 4; ++st) a[rb][st] = sc.convert(wj[st], st);
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if (cb < ncb) {  // wave-uniform: column blocks past the tile's pairs are skipped
          // the block's four token fragments read together, then its MFMAs
          bf16x8 bb[4];
#pragma unroll
          for (int st = 0; st < 4; ++st)
            bb[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + xrd[cb] + jj * 256 + 16 * st));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const bf16x8 b = bb[st];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mx::as_bf16x8(a[rb][st]), b, acc[rb][cb], 0, 0, 0);
          }
        }
      }
    }
  };
  for (int p = 0; p < npanels; p += 2) {
    compute(p);
    __syncthreads();  // every wave is done with panel p
    if (p + 1 >= npanels) break;  // uniform
    commit(1);
    __syncthreads();  // panel p+1 staged
    issue(p + 3, 1);
    compute(p + 1);
    __syncthreads();
    if (p + 2 >= npanels) break;
    commit(0);
    __syncthreads();  // panel p+2 staged
    issue(p + 4, 0);
  }

  if (n_wave >= N) return;
  const uint16_t* bias = args.bias + (size_t)e * N;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int n = n_wave + rb * 16 + 4 * q;  // first of this lane's four rows
    if (n >= N) continue;
    const f32x4 bv = load_bias4(bias, n, N, split);
    const float b0 = bv[0], b1 = bv[1], b2 = bv[2], b3 = bv[3];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int m = cb * 16 + lr;
      if (m >= count) continue;
      const float s2 = kNv ? args.scale2[e] : 1.0f;  // second-level scale, before the bias
      const f32x4 v = f32x4{s2 * acc[rb][cb][0], s2 * acc[rb][cb][1], s2 * acc[rb][cb][2], s2 * acc[rb][cb][3]};
      if (kGateUp) {
        const int I = N >> 1;
        const uint32_t packed = mx::pack_bf16x2_rne(swiglu_clamped(v[0] + b0, v[1] + b1), swiglu_clamped(v[2] + b2, v[3] + b3));
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(args.out) + (size_t)(row0 + m) * I + (n >> 1)) = packed;
      } else {
        const int pr = args.sorted_pairs[row0 + m];
        const float wt = args.topk_weights[pr];
        f32x4 o;
        o[0] = wt * (v[0] + b0);
        o[1] = wt * (v[1] + b1);
        o[2] = wt * (v[2] + b2);
        o[3] = wt * (v[3] + b3);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(args.out) + (size_t)pr * N + n) = pack_bf16x4(o);
      }
    }
  }
}

#ifndef MX_MID_PANEL
#define MX_MID_PANEL 1
#endif

template <bool kGateUp, bool kNv>
hipError_t launch_mid(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  constexpr int kP = MX_MID_PANEL;
  const long n_tiles = (a.N + 127) / 128;
  const long blocks = n_tiles * a.max_tiles;
  if (blocks == 0) return hipSuccess;
  const long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&expert_mid_kernel<kP, kGateUp, kNv>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)mid_lds_bytes<kP, kNv>(mxfp4moe::kMaxHidden));
  if (attr != hipSuccess) return attr;
  expert_mid_kernel<kP, kGateUp, kNv><<<(unsigned)grid, 256, mid_lds_bytes<kP, kNv>(a.K), stream>>>(a);
  return hipGetLastError();
}

// y[t, n] = bf16(sum_j zw[t*k + j, n]) summed in fp32, j ascending, over the
// bf16 pair outputs; eight features per thread.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ zw, uint16_t* __restrict__ y,
                                                      int T, int H, int top_k) {
  const int h8 = H >> 3;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * h8) return;
  const int t = (int)(idx / h8);
  const int n = (int)(idx - (size_t)t * h8) * 8;
  const uint16_t* src = zw + (size_t)t * top_k * H + n;
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.f;
  for (int j = 0; j < top_k; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)j * H);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[2 * i] += mx::bf16_to_f32(v[i] & 0xffffu);
      s[2 * i + 1] += mx::bf16_to_f32(v[i] >> 16);
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = mx::pack_bf16x2_rne(s[2 * i], s[2 * i + 1]);
  *reinterpret_cast<u32x4*>(y + (size_t)t * H + n) = o;
}

}  // namespace

namespace mxfp4moe {

// wide: blocks of 512 weight rows x 128 tokens; gate_up 4 waves of 128 x 128
// (one per SIMD, operands read a chunk ahead), down 8 waves of 128 x 64 (two
// per SIMD).
// mid: 16x16x32 MFMA, 4 waves of 32 weight rows x (up to) 64 tokens, panels
// of MX_MID_PANEL chunks of both operands staged in LDS.
// stream: 16x16x32 MFMA, 4 waves of 16*MX_STREAM_RN weight rows x (at most 4)
// tokens, weights streamed in batches of MX_STREAM_BATCH chunks of 128 K.
static_assert(kWideTokens == 128 && kStreamTokens == 4, "tile sizes");

template <bool kGateUp>
static hipError_t launch_all(GemmArgs a, const TileTables& tt, const TileBounds& tb, hipStream_t stream) {
  hipError_t err = hipSuccess;
  if (tb.max_big > 0 && a.scale2 != nullptr) return hipErrorInvalidValue;  // NVFP4 runs mid / streaming tiles only
  if (tb.max_big > 0) {
    ProfileScope prof(kGateUp ? kStageGateUpWide : kStageDownWide, stream);
    GemmArgs w = a;
    w.tiles = tt.big;
    w.num_tiles = tt.num_big;
    w.max_tiles = tb.max_big;
    if (a.act_mode != kActBf16) {  // full tiles on the FP4 scaled MFMA over MXFP8 activations
      w.act = reinterpret_cast<const uint16_t*>(a.act_codes);
      err = launch_fp4<kGateUp>(w, a.act_mode == kActMxfp8Split, stream);
    } else {
      // gate_up: four waves of 128 rows x 128 pairs, operands read a chunk
      // ahead; down: eight waves of 128 rows x 64 pairs (two per SIMD, one
      // operand set each), whose second wave covers the heavier epilogue and
      // the LDS waits (measured at the 120b prefill shape: down 264 against
      // 274 us, gate_up 499 against 478 us the other way round)
      if (kGateUp)
        err = launch_wide<4, 1, 4, 4, true>(w, stream);
      else
        err = launch_wide<4, 2, 4, 2, false, false>(w, stream);
    }
  }
  if (err == hipSuccess && tb.max_mid > 0) {
    ProfileScope prof(kGateUp ? kStageGateUpMid : kStageDownMid, stream);
    a.tiles = tt.mid;
    a.num_tiles = tt.num_mid;
    a.max_tiles = tb.max_mid;
    err = a.scale2 != nullptr ? launch_mid<kGateUp, true>(a, stream) : launch_mid<kGateUp, false>(a, stream);
  }
  if (err == hipSuccess && tb.max_small > 0) {
    ProfileScope prof(kGateUp ? kStageGateUpStream : kStageDownStream, stream);
    a.tiles = tt.small;
    a.num_tiles = tt.num_small;
    a.max_tiles = tb.max_small;
    err = a.scale2 != nullptr ? launch_stream<kGateUp, true>(a, stream) : launch_stream<kGateUp, false>(a, stream);
  }
  return err;
}

hipError_t launch_gate_up(GemmArgs a, const TileTables& tt, const TileBounds& tb, hipStream_t stream) {
  ProfileScope prof(kStageGateUp, stream);
  return launch_all<true>(a, tt, tb, stream);
}

hipError_t launch_down(GemmArgs a, const TileTables& tt, const TileBounds& tb, hipStream_t stream) {
  ProfileScope prof(kStageDown, stream);
  return launch_all<false>(a, tt, tb, stream);
}

hipError_t launch_combine(const uint16_t* zw, uint16_t* y, int T, int H, int top_k, hipStream_t stream) {
  const size_t n = (size_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  ProfileScope prof(kStageCombine, stream);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(zw, y, T, H, top_k);
  return hipGetLastError();
}

}  // namespace mxfp4moe
