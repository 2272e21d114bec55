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
// K runs in chunks of 64 = two E8M0 groups.  Within a chunk lane half h
// (lane / 32) takes group h: it loads that group's 16 packed bytes of its
// weight row with one 128-bit load and converts dword s (eight codes) to the
// eight bf16 it feeds to MFMA step s.  The tokens' bf16 rows of the chunk are
// staged in LDS (row stride 144 B, conflict-free 128-bit reads) and each lane
// reads the eight values matching its weight codes.  Any consistent
// assignment of k to (lane half, step, element) yields the same dot products,
// and this one needs no reshuffle of the checkpoint layout.  Weights are
// dequantized exactly (E2M1 x 2^(s-127) is a bf16 value) and MFMA
// accumulates in fp32.
#include "internal.h"
#include "mx_device.h"

namespace {

using mx::bf16x8;
using mx::f32x16;
using mx::f32x4;
using mx::u32x4;

template <int WN, int WM, int RN, int RM>
struct Shape {
  static constexpr int kWaves = WN * WM;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BN = WN * RN * 32;  // weight rows per block
  static constexpr int BM = WM * RM * 32;  // token columns per block
  static constexpr int kSlots = BM * 8;    // 16-byte slots of one staged chunk (64 bf16 per token)
  static constexpr int kSlotsPerThread = (kSlots + kThreads - 1) / kThreads;
};

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
  return g * (1.0f / (1.0f + __expf(-1.702f * g))) * (u + 1.0f);
}

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

// One 64-wide K chunk of MFMA work for a wave: `ncb` (wave-uniform, in an
// SGPR) of its RM 32-token blocks hold tokens; each of the four K steps
// converts the wave's weight codes and issues RN MFMAs per live block.  All
// LDS reads of the chunk are issued before any conversion or MFMA (the
// scheduling barrier keeps the compiler from sinking them next to their
// uses), so the LDS latency is paid once per chunk instead of once per step.
template <int RN, int RM>
__device__ __forceinline__ void chunk_mma_live(int ncb, f32x16 (&acc)[RN][RM], const u32x4* __restrict__ xb,
                                               const u32x4 (&w)[RN], const float (&sc)[RN], int m_wave, int lrow,
                                               int half) {
  bf16x8 b[4][RM];
#pragma unroll
  for (int cb = 0; cb < RM; ++cb) {
    if (cb < ncb) {
      const int row = m_wave + cb * 32 + lrow;
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s][cb] = __builtin_bit_cast(bf16x8, xb[row * 8 + slot_col(row, half * 4 + s)]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 a[RN];
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) a[rb] = mx::as_bf16x8(mx::fp4x8_to_bf16x8(w[rb][s], sc[rb]));
#pragma unroll
    for (int cb = 0; cb < RM; ++cb) {
      if (cb < ncb) {
#pragma unroll
        for (int rb = 0; rb < RN; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[s][cb], acc[rb][cb], 0, 0, 0);
      }
    }
  }
}

// Branch-free chunk for tiles whose RM token blocks all hold tokens.  The
// converts producing step s+1's weight fragments (into the other half of a
// double buffer) are interleaved one-for-one with step s's MFMAs, so the
// matrix core never waits for a burst of conversions.
template <int RN, int RM>
__device__ __forceinline__ void chunk_mma_full(f32x16 (&acc)[RN][RM], const u32x4* __restrict__ xb,
                                               const u32x4 (&w)[RN], const float (&sc)[RN], int lrow, int half) {
  static_assert(RN * RM >= 4 * RN, "one convert per MFMA needs RM >= 4");
  bf16x8 b[4][RM];
#pragma unroll
  for (int cb = 0; cb < RM; ++cb) {
    const int row = cb * 32 + lrow;
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s][cb] = __builtin_bit_cast(bf16x8, xb[row * 8 + slot_col(row, half * 4 + s)]);
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 a[2][RN];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) a[0][rb] = mx::fp4x8_to_bf16x8(w[rb][0], sc[rb]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < RN * RM; ++i) {
      const int rb = i % RN, cb = i / RN;
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mx::as_bf16x8(a[s & 1][rb]), b[s][cb], acc[rb][cb], 0, 0, 0);
      if (s + 1 < 4 && i < 4 * RN) {
        // convert dword (s+1) of weight fragment i/4, element pair i%4
        const int nrb = i / 4, sel = i % 4;
        const uint32_t packed = w[nrb][s + 1];
        uint32_t v;
        if (sel == 0) v = mx::fp4x2_to_bf16x2<0>(packed, sc[nrb]);
        else if (sel == 1) v = mx::fp4x2_to_bf16x2<1>(packed, sc[nrb]);
        else if (sel == 2) v = mx::fp4x2_to_bf16x2<2>(packed, sc[nrb]);
        else v = mx::fp4x2_to_bf16x2<3>(packed, sc[nrb]);
        a[(s + 1) & 1][nrb][sel] = v;
      }
    }
  }
}

// Epilogue.  Lane holds, for every (rb, cb), token m = m_wave + cb*32 + lrow
// and features n = n_wave + rb*32 + 8i + 4*half + {0,1,2,3}, i = 0..3.
// gate_up: add the bias, clamped SwiGLU of (gate, up) = (n, n+1), store a in
// bf16 at the pair's expert-ordered row.  down: add the bias, multiply by the
// pair's routing weight, store fp32 at the pair's own row.
template <int RN, int RM, bool kGateUp>
__device__ __forceinline__ void store_epilogue(const mxfp4moe::GemmArgs& args, const f32x16 (&acc)[RN][RM], int e,
                                               int row0, int count, int n_wave, int m_wave, int cb_live, int half,
                                               int lrow) {
  const int N = args.N;
  const uint16_t* bias = args.bias + (size_t)e * N;
  uint2 bv[RN][4];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int n = n_wave + rb * 32 + 8 * i + 4 * half;
      n = n < N ? n : N - 4;
      bv[rb][i] = *reinterpret_cast<const uint2*>(bias + n);
    }
#pragma unroll
  for (int cb = 0; cb < RM; ++cb) {
    if (cb >= cb_live) continue;
    const int m = m_wave + cb * 32 + lrow;
    if (m >= count) continue;
    if (kGateUp) {
      uint32_t* arow = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(args.out) + (size_t)(row0 + m) * (N >> 1));
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n_wave + rb * 32 + 8 * i + 4 * half;
          if (n < N) {
            const uint2 bb = bv[rb][i];
            const float b0 = mx::bf16_to_f32(bb.x & 0xffffu), b1 = mx::bf16_to_f32(bb.x >> 16);
            const float b2 = mx::bf16_to_f32(bb.y & 0xffffu), b3 = mx::bf16_to_f32(bb.y >> 16);
            const float a0 = swiglu_clamped(acc[rb][cb][4 * i + 0] + b0, acc[rb][cb][4 * i + 1] + b1);
            const float a1 = swiglu_clamped(acc[rb][cb][4 * i + 2] + b2, acc[rb][cb][4 * i + 3] + b3);
            arow[n >> 2] = mx::f32_to_bf16_rne(a0) | (mx::f32_to_bf16_rne(a1) << 16);
          }
        }
      }
    } else {
      const int p = args.sorted_pairs[row0 + m];
      const float w = args.topk_weights[p];
      float* zrow = static_cast<float*>(args.out) + (size_t)p * N;
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n_wave + rb * 32 + 8 * i + 4 * half;
          if (n < N) {
            const uint2 bb = bv[rb][i];
            f32x4 v;
            v[0] = w * (acc[rb][cb][4 * i + 0] + mx::bf16_to_f32(bb.x & 0xffffu));
            v[1] = w * (acc[rb][cb][4 * i + 1] + mx::bf16_to_f32(bb.x >> 16));
            v[2] = w * (acc[rb][cb][4 * i + 2] + mx::bf16_to_f32(bb.y & 0xffffu));
            v[3] = w * (acc[rb][cb][4 * i + 3] + mx::bf16_to_f32(bb.y >> 16));
            *reinterpret_cast<f32x4*>(zrow + n) = v;
          }
        }
      }
    }
  }
}

template <int WN, int WM, int RN, int RM, bool kGateUp>
__global__ __launch_bounds__(WN * WM * 64, (WN * WM * 64 >= 256 && RN * RM >= 8) ? 2 : 1) void expert_gemm_kernel(
    mxfp4moe::GemmArgs args) {
  using S = Shape<WN, WM, RN, RM>;
  __shared__ __attribute__((aligned(16))) u32x4 xs[2][S::kSlots];

  const int N = args.N, K = args.K;
  const int n_tiles = (N + S::BN - 1) / S::BN;
  int tile, ntile;
  if (!map_block(*args.num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
  const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  const int e = __builtin_amdgcn_readfirstlane(tl.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tl.y);
  const int count = __builtin_amdgcn_readfirstlane(tl.z);

  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 1) >> 1;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int lrow = lane & 31;
  const int wn = wave % WN, wm = wave / WN;
  const int n_wave = ntile * S::BN + wn * RN * 32;
  const int m_wave = wm * RM * 32;
  int cb_live = (count - m_wave + 31) >> 5;  // 32-token blocks of this wave holding tokens
  cb_live = __builtin_amdgcn_readfirstlane(cb_live < 0 ? 0 : (cb_live > RM ? RM : cb_live));

  // Weight rows of this lane (rows past N re-read row N-1; their outputs are dropped).
  const uint8_t* wrow[RN];
  const uint8_t* srow[RN];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) {
    int n = n_wave + rb * 32 + lrow;
    n = n < N ? n : N - 1;
    wrow[rb] = args.wblocks + ((size_t)e * N + n) * (size_t)(K >> 1);
    srow[rb] = args.wscales + ((size_t)e * N + n) * (size_t)kgroups;
  }

  // Slots this thread stages: slot p = t + i*threads holds token row p/8,
  // logical 16-byte column slot_col^-1 of p%8.  Rows past `count` re-read the
  // tile's first row (their columns are never stored).
  const uint16_t* xsrc[S::kSlotsPerThread];
  int xcol[S::kSlotsPerThread];
#pragma unroll
  for (int i = 0; i < S::kSlotsPerThread; ++i) {
    const int p = threadIdx.x + i * S::kThreads;
    const int r = p >> 3;
    const int part = slot_col(r, p & 7);  // the swizzle is an involution on the column
    int rr = r < count ? r : 0;
    size_t src_row;
    if (kGateUp)
      src_row = (size_t)(args.sorted_pairs[row0 + rr] / args.top_k);
    else
      src_row = (size_t)(row0 + rr);
    xsrc[i] = args.act + src_row * (size_t)K + part * 8;
    xcol[i] = part * 8;
  }

  u32x4 xstage[S::kSlotsPerThread];
  auto load_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < S::kSlotsPerThread; ++i) {
      if (S::kSlots % S::kThreads == 0 || threadIdx.x + i * S::kThreads < S::kSlots) {
        // K tail: the missing half chunk re-reads the first half (its weights are zero)
        const int koff = (c * 64 + xcol[i] < K) ? c * 64 : c * 64 - 32;
        xstage[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + koff);
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < S::kSlotsPerThread; ++i)
      if (S::kSlots % S::kThreads == 0 || threadIdx.x + i * S::kThreads < S::kSlots)
        xs[buf][threadIdx.x + i * S::kThreads] = xstage[i];
  };

  u32x4 wcur[RN], wnxt[RN];
  uint32_t scur[RN], snxt[RN];
  auto load_w = [&](int c, u32x4* w, uint32_t* s) {
    const int g = 2 * c + half;
    const int gg = g < kgroups ? g : g - 1;
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      w[rb] = *reinterpret_cast<const u32x4*>(wrow[rb] + (size_t)gg * 16);
      s[rb] = srow[rb][gg];
    }
  };

  f32x16 acc[RN][RM];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int cb = 0; cb < RM; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  load_w(0, wcur, scur);
  load_x(0);
  store_x(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(c + 1, wnxt, snxt);
      load_x(c + 1);
    }
    const bool glive = 2 * c + half < kgroups;
    {
      u32x4 w[RN];
      float sc[RN];
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
        w[rb] = glive ? wcur[rb] : u32x4{0u, 0u, 0u, 0u};
        sc[rb] = mx::e8m0_operand(scur[rb]);
      }
      chunk_mma_live<RN, RM>(cb_live, acc, xs[buf], w, sc, m_wave, lrow, half);
    }
    if (more) {
      store_x(buf ^ 1);
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
        wcur[rb] = wnxt[rb];
        scur[rb] = snxt[rb];
      }
    }
    __syncthreads();
  }

  store_epilogue<RN, RM, kGateUp>(args, acc, e, row0, count, n_wave, m_wave, cb_live, half, lrow);
}

// Wide tiles for prefill-sized expert groups.
//
// One wave per SIMD, each computing a (32*RN) x (32*RM) tile with its
// accumulators in registers; WN waves stack along the weight rows, so a block
// covers (32*RN*WN) weight rows x (32*RM) tokens and every staged token chunk
// feeds WN waves.  Per 64-wide K chunk a block moves BM*128 bytes of tokens
// and BN*32 bytes of packed weights from global memory: each thread loads its
// share of chunk c+kDepth into a register ring while the waves run MFMA on
// chunk c from LDS; all loads of a wave have the same age, so they complete in
// order without draining the ring.  Staged chunks are written to the spare of
// two LDS stages; one barrier per chunk.  The scale bytes of the block's
// weight rows are staged once, group-major.
constexpr int kWideMaxGroups = 128;  // K <= 4096

template <int WN, int RN, int RM, int kDepth, bool kGateUp>
__global__ __launch_bounds__(WN * 64, 1) void expert_gemm_wide_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kThreads = WN * 64;
  constexpr int BN = WN * RN * 32;
  constexpr int BM = RM * 32;
  constexpr int kXSlots = BM * 8;  // 16-byte token slots per chunk
  constexpr int kWSlots = BN * 2;  // 16-byte weight slots per chunk (one 32-code group each)
  constexpr int kXPer = kXSlots / kThreads;
  constexpr int kWPer = kWSlots / kThreads;
  static_assert(kXSlots % kThreads == 0 && kWSlots % kThreads == 0, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) u32x4 xs[2][kXSlots];
  __shared__ __attribute__((aligned(16))) u32x4 wsm[2][kWSlots];
  __shared__ uint8_t sst[BN * kWideMaxGroups];

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
  const int niter = (nchunks + kDepth - 1) / kDepth * kDepth;  // padded: every iteration is branch-free
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int half = lane >> 5;
  const int lrow = lane & 31;

  // scale bytes of the block's rows, group-major: sst[g * BN + row]
  for (int i = t; i < BN * kgroups; i += kThreads) {
    const int r = i / kgroups;
    const int g = i - r * kgroups;
    int n = ntile * BN + r;
    n = n < N ? n : N - 1;
    sst[g * BN + r] = args.wscales[((size_t)e * N + n) * (size_t)kgroups + g];
  }

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
    wr = wr < N ? wr : N - 1;
    wsrc[j] = args.wblocks + ((size_t)e * N + wr) * (size_t)(K >> 1);
  }
  const int wh = t & 1;

  u32x4 xr[kDepth][kXPer];
  u32x4 wr[kDepth][kWPer];
  auto issue = [&](int c, int d) {
    c = c < nchunks ? c : nchunks - 1;  // padding iterations re-read the last chunk
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      // K tail: the missing half chunk re-reads the first half (its weights are zero)
      const int koff = (c * 64 + xcol[i] < K) ? c * 64 : c * 64 - 32;
      xr[d][i] = *reinterpret_cast<const u32x4*>(xsrc[i] + koff);
    }
    int g = 2 * c + wh;
    g = g < kgroups ? g : g - 1;
#pragma unroll
    for (int j = 0; j < kWPer; ++j) wr[d][j] = *reinterpret_cast<const u32x4*>(wsrc[j] + (size_t)g * 16);
  };
  auto commit = [&](int d, int st) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) xs[st][t + i * kThreads] = xr[d][i];
#pragma unroll
    for (int j = 0; j < kWPer; ++j) wsm[st][t + j * kThreads] = wr[d][j];
  };

  // compute-side constants
  const int n_wave = ntile * BN + wave * RN * 32;
  int cb_live = (count + 31) >> 5;
  cb_live = __builtin_amdgcn_readfirstlane(cb_live > RM ? RM : cb_live);
  const int wslot0 = (wave * RN * 32 + lrow) * 2 + half;
  const uint8_t* srow = sst + wave * RN * 32 + lrow;

  f32x16 acc[RN][RM];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int cb = 0; cb < RM; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(d, d);
  commit(0, 0);
  issue(kDepth, 0);
  __syncthreads();  // also publishes the scale table

  for (int c0 = 0; c0 < niter; c0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int c = c0 + u;
      // stage chunk c+1 (register slot (u+1)%kDepth) into the spare LDS stage,
      // then refill that slot with chunk c+1+kDepth
      commit((u + 1) % kDepth, (c + 1) & 1);
      issue(c + 1 + kDepth, (u + 1) % kDepth);
      if (c < nchunks) {
        const int st = c & 1;
        const int g = 2 * c + half;
        const bool glive = g < kgroups;
        const int gg = glive ? g : g - 1;
        u32x4 w[RN];
        float sc[RN];
#pragma unroll
        for (int rb = 0; rb < RN; ++rb) {
          w[rb] = wsm[st][wslot0 + rb * 64];
          sc[rb] = mx::e8m0_operand(srow[gg * BN + rb * 32]);
          if (!glive) w[rb] = u32x4{0u, 0u, 0u, 0u};
        }
        chunk_mma_full<RN, RM>(acc, xs[st], w, sc, lrow, half);
      }
      __syncthreads();
    }
  }
  store_epilogue<RN, RM, kGateUp>(args, acc, e, row0, count, n_wave, 0, cb_live, half, lrow);
}

template <int WN, int RN, int RM, int kDepth, bool kGateUp>
hipError_t launch_wide(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  constexpr int BN = WN * RN * 32;
  const long n_tiles = (a.N + BN - 1) / BN;
  const long blocks = n_tiles * a.max_tiles;
  const long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  expert_gemm_wide_kernel<WN, RN, RM, kDepth, kGateUp><<<(unsigned)grid, WN * 64, 0, stream>>>(a);
  return hipGetLastError();
}

// y[t, n] = bf16(sum_j zw[t*k + j, n]), j ascending; four features per thread.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ zw, uint16_t* __restrict__ y,
                                                      int T, int H, int top_k) {
  const int h4 = H >> 2;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * h4) return;
  const int t = (int)(idx / h4);
  const int n = (int)(idx - (size_t)t * h4) * 4;
  const float* src = zw + (size_t)t * top_k * H + n;
  f32x4 s = *reinterpret_cast<const f32x4*>(src);
  for (int j = 1; j < top_k; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (size_t)j * H);
    s[0] += v[0];
    s[1] += v[1];
    s[2] += v[2];
    s[3] += v[3];
  }
  uint2 o;
  o.x = mx::f32_to_bf16_rne(s[0]) | (mx::f32_to_bf16_rne(s[1]) << 16);
  o.y = mx::f32_to_bf16_rne(s[2]) | (mx::f32_to_bf16_rne(s[3]) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + n) = o;
}

template <int WN, int WM, int RN, int RM, bool kGateUp>
hipError_t launch_cfg(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  using S = Shape<WN, WM, RN, RM>;
  const long n_tiles = (a.N + S::BN - 1) / S::BN;
  const long blocks = n_tiles * a.max_tiles;
  const long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  expert_gemm_kernel<WN, WM, RN, RM, kGateUp><<<(unsigned)grid, S::kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

namespace mxfp4moe {

// small: 4 waves x 32 weight rows, 32 tokens; mid: 2x2 waves of 64 rows x 32 tokens;
// wide: 4 waves of 128 rows x 128 tokens (block 512 x 128), register-ring staging.
#define MX_SMALL 4, 1, 1, 1
#define MX_MID 2, 2, 2, 1
#define MX_WIDE_WN 4
#define MX_WIDE_RN 4
#define MX_WIDE_RM 4
#define MX_WIDE_DEPTH 2

int gemm_tile_tokens(GemmConfig cfg) {
  return cfg == kGemmSmall ? Shape<MX_SMALL>::BM : cfg == kGemmMid ? Shape<MX_MID>::BM : (MX_WIDE_RM * 32);
}

hipError_t launch_gate_up(const GemmArgs& a, GemmConfig cfg, hipStream_t stream) {
  if (a.max_tiles == 0) return hipSuccess;
  ProfileScope prof(kStageGateUp, stream);
  if (cfg == kGemmSmall) return launch_cfg<MX_SMALL, true>(a, stream);
  if (cfg == kGemmMid) return launch_cfg<MX_MID, true>(a, stream);
  return launch_wide<MX_WIDE_WN, MX_WIDE_RN, MX_WIDE_RM, MX_WIDE_DEPTH, true>(a, stream);
}

hipError_t launch_down(const GemmArgs& a, GemmConfig cfg, hipStream_t stream) {
  if (a.max_tiles == 0) return hipSuccess;
  ProfileScope prof(kStageDown, stream);
  if (cfg == kGemmSmall) return launch_cfg<MX_SMALL, false>(a, stream);
  if (cfg == kGemmMid) return launch_cfg<MX_MID, false>(a, stream);
  return launch_wide<MX_WIDE_WN, MX_WIDE_RN, MX_WIDE_RM, MX_WIDE_DEPTH, false>(a, stream);
}

hipError_t launch_combine(const float* zw, uint16_t* y, int T, int H, int top_k, hipStream_t stream) {
  const size_t n = (size_t)T * (H / 4);
  if (n == 0) return hipSuccess;
  ProfileScope prof(kStageCombine, stream);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(zw, y, T, H, top_k);
  return hipGetLastError();
}

}  // namespace mxfp4moe
