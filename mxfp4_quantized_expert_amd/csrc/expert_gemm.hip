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
#include <type_traits>

#include "expert_device.h"
#include "internal.h"
#include "mx_device.h"
#include "route_device.h"

namespace {

using mxgemm::GroupScale;
using mxgemm::bias4_of;
using mxgemm::load_bias4;
using mxgemm::load_bias4_raw;
using mxgemm::load_lds16;
using mxgemm::lds_reads_then_barrier;
using mxgemm::load_lds4;
using mxgemm::pack_bf16x4;
using mxgemm::stage_scales;
using mxgemm::staged_row;
using mxgemm::swiglu_clamped;
using mxgemm::w13_row;
using mxgemm::wait_loads_then_barrier;

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

// Block -> (tile, weight-row tile).  Blocks are dealt to the 8 XCDs round
// robin (block b runs on XCD b % 8), so the id is first remapped so that each
// XCD owns a contiguous range of the work, then walked in groups of kGroup
// token tiles with the token tile fastest: blocks running together on one XCD
// share the weight rows of one expert (and the staged tokens of a few tiles)
// through that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroup = 4;

__device__ __forceinline__ bool map_job(int b, int num_tiles, int n_tiles, int& tile, int& ntile) {
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
__device__ __forceinline__ bool map_block(int num_tiles, int n_tiles, int& tile, int& ntile) {
  return map_job(blockIdx.x, num_tiles, n_tiles, tile, ntile);
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
// MXFP4 (kNv = false): sc[rb] is fragment rb's E8M0 scale as a convert
// operand; sc_hi is unused.  NVFP4: sc[rb] and sc_hi[rb] are the E4M3 block
// scales of steps 0-1 and 2-3 as floats, applied by the exact float32
// conversion.
// kF16 (NVFP4 only): the tokens are f16; each E4M3 block scale comes as its
// power of two (sc, sc_hi) and its significand as an f16 pair (mt, mt_hi),
// the codes are converted to f16 by the scaled convert and one packed
// multiply, and the MFMAs are f16.
// RML <= RM: only the first RML token blocks hold pairs of the tile (the
// others are neither read nor multiplied); extra(k) runs for k < 4*RN*RML.
template <int RN, int RM, bool kNv = false, bool kF16 = false, int RML = RM, typename Extra = NoExtra>
__device__ __forceinline__ void chunk_mma_regs(f32x16 (&acc)[RN][RM], const bf16x8 (&b)[4][RM],
                                               const u32x4 (&w)[RN], const float (&sc)[RN],
                                               const float (&sc_hi)[RN], Extra extra = Extra(),
                                               const uint32_t* mt = nullptr, const uint32_t* mt_hi = nullptr) {
  static_assert(!kF16 || kNv, "f16 operands for NVFP4 weights");
  auto f16_pair = [&](uint32_t packed, int sel, float pow2, uint32_t mant2) {
    uint32_t v;
    if (sel == 0) v = mx::fp4x2_to_f16x2<0>(packed, pow2);
    else if (sel == 1) v = mx::fp4x2_to_f16x2<1>(packed, pow2);
    else if (sel == 2) v = mx::fp4x2_to_f16x2<2>(packed, pow2);
    else v = mx::fp4x2_to_f16x2<3>(packed, pow2);
    return mx::mul_f16x2(v, mant2);
  };
  u32x4 a[2][RN];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb) {
    if constexpr (kF16) {
#pragma unroll
      for (int sel = 0; sel < 4; ++sel) a[0][rb][sel] = f16_pair(w[rb][0], sel, sc[rb], mt[rb]);
    } else {
      a[0][rb] = kNv ? mx::fp4x8_to_bf16x8_any_scale(w[rb][0], sc[rb]) : mx::fp4x8_to_bf16x8(w[rb][0], sc[rb]);
    }
  }
  auto convert = [&](int s, int i) {  // converts pair i%4 of fragment i/4 for step s
    const int rb = i / 4, sel = i % 4;
    const uint32_t packed = w[rb][s];
    uint32_t v;
    if (kF16) {
      v = s < 2 ? f16_pair(packed, sel, sc[rb], mt[rb]) : f16_pair(packed, sel, sc_hi[rb], mt_hi[rb]);
    } else if (kNv) {
      const float f = s < 2 ? sc[rb] : sc_hi[rb];
      if (sel == 0) v = mx::fp4x2_to_bf16x2_any_scale<0>(packed, f);
      else if (sel == 1) v = mx::fp4x2_to_bf16x2_any_scale<1>(packed, f);
      else if (sel == 2) v = mx::fp4x2_to_bf16x2_any_scale<2>(packed, f);
      else v = mx::fp4x2_to_bf16x2_any_scale<3>(packed, f);
    } else {
      if (sel == 0) v = mx::fp4x2_to_bf16x2<0>(packed, sc[rb]);
      else if (sel == 1) v = mx::fp4x2_to_bf16x2<1>(packed, sc[rb]);
      else if (sel == 2) v = mx::fp4x2_to_bf16x2<2>(packed, sc[rb]);
      else v = mx::fp4x2_to_bf16x2<3>(packed, sc[rb]);
    }
    a[s & 1][rb][sel] = v;
  };
  static_assert(RML >= 1 && RML <= RM, "live token blocks");
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < RN * RML; ++i) {
      const int rb = i % RN, cb = i / RN;
      if constexpr (kF16)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(mx::f16x8, a[s & 1][rb]),
                                                             __builtin_bit_cast(mx::f16x8, b[s][cb]), acc[rb][cb], 0, 0, 0);
      else
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mx::as_bf16x8(a[s & 1][rb]), b[s][cb], acc[rb][cb], 0, 0, 0);
      if (s + 1 < 4 && i < 4 * RN) convert(s + 1, i);
      extra(s * RN * RML + i);
    }
    if (s + 1 < 4) {
#pragma unroll
      for (int i = RN * RML; i < 4 * RN; ++i) convert(s + 1, i);
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

template <bool kValue>
struct Flag {
  static constexpr bool value = kValue;
};

// Epilogue, staged through an LDS region of RM*32*128 bytes per wave so
// that every token's outputs leave as full 128-byte rows: the lane layout of
// the MFMA results (four consecutive features of one token per lane) is
// written to LDS as [token][features] (16-byte chunks XOR-swizzled by token),
// then read back along the features and stored as whole rows.
// gate_up: bias, clamped SwiGLU, bf16 -> a[pair row][I] (16*RN activations,
// 32*RN bytes, per token per wave).  down: bias and routing weight in fp32,
// rounded to bf16 -> zw[pair][H], one 32-feature slab (staged as 128 bytes,
// stored as 64 per token) per pass.  NVFP4: the sums are first multiplied by
// the expert's second-level scale (before the bias).
template <int RN, int RM, bool kGateUp, bool kNv = false, bool kF16Out = false>
__device__ __forceinline__ void store_epilogue(const mxfp4moe::GemmArgs& args, const f32x16 (&acc)[RN][RM], int e,
                                              int row0, int count, int n_wave, int lane, uint8_t* region,
                                              bool add_bias = true) {
  const int N = args.N;
  const int half = lane >> 5, lrow = lane & 31;
  const uint16_t* bias = args.bias + (size_t)e * N;
  const float s2 = kNv ? args.scale2[e] : 1.0f;
  auto sum = [&](int rb, int cb, int r) { return kNv ? s2 * acc[rb][cb][r] : acc[rb][cb][r]; };
  auto chunk_addr = [](int m, int chunk) { return m * 128 + ((chunk ^ (m & 7)) << 4); };
  const bool split = kGateUp && args.split_gate_up != 0;
  // Every global value the epilogue reads (this lane's biases, and for down
  // its pairs' routing weights and pair ids) is loaded in one batch before
  // the first use: loaded where used, each would be a round trip of its own.
  // (add_bias = false: gate_up sums that started at their biases)
  uint2 braw[RN][4];
  if (add_bias) {
#pragma unroll
    for (int rb = 0; rb < RN; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n_wave + rb * 32 + 8 * i + 4 * half;
        braw[rb][i] = load_bias4_raw(bias, n < N ? n : N - 4, N, split);
      }
  }
  if (kGateUp) {
    // stage a[m][q_local], q_local = 0..16*RN-1 for this wave's 32*RN rows of w13
    auto stage = [&](auto with_bias) {
      constexpr bool kB = decltype(with_bias)::value;
#pragma unroll
      for (int rb = 0; rb < RN; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 bv = kB ? bias4_of(braw[rb][i], split) : f32x4{};
          const int byte = rb * 32 + 8 * i + 4 * half;  // 2 * q_local
#pragma unroll
          for (int cb = 0; cb < RM; ++cb) {
            const int m = cb * 32 + lrow;
            float h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = kB ? sum(rb, cb, 4 * i + j) + bv[j] : sum(rb, cb, 4 * i + j);
            const float a0 = swiglu_clamped(h[0], h[1]);
            const float a1 = swiglu_clamped(h[2], h[3]);
            *reinterpret_cast<uint32_t*>(region + chunk_addr(m, byte >> 4) + (byte & 15)) =
                kF16Out ? mx::pack_f16x2_rne(a0, a1) : mx::pack_bf16x2_rne(a0, a1);
          }
        }
      }
    };
    if (add_bias) stage(Flag<true>{});
    else stage(Flag<false>{});
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
    // token m = cb*32 + lrow of each column block: its routing weight (0 past
    // the tile's pairs); store pass j: the pair of token (j*64 + lane) / 8
    constexpr int kStores = RM * 32 * 8 / 64;
    const int last = count - 1;
    int spw[RM], pid[kStores];
#pragma unroll
    for (int cb = 0; cb < RM; ++cb) spw[cb] = args.sorted_pairs[row0 + min(cb * 32 + lrow, last)];
#pragma unroll
    for (int j = 0; j < kStores; ++j) pid[j] = args.sorted_pairs[row0 + min((j * 64 + lane) >> 3, last)];
    float wt[RM];
#pragma unroll
    for (int cb = 0; cb < RM; ++cb) wt[cb] = cb * 32 + lrow < count ? args.topk_weights[spw[cb]] : 0.f;
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      // stage zw[m][32 features of block rb]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 bv = bias4_of(braw[rb][i], false);
        const float b0 = bv[0], b1 = bv[1], b2 = bv[2], b3 = bv[3];
#pragma unroll
        for (int cb = 0; cb < RM; ++cb) {
          const int m = cb * 32 + lrow;
          const float w = wt[cb];
          f32x4 v;
          v[0] = w * (sum(rb, cb, 4 * i + 0) + b0);
          v[1] = w * (sum(rb, cb, 4 * i + 1) + b1);
          v[2] = w * (sum(rb, cb, 4 * i + 2) + b2);
          v[3] = w * (sum(rb, cb, 4 * i + 3) + b3);
          *reinterpret_cast<f32x4*>(region + chunk_addr(m, 2 * i + half)) = v;
        }
      }
#pragma unroll
      for (int j = 0; j < kStores; ++j) {
        const int idx = j * 64 + lane;
        const int m = idx >> 3, chunk = idx & 7;
        const int n = n_wave + rb * 32 + chunk * 4;
        if (m < count && n < N) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(region + chunk_addr(m, chunk));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(args.out) + (size_t)pid[j] * N + n) = pack_bf16x4(v);
        }
      }
    }
  }
}

// The wide kernel.  Operand chunks move from global memory to LDS by the
// load unit itself (global_load_lds_dwordx4: 16 bytes per lane, written at
// the wave's LDS address + 16 * lane; no staging registers, no LDS stores in
// the wave's stream), two or three LDS stages deep.  Per chunk c: wait for
// this wave's loads of chunk c (those of chunk c+1 stay in flight), barrier
// (every wave's share is in LDS), read the chunk's operands (weight groups,
// scale bytes, token fragments) into registers, then its MFMAs with the
// loads of chunk c+2 spread between them, one after every other MFMA (issued
// as a burst they would stall the wave with the matrix core idle).  With
// three stages chunk c+2 goes to the stage of chunk c-1; with two, to chunk
// c's own stage, after a second barrier that every wave reaches once it has
// read chunk c.  The wait for a chunk's loads is covered by the other wave
// on the SIMD: blocks run two waves per SIMD, either as eight waves of one
// block or as two blocks of four waves per CU, whose epilogues, barriers
// and conversions then also run beside the other block's MFMAs.
// kNv: NVFP4 weights (E4M3 block scales per 16 codes, K a multiple of 64).  A
// chunk's four scale bytes of a row are one aligned dword; they reach LDS
// through a two-slot ring in groups of consecutive chunks (described in the
// kernel), in place of the MXFP4 path's table of whole scale rows.
// kTail: the general form, for any K (a multiple of 32): when K is not a
// multiple of 64 the last chunk holds one group, whose missing group re-reads
// the one before and multiplies zeroed weights; operands are addressed by
// 64-bit pointers.  Without it (K a multiple of 64, every byte offset into the
// activations and into one expert's weights below 2^31) the selects are
// compiled out and the loads are buffer loads into LDS: a thread keeps a
// 32-bit offset per operand row and the chunk's offset moves in a scalar
// register, so a chunk's loads cost no vector address arithmetic.
// Whether a wide-kernel configuration's fast form is persistent (one block
// per CU walking its jobs, the next job's first chunk loading during the
// epilogue): the down GEMM at one block per CU whose epilogue regions stay
// below the last LDS stage.  The launcher sizes the grid by the same rule.
template <int WN, int WM, int RN, int RM, bool kGateUp, int kBlocksPerCu, int kStage16>
constexpr bool wide_persistent() {
  return !kGateUp && kBlocksPerCu == 1 && WN * WM * RM * 32 * 128 <= 2 * kStage16 * 16;
}

template <int WN, int WM, int RN, int RM, bool kGateUp, bool kNv = false, bool kTail = false, int kStageCount = 3,
          int kBlocksPerCu = 1>
__global__ __launch_bounds__(WN * WM * 64, kBlocksPerCu) void expert_wide_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kThreads = WN * WM * 64;
  constexpr int BN = WN * RN * 32;
  constexpr int BM = WM * RM * 32;
  constexpr int kXSlots = BM * 8;
  constexpr int kWSlots = BN * 2;
  constexpr int kXPer = kXSlots / kThreads;
  constexpr int kWPer = kWSlots / kThreads;
  static_assert(kXSlots % kThreads == 0 && kWSlots % kThreads == 0, "tile / thread mismatch");
  constexpr int kStages = kStageCount;  // LDS stages (see above)
  // NVFP4 scales: a row's four scale bytes of a chunk are one dword, and the
  // dwords of consecutive chunks in a row are contiguous.  They travel in
  // groups of kSG chunks (4 beside three stages, 8 beside two) into a ring of
  // two slots of BN rows x 4*kSG bytes, kSG lanes per row (one 4*kSG-byte
  // piece per row and line, instead of one line per row and chunk), one
  // kSG-th of the next group with each chunk.
  constexpr int kSG = kStages == 2 ? 8 : 4;
  static_assert(!kNv || BN == kThreads, "NVFP4: one scale dword per thread and chunk");
  constexpr int kRing = kNv ? 2 * BN * 4 * kSG : 0;
  static_assert(kStages == 2 || kStages == 3, "two or three stages");
  constexpr int kLoads = kXPer + kWPer;  // operand loads per thread per chunk
  constexpr int kStage = kXSlots + kWSlots;  // 16-byte slots per stage
  constexpr int kArena = kStages * kStage * 16 + (kNv ? kRing : BN * kWideMaxGroups);
  static_assert(WN * WM * RM * 32 * 128 <= kArena, "epilogue regions fit in the arena");
  constexpr bool kPersist = !kTail && wide_persistent<WN, WM, RN, RM, kGateUp, kBlocksPerCu, kStage>();
  static_assert(!(kNv && kPersist), "the NVFP4 scale ring is per job");
  // NVFP4 full tiles pass the gate_up output to the down GEMM in f16 (|a| <=
  // 56: the clamps bound it): gate_up stores it so, the down GEMM converts
  // its weights to f16 (two instructions per pair of codes instead of four)
  // and multiplies in f16
  constexpr bool kF16Out = kNv && kGateUp;
  constexpr bool kF16In = kNv && !kGateUp;
  __shared__ __attribute__((aligned(16))) u32x4 arena[kArena / 16];
  uint8_t* const sst = reinterpret_cast<uint8_t*>(arena + kStages * kStage);

  const int N = args.N, K = args.K;
  const int n_tiles = (N + BN - 1) / BN;
  const int num_tiles = *args.num_tiles;
  // this block's jobs: virtual block ids blockIdx.x + j * gridDim.x (gridDim.x
  // a multiple of 8, so every one is on this block's XCD), in the order the
  // dispatcher would hand them out
  int vb = blockIdx.x;
  int tile, ntile;
  if (!map_job(vb, num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
  int e, row0, count;
  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 1) >> 1;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int lane = t & 63;

  const bool split = kGateUp && args.split_gate_up;  // uniform
  const int wh = t & 1;
  // the fast form's buffer resources and per-thread byte offsets (the same
  // rows as the pointers); raw buffers, no swizzle, range-checked against
  // their byte counts (built in the general form too, where nothing uses them)
  constexpr int kRawBuffer = 0x00020000;  // descriptor word 3: 32-bit data format, for untyped loads
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(args.act), (short)0, (int)(args.act_rows * K * 2), kRawBuffer);
  __amdgpu_buffer_rsrc_t rw, rs;
  const uint16_t* xsrc[kXPer];
  int xcol[kXPer];
  const uint8_t* wsrc[kWPer];
  int xoff[kXPer], woff[kWPer];
  int sq0 = 0, sdw = 0;  // NVFP4: this thread's scale row (logical, part 0) and dword in the group
  // one job's operand addresses: the fast form keeps 32-bit offsets only, the
  // general form 64-bit pointers (and the column of each token slot)
  auto setup = [&]() {
    // the thread index through an opaque copy: what is derived from it is
    // recomputed per job instead of hoisted out of the job loop and held in
    // registers through the K loop and the epilogue
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
    e = __builtin_amdgcn_readfirstlane(tl.x);
    row0 = __builtin_amdgcn_readfirstlane(tl.y);
    count = __builtin_amdgcn_readfirstlane(tl.z);
    // token slot p = t + i*threads -> row p/8, logical column slot_col(row, p%8);
    // rows past `count` re-read the tile's first row (their columns are never stored)
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int p = t + i * kThreads;
      const int r = p >> 3;
      const int part = slot_col(r, p & 7);
      const int rr = r < count ? r : 0;
      const int src_row = kGateUp ? args.sorted_pairs[row0 + rr] / args.top_k : row0 + rr;
      if constexpr (kTail) {
        xsrc[i] = args.act + (size_t)src_row * (size_t)K + part * 8;
        xcol[i] = part * 8;
      } else {
        xoff[i] = (src_row * K + part * 8) * 2;
      }
    }
    // weight slot q = t + j*threads: row q/2 of the block, group 2c + (q&1) of chunk c
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      int wr = ntile * BN + ((t + j * kThreads) >> 1);
      wr = w13_row(wr < N ? wr : N - 1, N, split);
      if constexpr (kTail) wsrc[j] = args.wblocks + ((size_t)e * N + wr) * (size_t)(K >> 1);
      else woff[j] = wr * (K >> 1) + 16 * wh;
    }
    // NVFP4 scale part j of a group: row t/kSG + j*threads/kSG of the
    // block, dword t%kSG of the group's kSG (fewer than kSG chunks: the
    // dwords past the row's last re-read it)
    if constexpr (kNv) {
      sq0 = ntile * BN + t / kSG;
      sdw = min(t % kSG, nchunks - 1);
    }
    if constexpr (!kTail) {
      rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.wblocks + (size_t)e * N * (K >> 1)), (short)0,
                                             N * (K >> 1), kRawBuffer);
      if (kNv)
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.wscales + (size_t)e * N * (K >> 4)),
                                               (short)0, N * (K >> 4), kRawBuffer);
    }
  };
  setup();
  auto buf_lds = [](__amdgpu_buffer_rsrc_t r, void* lds, int bytes, int voff, int soffs) {
    if (bytes == 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soffs, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soffs, 0, 0);
  };

  // chunk c (the last chunk again past the end) into stage st; lane l of the
  // wave lands in slot wave*64 + l (+ i*threads), as the register path stores it
  auto issue = [&](int c, int st) {
    c = c < nchunks ? c : nchunks - 1;
    u32x4* xs = arena + st * kStage + wave * 64;
    u32x4* ws = xs + kXSlots;
    if (!kTail) {
#pragma unroll
      for (int i = 0; i < kXPer; ++i) buf_lds(rx, xs + i * kThreads, 16, xoff[i], c * 128);
#pragma unroll
      for (int j = 0; j < kWPer; ++j) buf_lds(rw, ws + j * kThreads, 16, woff[j], c * 32);
      return;
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      // K tail: the missing half chunk re-reads the first half (its weights are zero)
      const int koff = c * 64 + xcol[i] < K ? c * 64 : c * 64 - 32;
      load_lds16(xsrc[i] + koff, xs + i * kThreads);
    }
    int g = 2 * c + wh;
    g = g < kgroups ? g : g - 1;
#pragma unroll
    for (int j = 0; j < kWPer; ++j) load_lds16(wsrc[j] + (size_t)g * 16, ws + j * kThreads);
  };
  // NVFP4: first chunk of scale group g in the ring (the last group re-reads
  // earlier chunks so that its kSG dwords stay in the row)
  auto group_start = [&](int g) { return max(0, min(kSG * g, nchunks - kSG)); };
  // part j of scale group g into its ring slot (g & 1); lane l of the wave
  // lands at dword wave*64 + l (+ j*threads) of the slot: row (that index)/kSG
  auto issue_scales = [&](int g, int j) {
    uint32_t* const dst =
        reinterpret_cast<uint32_t*>(sst + (g & 1) * (BN * 4 * kSG)) + j * kThreads + wave * 64;
    const int c0 = group_start(g);
    if constexpr (!kTail) {
      // rows past N read past the expert's scale range (zero; their outputs
      // are dropped) or another of its rows (split layout)
      const int step = (split ? kThreads / (2 * kSG) : kThreads / kSG) * (K >> 4);  // part j+1's rows
      buf_lds(rs, dst, 4, w13_row(sq0, N, split) * (K >> 4) + 4 * sdw, j * step + 4 * c0);
    } else {
      const int r = sq0 + j * (kThreads / kSG);
      const int wr = w13_row(r < N ? r : N - 1, N, split);
      load_lds4(args.wscales + ((size_t)e * N + wr) * (size_t)(K >> 4) + 4 * (c0 + sdw), dst);
    }
  };

  // a job's lane quantities and LDS read positions, derived for every job
  // (before its first loads, or after the previous job's epilogue) from an
  // opaque copy of the lane (as in setup()), so that they are not held
  // through the epilogue
  int half, lrow, wslot0, nvs0;
  const uint8_t* srow;
  int n_wave;
  const int m_wave = wm * RM * 32;
  bool live;
  auto setup_rows = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    half = l >> 5;
    lrow = l & 31;
    wslot0 = (wn * RN * 32 + lrow) * 2 + half;
    // NVFP4: byte offset in a ring slot of this lane's two scale bytes (group 2c + half) of its
    // first row, chunk 0 of the slot's group
    nvs0 = (wn * RN * 32 + lrow) * (4 * kSG) + 2 * half;
    srow = sst + staged_row(wn * RN * 32 + lrow, min(BN, N - ntile * BN), split) * kgroups;
    n_wave = ntile * BN + wn * RN * 32;
    // wave-uniform: the wave holds some of the tile's pairs (a tile holds at
    // least one) and some rows below N (the last row tile of a GEMM leaves
    // whole waves past N: they issue their share of the loads but convert
    // and multiply nothing; 3-5 us less for the down GEMM's full tiles of a
    // 4096-token gpt-oss-120b prefill)
    live = (WM == 1 || m_wave < count) && n_wave < N;
  };
  const int rb_stride = (split ? 16 : 32) * kgroups;

  f32x16 acc[RN][RM];
  auto clear_acc = [&]() {
#pragma unroll
    for (int rb = 0; rb < RN; ++rb)
#pragma unroll
      for (int cb = 0; cb < RM; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
  };
  // MXFP4 gate_up: the sums start at their rows' biases (nothing scales them
  // afterwards), so the epilogue adds none.  The block's biases travel to LDS
  // behind its scale rows with the scale table (bias rows as in memory: the
  // block's rows, or its gate rows then its up rows), and each wave starts
  // its accumulators from them once the first chunk has landed.  Loaded into
  // registers instead, they would make the compiler wait for every load in
  // flight before their first use.  They need K <= 4032 (room behind the
  // scale rows) and a 16-byte aligned bias array; otherwise the sums start at
  // zero and the epilogue adds the biases.
  constexpr bool kBiasInAcc = kGateUp && !kNv && !kPersist;
  const bool bias_lds = kBiasInAcc && kgroups + 2 <= kWideMaxGroups && (reinterpret_cast<uintptr_t>(args.bias) & 15) == 0;
  uint8_t* const sbias = sst + BN * kgroups;
  auto stage_bias = [&]() {
    const int nv = min(BN, N - ntile * BN);
    const int n16 = nv >> 3;  // 16-byte pieces, at most 64: wave 0's lanes
    const int h = split ? n16 >> 1 : n16;
    const u32x4* g = reinterpret_cast<const u32x4*>(args.bias + (size_t)e * N + (split ? ntile * BN / 2 : ntile * BN));
    const u32x4* u = reinterpret_cast<const u32x4*>(args.bias + (size_t)e * N + N / 2 + ntile * BN / 2);
    if (t < n16) load_lds16(t < h ? g + t : u + (t - h), reinterpret_cast<u32x4*>(sbias));
  };
  auto init_acc_from_lds = [&]() {
    const int nv = min(BN, N - ntile * BN);
#pragma unroll
    for (int rb = 0; rb < RN; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = wn * RN * 32 + rb * 32 + 8 * i + 4 * (lane >> 5);  // block-local, a multiple of 4
        const int a0 = split ? n : 2 * n, a1 = split ? nv + n : 2 * n + 4;
        const uint2 raw{*reinterpret_cast<const uint32_t*>(sbias + a0), *reinterpret_cast<const uint32_t*>(sbias + a1)};
        const f32x4 bv = bias4_of(raw, split);
#pragma unroll
        for (int cb = 0; cb < RM; ++cb)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[rb][cb][4 * i + j] = bv[j];
      }
  };
  if (!bias_lds) clear_acc();

  // the operands of one chunk in registers, as read (nothing computed from
  // them until the chunk runs, a chunk later)
  struct Ops {
    u32x4 w[RN];
    uint32_t sb[RN];  // E8M0 scale byte (NVFP4: the group's two E4M3 bytes, low byte first)
    bf16x8 b[4][RM];
  };
  auto read_scale = [&](int c, int rb) -> uint32_t {
    if (kNv) {
      const int g = c / kSG;
      const uint8_t* ss = sst + (g & 1) * (BN * 4 * kSG) + 4 * (c - group_start(g));
      return *reinterpret_cast<const uint16_t*>(ss + nvs0 + rb * (32 * 4 * kSG));
    }
    const int g = 2 * c + half;
    return srow[rb * rb_stride + (!kTail || g < kgroups ? g : g - 1)];
  };
  // load k (0 .. kLoads-1) of chunk c into stage st
  auto issue_one = [&](int c, int st, int k) {
    c = c < nchunks ? c : nchunks - 1;
    u32x4* xs = arena + st * kStage + wave * 64;
    if (k < kXPer) {
      if (!kTail) {
        buf_lds(rx, xs + k * kThreads, 16, xoff[k], c * 128);
      } else {
        const int koff = c * 64 + xcol[k] < K ? c * 64 : c * 64 - 32;
        load_lds16(xsrc[k] + koff, xs + k * kThreads);
      }
    } else {
      if (!kTail) {
        buf_lds(rw, xs + kXSlots + (k - kXPer) * kThreads, 16, woff[k - kXPer], c * 32);
      } else {
        int g = 2 * c + wh;
        g = g < kgroups ? g : g - 1;
        load_lds16(wsrc[k - kXPer] + (size_t)g * 16, xs + kXSlots + (k - kXPer) * kThreads);
      }
    }
  };
  // LDS read j of chunk c's operands (weights, scale bytes, token fragments) from stage st
  constexpr int kReads = 2 * RN + 4 * RM;
  auto read_one = [&](Ops& o, int c, int st, int j) {
    c = c < nchunks ? c : nchunks - 1;
    const u32x4* xs = arena + st * kStage;
    if (j < RN) {
      o.w[j] = xs[kXSlots + wslot0 + j * 64];
    } else if (j < 2 * RN) {
      o.sb[j - RN] = read_scale(c, j - RN);
    } else {
      const int s = (j - 2 * RN) / RM, cb = (j - 2 * RN) % RM;
      const int row = cb * 32 + lrow;
      o.b[s][cb] = __builtin_bit_cast(bf16x8, xs[m_wave * 8 + row * 8 + slot_col(row, half * 4 + s)]);
    }
  };
  // conversion operands of a fragment's scale byte(s) (see chunk_mma_regs)
  auto scales_of = [](uint32_t sb, float& lo, float& hi) {
    if (kNv) {
      const mx::f32x2p v = mx::e4m3x2_operands(sb);
      lo = v.x;
      hi = v.y;
    } else {
      lo = hi = mx::e8m0_operand(sb);
    }
  };
  // Chunk c sits in LDS stage (c + kStages - 1) % kStages, so that chunk 0 of
  // a persistent block's next job goes to the last stage: the epilogue's
  // regions use only the stages below it (and the scale table is no longer
  // read then), so the next job's scale table and first chunk load while this
  // job's epilogue runs; its second chunk follows once the epilogue is done.
  constexpr int kNext = kStages - 1;  // stage of chunk 0
  static_assert(!kPersist || WN * WM * RM * 32 * 128 <= kNext * kStage * 16,
                "the epilogue regions stay below the next job's first stage");
  setup_rows();
  if (!kNv) stage_scales<BN, kThreads, true>(sst, args.wscales, args.N, e, ntile, kgroups, t, split);
  if (bias_lds) stage_bias();
  if constexpr (kNv) {
#pragma unroll
    for (int j = 0; j < kSG; ++j) issue_scales(0, j);
  }
  issue(0, kNext);
  auto issue_rest = [&]() { issue(1, (1 + kNext) % kStages); };  // the job's second chunk
  issue_rest();
  while (true) {
    // chunk c from stage st: read after the barrier that makes it visible
    // (the other wave on the SIMD covers the wait); chunk c+2 into stage
    // (st + 2) % kStages, its loads spread between the MFMAs
    // rml_c: the wave's live token blocks (RML of RM; see live_blocks below)
    auto step1 = [&](int c, int st, auto rml_c) {
      constexpr int RML = decltype(rml_c)::value;
      wait_loads_then_barrier<kLoads>();  // chunk c landed; chunk c+1 may be in flight
      Ops cur;
      if (live) {
#pragma unroll
        for (int j = 0; j < 2 * RN; ++j) read_one(cur, c, st, j);
#pragma unroll
        for (int j = 0; j < 4 * RML; ++j) read_one(cur, c, st, 2 * RN + (j / RML) * RM + j % RML);
      }
      if constexpr (kStages == 2) lds_reads_then_barrier();  // chunk c+2 overwrites chunk c
      if (live) {
        // NVFP4: part c%kSG of the next scale group first, so that the
        // waits, which leave the last kLoads loads in flight, cover it
        constexpr int kIssue = kLoads + (kNv ? 1 : 0);
        constexpr int kMfma = 4 * RN * RML;
        constexpr int kEvery = kMfma / kIssue >= 2 ? 2 : 1;
        static_assert(kEvery * kIssue <= kMfma, "room between the MFMAs");
        auto extra = [&](int k) {
          if (k % kEvery != 0 || k / kEvery >= kIssue) return;
          const int i = k / kEvery;
          if (kNv && i == 0) issue_scales(c / kSG + 1, c % kSG);
          else issue_one(c + 2, (st + 2) % kStages, i - (kNv ? 1 : 0));
          __builtin_amdgcn_sched_barrier(0);
        };
        const bool glive = !kTail || 2 * c + half < kgroups;
        u32x4 w[RN];
        float sc[RN], sc_hi[RN];
        uint32_t mt[RN], mt_hi[RN];
#pragma unroll
        for (int rb = 0; rb < RN; ++rb) {
          w[rb] = glive ? cur.w[rb] : u32x4{0u, 0u, 0u, 0u};
          scales_of(cur.sb[rb], sc[rb], sc_hi[rb]);
          if constexpr (kF16In) {
            mx::split_scale_f16(sc[rb], sc[rb], mt[rb]);
            mx::split_scale_f16(sc_hi[rb], sc_hi[rb], mt_hi[rb]);
          }
        }
        chunk_mma_regs<RN, RM, kNv, kF16In, RML>(acc, cur.b, w, sc, sc_hi, extra, mt, mt_hi);
      } else {
        if constexpr (kNv) issue_scales(c / kSG + 1, c % kSG);
        issue(c + 2, (st + 2) % kStages);
      }
    };
    // The K loop, in one form per count of live token blocks: in a tile's
    // last, partial job the blocks past its pairs are neither read nor
    // multiplied (wave-uniform, chosen once per job; every form runs the
    // same loads and barriers).
    const int nfull = nchunks / kStages * kStages;
    auto k_loop = [&](auto rml_c) {
      if (bias_lds) {
        wait_loads_then_barrier<kLoads>();  // chunk 0 (and the biases) landed
        init_acc_from_lds();
      }
      for (int c0 = 0; c0 < nfull; c0 += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u) step1(c0 + u, (u + kNext) % kStages, rml_c);
      }
#pragma unroll
      for (int u = 0; u < kStages - 1; ++u)
        if (nfull + u < nchunks) step1(nfull + u, (u + kNext) % kStages, rml_c);
    };
    const int live_blocks = __builtin_amdgcn_readfirstlane(min(RM, max(0, (count - m_wave + 31) >> 5)));
    if (RM >= 4 && live_blocks == 3) k_loop(std::integral_constant<int, (RM >= 4 ? 3 : RM)>{});
    else if (RM >= 3 && live_blocks == 2) k_loop(std::integral_constant<int, (RM >= 3 ? 2 : RM)>{});
    else if (RM >= 2 && live_blocks == 1) k_loop(std::integral_constant<int, 1>{});
    else k_loop(std::integral_constant<int, RM>{});
    // the chunks issued past the end land before the arena is reused
    wait_loads_then_barrier<0>();
    // this job's epilogue values; the next job (if any) is set up and its
    // scale table and first chunk requested before the epilogue runs
    const int e_j = e, row0_j = row0, count_j = count;
    vb += gridDim.x;
    // (only a down GEMM fast form at one block per CU walks several jobs)
    const bool more = kPersist && map_job(vb, num_tiles, n_tiles, tile, ntile);
    if (more) {
      setup();
      if (!kNv) stage_scales<BN, kThreads, true>(sst, args.wscales, args.N, e, ntile, kgroups, t, split);
      issue(0, kNext);
    }
    uint8_t* region = reinterpret_cast<uint8_t*>(arena) + wave * (RM * 32 * 128);
    int lane_j = lane;  // opaque copy, as in setup()
    asm volatile("" : "+v"(lane_j));
    if (live)
      store_epilogue<RN, RM, kGateUp, kNv, kF16Out>(args, acc, e_j, row0_j + m_wave, count_j - m_wave, n_wave, lane_j,
                                                    region, !bias_lds);
    if (!more) break;
    __syncthreads();  // every wave is done with the epilogue regions (stages 0 and 1)
    setup_rows();
    issue_rest();
    clear_acc();
  }
}

template <int WN, int WM, int RN, int RM, bool kGateUp, bool kNv = false, int kStageCount = 3, int kBlocksPerCu = 1>
hipError_t launch_wide(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  constexpr int BN = WN * RN * 32;
  const long n_tiles = (a.N + BN - 1) / BN;
  const long blocks = n_tiles * a.max_tiles;
  if (blocks == 0) return hipSuccess;
  if (kNv && (a.K & 63) != 0) return hipErrorInvalidValue;  // NVFP4 full tiles: whole 64-wide chunks only
  // the fast form: whole 64-wide chunks and 32-bit buffer offsets
  const bool fast = (a.K & 63) == 0 && a.act_rows * a.K * 2 < ((int64_t)1 << 31) &&
                    (int64_t)a.N * (a.K >> 1) < ((int64_t)1 << 31);
  // one block per job; the down GEMM's fast form instead runs one block per
  // CU (a multiple of the XCD count), each walking its jobs, so that a job's
  // first loads fly during the previous job's epilogue
  long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  const long cus = (long)mxfp4moe::device_cu_count() / kXcds * kXcds;
  constexpr int kStage16 = (WM * RM * 32) * 8 + BN * 2;  // the kernel's kStage
  constexpr bool kPersistent = wide_persistent<WN, WM, RN, RM, kGateUp, kBlocksPerCu, kStage16>();
  if (fast && kPersistent && cus >= kXcds && grid > cus) grid = cus;
  if (fast)
    expert_wide_kernel<WN, WM, RN, RM, kGateUp, kNv, false, kStageCount, kBlocksPerCu>
        <<<(unsigned)grid, WN * WM * 64, 0, stream>>>(a);
  else
    expert_wide_kernel<WN, WM, RN, RM, kGateUp, kNv, true, kStageCount, kBlocksPerCu>
        <<<(unsigned)grid, WN * WM * 64, 0, stream>>>(a);
  return hipGetLastError();
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
  stage_scales<BN, kThreads, true>(sst, args.wscales, args.N, e, ntile, kgroups, t, split);

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

// kRoute (gate_up of a decode batch): the block routes and groups the batch
// itself before it knows its tile (route_group_small, in LDS past the
// regions above), so no routing launch runs before this one.
template <int RN, bool kNv = false, int kKSplit = 1>
__host__ __device__ constexpr size_t stream_route_offset(int K) {
  return (stream_lds_bytes<RN, kNv, kKSplit>(K) + 15) / 16 * 16;
}

template <int RN, int kBatch, bool kGateUp, bool kNv, int kKSplit = 1, bool kRoute = false>
__global__ __launch_bounds__(256, 5) void expert_stream_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kThreads = 256;
  constexpr int BN = 64 * RN / kKSplit;
  static_assert(kKSplit == 1 || kKSplit == 2, "one or two K parts");
  static_assert(!kRoute || kGateUp, "routing in the gate_up launch only");
  extern __shared__ u32x4 dyn[];
  uint8_t* const lds = reinterpret_cast<uint8_t*>(dyn);

  const int N = args.N, K = args.K;
  const int n_tiles = (N + BN - 1) / BN;
  int tile, ntile;
  int4 tl;
  mxroute::SmallRoute* const sr = reinterpret_cast<mxroute::SmallRoute*>(lds + stream_route_offset<RN, kNv, kKSplit>(K));
  if constexpr (kRoute) {
    mxroute::route_group_small(*sr, args.route_logits, args.route_T, args.route_E, args.top_k, blockIdx.x == 0,
                               args.route_ids, args.route_weights, args.route_offsets, args.route_sorted,
                               reinterpret_cast<int4*>(args.route_tiles), args.route_counts);
    if (!map_block(sr->num_active, n_tiles, tile, ntile)) return;  // uniform per block
    tl = sr->tiles[tile];
  } else {
    if (!map_block(*args.num_tiles, n_tiles, tile, ntile)) return;  // uniform per block
    tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  }
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
      const int pr = kRoute ? sr->sorted[row0 + rr] : kGateUp ? args.sorted_pairs[row0 + rr] : 0;
      xsrc[r] = (kGateUp ? (size_t)(pr / args.top_k) : (size_t)(row0 + rr)) * (size_t)K;
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
    stage_scales<BN, kThreads>(sl, args.wscales, args.N, e, ntile, kNv ? 2 * kgroups : kgroups, t, split);
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
  if constexpr (kGateUp) {
    if (a.route_logits != nullptr) {  // the decode batch routed inside the launch
      constexpr size_t kRouteLds = sizeof(mxroute::SmallRoute);
      static const hipError_t attr_r = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&expert_stream_kernel<RN, kBatch, kGateUp, kNv, kKSplit, true>),
          hipFuncAttributeMaxDynamicSharedMemorySize,
          (int)(stream_route_offset<RN, kNv, kKSplit>(mxfp4moe::kMaxHidden) + kRouteLds));
      if (attr_r != hipSuccess) return attr_r;
      expert_stream_kernel<RN, kBatch, kGateUp, kNv, kKSplit, true>
          <<<(unsigned)grid, 256, stream_route_offset<RN, kNv, kKSplit>(a.K) + kRouteLds, stream>>>(a);
      return hipGetLastError();
    }
  }
  const size_t lds = stream_lds_bytes<RN, kNv, kKSplit>(a.K);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&expert_stream_kernel<RN, kBatch, kGateUp, kNv, kKSplit>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)stream_lds_bytes<RN, kNv, kKSplit>(mxfp4moe::kMaxHidden));
  if (attr != hipSuccess) return attr;
  expert_stream_kernel<RN, kBatch, kGateUp, kNv, kKSplit><<<(unsigned)grid, 256, lds, stream>>>(a);
  return hipGetLastError();
}

// Mid-size tiles (kStreamTokens < pairs, at most kMidTokens = 48 per tile):
// the per-expert remainders of prefill.  16x16x32 MFMA (A: lane (r, q) takes
// group 4c+q of row r, step s its codes [8s, 8s+8), so K = 128c + 32q + 8s + i;
// B: the same K values of token l%16).  A block owns 128 weight rows (four
// waves of 2 x 16 rows) and up to 48 tokens (three 16-token column blocks).  K
// runs in panels of one chunk (128 K).  Each wave loads its own weights
// straight into the A operand's registers (lane (r, q) the 16 bytes of group
// 4c+q of its row: the four lanes of a row read its 64 contiguous bytes of
// the panel, the pattern HBM streams at full rate); the tile's token rows
// (256 bytes each per panel) are shared by the four waves through LDS.  kS
// register slots (see mid_slots) each
// hold the loads of one panel's weights (used by that panel's MFMAs, then
// refilled with the panel kS ahead) and one panel's tokens (stored to the
// single LDS token buffer a panel before they are used, then refilled): per
// panel, after its MFMAs and a barrier, the next panel's tokens are stored,
// their slot refilled, and a second barrier makes them visible.  The token
// bytes of a panel (at most 12 KB, from L2) are at most 1.5 times its weight
// bytes (8 KB, from HBM), which is what lets the slots fit in registers
// at three or four blocks per CU (with 64-token tiles they did not).  The loop body
// is kS panels of straight-line code with the same loads in flight at entry
// and at the back edge (the compiler then waits for each slot alone); panels
// past the last re-read the last one (in bounds, never computed).  Token
// rows past the tile's pairs re-read its first pair (their outputs are
// dropped).
//
// Dynamic LDS: tokens [48][256 + 16] | scales [128][K/32] (the 16-byte row
// pad makes the 16-lane column reads conflict-free).
template <bool kNv = false>
__host__ __device__ constexpr size_t mid_lds_bytes(int K) {
  return (size_t)mxfp4moe::kMidTokens * (256 + 16) + (size_t)128 * (K / (kNv ? 16 : 32));
}

// Register slots of panel loads: two, at four blocks per CU (126-128
// registers).  Measured against three slots at three blocks per CU: 20b
// prefill 0.156 against 0.159 ms (mid gate_up 98 against 102 us), NVFP4 0.167
// against 0.171 ms, the 120b long prefill within noise (MXFP4 mid down 74.4-
// 74.8 against 76.6-76.9 us when it alone changed).
template <bool kGateUp, bool kNv>
constexpr int mid_slots() { return 2; }
template <bool kGateUp, bool kNv>
__global__ __launch_bounds__(256, (mid_slots<kGateUp, kNv>() == 2 ? 4 : 2)) void expert_mid_kernel(mxfp4moe::GemmArgs args) {
  constexpr int kS = mid_slots<kGateUp, kNv>();
  constexpr int kThreads = 256;
  constexpr int BN = 128;
  constexpr int BM = mxfp4moe::kMidTokens;
  constexpr int kCB = BM / 16;  // 16-token column blocks
  static_assert(BM % 16 == 0 && kCB <= 4, "16-token column blocks");
  constexpr int kXRow = 256 + 16;     // LDS bytes per token row of a panel
  constexpr int kXPieces = 16;        // 16-byte pieces per token row of a panel
  constexpr int kXPer = BM * kXPieces / kThreads;
  static_assert(BM * kXPieces % kThreads == 0 && BN == 4 * 32, "panel / thread mismatch");
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
  const int npanels = (kgroups + 3) >> 2;
  const int k16 = K >> 3;   // 16-byte pieces of a token row
  const int kg16 = K >> 5;  // 16-byte pieces (groups) of a weight row
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int q = lane >> 4;
  const int lr = lane & 15;

  uint8_t* const xs = lds;
  uint8_t* const sl = lds + BM * kXRow;
  const bool split = kGateUp && args.split_gate_up;  // uniform
  stage_scales<BN, kThreads>(sl, args.wscales, args.N, e, ntile, kNv ? 2 * kgroups : kgroups, t, split);

  // load slots: token piece i = t + j*256 -> token i / 16; weight piece
  // i = t + j*256 -> row i / 4 (rows past N re-read row N-1)
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
  // weights straight into the MFMA's A operand: lane (lr, q) of row block rb
  // loads group 4p + q of its row (the four lanes of a row read its 64
  // contiguous bytes of the panel; rows past N re-read row N-1)
  const u32x4* wsrc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int gr = w13_row(min(ntile * BN + wave * 32 + rb * 16 + lr, N - 1), N, split);
    wsrc[rb] = reinterpret_cast<const u32x4*>(args.wblocks + ((size_t)e * N + gr) * (size_t)(K >> 1));
  }
  // Three register slots of panel loads each for the weights (consumed by a
  // panel's MFMAs) and the tokens (consumed when stored to LDS, a panel
  // earlier).  Groups / pieces past the end re-read the last one (finite;
  // the weights of a missing group are zeroed at use); panels past the last
  // re-read the last panel.
  u32x4 xv[kS][kXPer], wv[kS][2];
  auto issue_w = [&](int p, int sl3) {
    p = min(p, npanels - 1);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) wv[sl3][rb] = wsrc[rb][min(4 * p + q, kg16 - 1)];
  };
  auto issue_x = [&](int p, int sl3) {
    p = min(p, npanels - 1);
#pragma unroll
    for (int j = 0; j < kXPer; ++j) xv[sl3][j] = xsrc[j][min(p * kXPieces + xpiece[j], k16 - 1)];
  };
  // every token row is stored (rows past the tile's pairs hold its first
  // pair's values, never read for an output): no branch between the loads
  // and their uses
  auto commit = [&](int sl3) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) *reinterpret_cast<u32x4*>(xs + xdst[j]) = xv[sl3][j];
  };

  const int n_wave = ntile * BN + wave * 32;
  const uint8_t* srow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
    srow[rb] = sl + staged_row(wave * 32 + rb * 16 + lr, min(BN, N - ntile * BN), split) * (kNv ? 2 : 1) * kgroups;
  const int ncb = (count + 15) >> 4;  // live 16-token column blocks
  // LDS byte offset of this lane's token row in column block 0 (block cb adds
  // a constant; rows past the tile's pairs hold its first pair, finite)
  const int xrd = lr * kXRow + 64 * q;
  f32x4 acc[2][kCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the MFMAs of panel p: weights from register slot sl3, tokens from LDS
  auto compute = [&](int p, int sl3) {
    const int g0 = 4 * p + q;
    const bool glive = g0 < kgroups;
    const int g = glive ? g0 : kgroups - 1;
    u32x4 a[2][4];  // [rb][step] converted A fragments
    // both row blocks' scale bytes read together
    const u32x4* const wr = wv[sl3];
    uint32_t sb[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
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
    for (int cb = 0; cb < kCB; ++cb) {
      if (cb < ncb) {  // wave-uniform: a column block past the tile's pairs is skipped
        // the block's four token fragments read together, then its MFMAs
        bf16x8 bb[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
          bb[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + xrd + cb * 16 * kXRow + 16 * st));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mx::as_bf16x8(a[rb][st]), bb[st], acc[rb][cb], 0, 0, 0);
        }
      }
    }
  };
  // after the MFMAs of panel p (weights from slot p % 3, now free: refilled
  // with panel p + 3): every wave is done with the LDS buffer, the next
  // panel's token slot `nx` is stored, refilled with panel `ahead`, and the
  // stored panel made visible
  auto advance = [&](int p, int nx, int ahead) {
    issue_w(p + kS, p % kS);
    __syncthreads();
    commit(nx);
    issue_x(ahead, nx);
    __syncthreads();
  };

#pragma unroll
  for (int j = 0; j < kS; ++j) {
    issue_w(j, j);
    issue_x(j, j);
  }
  commit(0);
  issue_x(kS, 0);
  __syncthreads();  // panel 0's tokens and the scale rows staged; the next panels in flight
  int p = 0;
  for (; p + kS <= npanels; p += kS) {
#pragma unroll
    for (int u = 0; u < kS; ++u) {
      compute(p + u, u);
      advance(p + u, (u + 1) % kS, p + u + kS + 1);
    }
  }
  // the last kS - 1 panels at most (slots 0, 1, ... hold them, in order)
  if (p < npanels) compute(p, 0);
  if (kS == 3 && p + 1 < npanels) {
    advance(p, 1, p + 4);
    compute(p + 1, 1 % kS);
  }

  if (n_wave >= N) return;
  const uint16_t* bias = args.bias + (size_t)e * N;
  const float s2 = kNv ? args.scale2[e] : 1.0f;  // second-level scale, before the bias
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int n = n_wave + rb * 16 + 4 * q;  // first of this lane's four rows
    if (n >= N) continue;
    const f32x4 bv = load_bias4(bias, n, N, split);
    const float b0 = bv[0], b1 = bv[1], b2 = bv[2], b3 = bv[3];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int m = cb * 16 + lr;
      if (m >= count) continue;
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

template <bool kGateUp, bool kNv>
hipError_t launch_mid(const mxfp4moe::GemmArgs& a, hipStream_t stream) {
  const long n_tiles = (a.N + 127) / 128;
  const long blocks = n_tiles * a.max_tiles;
  if (blocks == 0) return hipSuccess;
  const long grid = (blocks + kXcds - 1) / kXcds * kXcds;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_mid_kernel<kGateUp, kNv>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)mid_lds_bytes<kNv>(mxfp4moe::kMaxHidden));
  if (attr != hipSuccess) return attr;
  expert_mid_kernel<kGateUp, kNv><<<(unsigned)grid, 256, mid_lds_bytes<kNv>(a.K), stream>>>(a);
  return hipGetLastError();
}

// y[t, n] = bf16(sum_j zw[t*k + j, n]) summed in fp32, j ascending, over the
// bf16 pair outputs; eight features per thread.  kK > 0: top_k == kK, all k
// rows loaded before the sum (one round trip instead of k); kK == 0: any k.
template <int kK>
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
  auto add = [&](const u32x4& v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[2 * i] += mx::bf16_to_f32(v[i] & 0xffffu);
      s[2 * i + 1] += mx::bf16_to_f32(v[i] >> 16);
    }
  };
  if constexpr (kK > 0) {
    u32x4 v[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) v[j] = *reinterpret_cast<const u32x4*>(src + (size_t)j * H);
#pragma unroll
    for (int j = 0; j < kK; ++j) add(v[j]);
  } else {
    for (int j = 0; j < top_k; ++j) add(*reinterpret_cast<const u32x4*>(src + (size_t)j * H));
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
// mid: 16x16x32 MFMA, 4 waves of 32 weight rows x (up to) 48 tokens, panels
// of one chunk of both operands staged in LDS, three panels in flight.
// stream: 16x16x32 MFMA, 4 waves of 16*MX_STREAM_RN weight rows x (at most 4)
// tokens, weights streamed in batches of MX_STREAM_BATCH chunks of 128 K.
static_assert(kWideTokens == 128 && kStreamTokens == 4, "tile sizes");

template <bool kGateUp>
static hipError_t launch_all(GemmArgs a, const TileTables& tt, const TileBounds& tb, hipStream_t stream) {
  hipError_t err = hipSuccess;
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
      // Two waves per SIMD, so that one wave's conversions, waits and
      // epilogue run beside the other's MFMAs.  gate_up (MXFP4 and NVFP4) and
      // the NVFP4 down GEMM: two blocks per CU of four waves x (64 rows x 128
      // pairs) (MXFP4 gate_up: two LDS stages beside its scale table, within
      // half the LDS).  MXFP4 down: one persistent block per CU of eight waves
      // x (128 rows x 64 pairs).  Measured at the 120b long prefill: gate_up
      // 444 against 454 us for four waves of 128 x 128 with operands read a
      // chunk ahead (NVFP4 547 against 560); down 221 (persistent) against
      // 229 us in two blocks (NVFP4 297 against 305 the other way round).
      const bool nv = a.scale2 != nullptr;
      if (kGateUp)
        err = nv ? launch_wide<4, 1, 2, 4, true, true, 3, 2>(w, stream)
                 : launch_wide<4, 1, 2, 4, true, false, 2, 2>(w, stream);
      else
        err = nv ? launch_wide<4, 1, 2, 4, false, true, 3, 2>(w, stream)
                 : launch_wide<4, 2, 4, 2, false, false>(w, stream);
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
  const unsigned grid = (unsigned)((n + 255) / 256);
  switch (top_k) {
    case 1: combine_kernel<1><<<grid, 256, 0, stream>>>(zw, y, T, H, top_k); break;
    case 2: combine_kernel<2><<<grid, 256, 0, stream>>>(zw, y, T, H, top_k); break;
    case 4: combine_kernel<4><<<grid, 256, 0, stream>>>(zw, y, T, H, top_k); break;
    case 8: combine_kernel<8><<<grid, 256, 0, stream>>>(zw, y, T, H, top_k); break;
    default: combine_kernel<0><<<grid, 256, 0, stream>>>(zw, y, T, H, top_k); break;
  }
  return hipGetLastError();
}

}  // namespace mxfp4moe
