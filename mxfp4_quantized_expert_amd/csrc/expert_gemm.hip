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

constexpr int kLdsStride = 72;  // bf16 per staged token row: 64 + 8 padding

template <int WN, int WM, int RN, int RM>
struct Shape {
  static constexpr int kWaves = WN * WM;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BN = WN * RN * 32;  // weight rows per block
  static constexpr int BM = WM * RM * 32;  // token columns per block
  static constexpr int kPieces = BM * 8;   // 16-byte pieces of one staged chunk
  static constexpr int kPiecesPerThread = (kPieces + kThreads - 1) / kThreads;
};

__device__ __forceinline__ float swiglu_clamped(float gate, float up) {
  // gpt-oss family constants: alpha 1.702, limit 7; gate clamped from above,
  // up clamped on both sides, +1 after the clamp.
  const float g = fminf(gate, 7.0f);
  const float u = fminf(fmaxf(up, -7.0f), 7.0f);
  return g * (1.0f / (1.0f + __expf(-1.702f * g))) * (u + 1.0f);
}

template <int WN, int WM, int RN, int RM, bool kGateUp>
__global__ __launch_bounds__(WN * WM * 64) void expert_gemm_kernel(
    mxfp4moe::GemmArgs args) {
  using S = Shape<WN, WM, RN, RM>;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][S::BM * kLdsStride];

  const int tile = blockIdx.y;
  if (tile >= *args.num_tiles) return;  // uniform per block
  const int4 tl = reinterpret_cast<const int4*>(args.tiles)[tile];
  const int e = tl.x, row0 = tl.y, count = tl.z;

  const int N = args.N, K = args.K;
  const int kgroups = K >> 5;
  const int nchunks = (kgroups + 1) >> 1;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int lrow = lane & 31;
  const int wn = wave % WN, wm = wave / WN;
  const int n_wave = blockIdx.x * S::BN + wn * RN * 32;
  const int m_wave = wm * RM * 32;
  int cb_live = (count - m_wave + 31) >> 5;  // 32-token blocks of this wave holding tokens
  cb_live = cb_live < 0 ? 0 : (cb_live > RM ? RM : cb_live);

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

  // Token rows this thread stages: piece q = row * 8 + part (16 bytes each).
  const uint16_t* xsrc[S::kPiecesPerThread];
  int xdst[S::kPiecesPerThread];
  int xk[S::kPiecesPerThread];
  bool xval[S::kPiecesPerThread];
#pragma unroll
  for (int i = 0; i < S::kPiecesPerThread; ++i) {
    const int q = threadIdx.x + i * S::kThreads;
    const int r = q >> 3, part = q & 7;
    xval[i] = q < S::kPieces && r < count;
    xdst[i] = r * kLdsStride + part * 8;
    xk[i] = part * 8;
    xsrc[i] = args.act;
    if (xval[i]) {
      size_t src_row;
      if (kGateUp)
        src_row = (size_t)(args.sorted_pairs[row0 + r] / args.top_k);
      else
        src_row = (size_t)(row0 + r);
      xsrc[i] = args.act + src_row * (size_t)K + part * 8;
    }
  }

  u32x4 xstage[S::kPiecesPerThread];
  auto load_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < S::kPiecesPerThread; ++i) {
      if (xval[i]) {
        if (c * 64 + xk[i] < K)
          xstage[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + c * 64);
        else
          xstage[i] = u32x4{0u, 0u, 0u, 0u};  // K tail: half a chunk of zeros
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < S::kPiecesPerThread; ++i)
      if (xval[i]) *reinterpret_cast<u32x4*>(&xs[buf][xdst[i]]) = xstage[i];
  };

  u32x4 wcur[RN], wnxt[RN];
  uint32_t scur[RN], snxt[RN];
  auto load_w = [&](int c, u32x4* w, uint32_t* s) {
    const int g = 2 * c + half;
#pragma unroll
    for (int rb = 0; rb < RN; ++rb) {
      if (g < kgroups) {
        w[rb] = *reinterpret_cast<const u32x4*>(wrow[rb] + (size_t)g * 16);
        s[rb] = srow[rb][g];
      } else {
        w[rb] = u32x4{0u, 0u, 0u, 0u};
        s[rb] = 127u;
      }
    }
  };

  f32x16 acc[RN][RM];
#pragma unroll
  for (int rb = 0; rb < RN; ++rb)
#pragma unroll
    for (int cb = 0; cb < RM; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  load_x(0);
  load_w(0, wcur, scur);
  store_x(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_x(c + 1);
      load_w(c + 1, wnxt, snxt);
    }
    const uint16_t* xb = xs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[RN];
#pragma unroll
      for (int rb = 0; rb < RN; ++rb)
        a[rb] = mx::as_bf16x8(mx::fp4x8_to_bf16x8(wcur[rb][s], mx::e8m0_operand(scur[rb])));
#pragma unroll
      for (int cb = 0; cb < RM; ++cb) {
        if (cb < cb_live) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(
              xb + (m_wave + cb * 32 + lrow) * kLdsStride + half * 32 + s * 8);
#pragma unroll
          for (int rb = 0; rb < RN; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b, acc[rb][cb], 0, 0, 0);
        }
      }
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

  // Epilogue.  Lane holds, for every (rb, cb), token m = m_wave + cb*32 + lrow
  // and features n = n_wave + rb*32 + 8i + 4*half + {0,1,2,3}, i = 0..3.
  const uint16_t* bias = args.bias + (size_t)e * N;
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
            const uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
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
            const uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
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
  dim3 grid((unsigned)((a.N + S::BN - 1) / S::BN), (unsigned)a.max_tiles);
  expert_gemm_kernel<WN, WM, RN, RM, kGateUp><<<grid, S::kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

namespace mxfp4moe {

int gemm_tile_tokens(GemmConfig cfg) { return cfg == kGemmSmall ? Shape<3, 1, 1, 1>::BM : Shape<3, 1, 2, 4>::BM; }

hipError_t launch_gate_up(const GemmArgs& a, GemmConfig cfg, hipStream_t stream) {
  if (a.max_tiles == 0) return hipSuccess;
  ProfileScope prof(kStageGateUp, stream);
  if (cfg == kGemmSmall) return launch_cfg<3, 1, 1, 1, true>(a, stream);
  return launch_cfg<3, 1, 2, 4, true>(a, stream);
}

hipError_t launch_down(const GemmArgs& a, GemmConfig cfg, hipStream_t stream) {
  if (a.max_tiles == 0) return hipSuccess;
  ProfileScope prof(kStageDown, stream);
  if (cfg == kGemmSmall) return launch_cfg<3, 1, 1, 1, false>(a, stream);
  return launch_cfg<3, 1, 2, 4, false>(a, stream);
}

hipError_t launch_combine(const float* zw, uint16_t* y, int T, int H, int top_k, hipStream_t stream) {
  const size_t n = (size_t)T * (H / 4);
  if (n == 0) return hipSuccess;
  ProfileScope prof(kStageCombine, stream);
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(zw, y, T, H, top_k);
  return hipGetLastError();
}

}  // namespace mxfp4moe
