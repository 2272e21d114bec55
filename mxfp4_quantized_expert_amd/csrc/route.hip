// Routing data for the MXFP4 experts: top-k with softmax over the selected
// logits, then the pairs grouped by expert ("Restore GPT-OSS's router-masked
// expert-parallel plan", transformers PR #49431, description: the experts
// consume routing data and route their tokens themselves; "feat(gguf): serve
// gpt-oss gguf checkpoints on gpt_oss", FreeToken PR #838, "What it does":
// expert-ordered views of the tokens).
#include "../../include/mxfp4moe.h"
#include "internal.h"
#include "mx_device.h"

namespace {

constexpr int kRouteThreads = 256;  // four tokens per block, one wave each
constexpr int kPerLane = MXFP4MOE_MAX_EXPERTS / 64;

// Token t, by one wave.  Lane l holds logits l, l+64, ...; k rounds of a
// wave-wide argmax (ties to the lower expert index) pick the experts in
// descending order; lane j keeps the j-th pick.  The softmax runs over the
// picks relative to the largest one.
__device__ void route_row(const float* row, int t, int E, int top_k, int32_t* __restrict__ ids,
                          float* __restrict__ weights, int32_t* ids_copy = nullptr) {
  const int lane = mx::lane_id();
  float v[kPerLane];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = 0.f;
    if (e < E) {
      v[i] = row[e];
      avail |= 1u << i;
    }
  }
  float my_v = 0.f, v0 = 0.f;
  int my_e = 0;
  for (int j = 0; j < top_k; ++j) {
    bool have = false;
    float bv = 0.f;
    int be = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if ((avail >> i) & 1u) {
        if (!have || v[i] > bv) {  // strict: the lower index wins ties inside a lane
          bv = v[i];
          be = lane + 64 * i;
          have = true;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const int oh = __shfl_xor((int)have, off, 64);
      if (oh && (!have || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
        have = true;
      }
    }
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) v0 = bv;
  }
  float ex = lane < top_k ? expf(my_v - v0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_e;
    weights[(size_t)t * top_k + lane] = ex / sum;
    if (ids_copy != nullptr) ids_copy[t * top_k + lane] = my_e;
  }
}

__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int top_k,
                                            int32_t* __restrict__ ids, float* __restrict__ weights) {
  route_row(logits + (size_t)t * E, t, E, top_k, ids, weights);
}

// Router projection fused ahead of the top-k ("feat(gguf): serve gpt-oss gguf
// checkpoints on gpt_oss", FreeToken PR #838: the router is mlp.router, a
// linear layer whose bias is a required tensor):
//   logits[t, e] = sum_h x[t, h] W_r[e, h] + b_r[e]
// for a tile of 16 tokens on the 16x16x32 bf16 MFMA (A: 16 router rows, B:
// the 16 tokens; bf16 products are exact, accumulation is fp32).  Wave w
// takes K quarter w % 4 of the 16-expert blocks w / 4, w / 4 + 4, ... and
// parks its partial sums in LDS; after a barrier the quarters are added in
// order (so the logits do not depend on scheduling), the bias last, and
// written out; then one wave per token routes from the LDS row as
// route_kernel does.
constexpr int kProjTokens = 16;
constexpr int kProjThreads = 1024;
constexpr int kProjWaves = kProjThreads / 64;
constexpr int kProjParts = 4;  // K parts
constexpr int kProjBatch = 8;  // K steps of 32 whose loads are issued together

__global__ __launch_bounds__(kProjThreads) void route_proj_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w,
                                                                   const uint16_t* __restrict__ b, int T, int H,
                                                                   int E, int top_k, float* __restrict__ logits,
                                                                   int32_t* __restrict__ ids,
                                                                   float* __restrict__ weights) {
  extern __shared__ float part[];  // [nq][kProjTokens][E] partial sums, then [kProjTokens][E] logits in part 0
  const int t0 = blockIdx.x * kProjTokens;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int lr = lane & 15;
  const int nk = H >> 5;                    // K steps of 32
  const int neb = (E + 15) >> 4;
  constexpr int nq = kProjParts;
  const int kq = wave % nq;
  const int k_begin = nk * kq / nq, k_end = nk * (kq + 1) / nq;
  const uint16_t* xrow = x + (size_t)min(t0 + lr, T - 1) * H + 8 * q;  // B: token lr, K values 8q..8q+7
  // the bias of the logits this thread adds up after the barrier
  constexpr int kPerThread = kProjTokens * MXFP4MOE_MAX_EXPERTS / kProjThreads;
  float bias[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int i = threadIdx.x + j * kProjThreads;
    bias[j] = i < kProjTokens * E ? mx::bf16_to_f32(b[i % E]) : 0.f;
  }
  for (int eb = wave / nq; eb < neb; eb += kProjWaves / nq) {
    const uint16_t* wrow = w + (size_t)min(eb * 16 + lr, E - 1) * H + 8 * q;  // A: router row lr of the block
    mx::f32x4 acc[2] = {mx::f32x4{0.f, 0.f, 0.f, 0.f}, mx::f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int k0 = k_begin; k0 < k_end; k0 += kProjBatch) {
      mx::u32x4 av[kProjBatch], bv[kProjBatch];
#pragma unroll
      for (int j = 0; j < kProjBatch; ++j) {
        const int kk = min(k0 + j, k_end - 1);  // steps past the quarter re-read its last one (zeroed below)
        av[j] = *reinterpret_cast<const mx::u32x4*>(wrow + (size_t)kk * 32);
        bv[j] = *reinterpret_cast<const mx::u32x4*>(xrow + (size_t)kk * 32);
      }
#pragma unroll
      for (int j = 0; j < kProjBatch; ++j) {
        const mx::u32x4 a = k0 + j < k_end ? av[j] : mx::u32x4{0u, 0u, 0u, 0u};
        acc[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mx::as_bf16x8(a), mx::as_bf16x8(bv[j]), acc[j & 1], 0, 0, 0);
      }
    }
    // lane (lr, q) holds experts eb*16 + 4q + i of token lr
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = eb * 16 + 4 * q + i;
      if (e < E) part[((size_t)kq * kProjTokens + lr) * E + e] = acc[0][i] + acc[1][i];
    }
  }
  __syncthreads();
  const size_t slab = (size_t)kProjTokens * E;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int i = threadIdx.x + j * kProjThreads;
    if (i < kProjTokens * E) {
      float v = part[i];
      for (int pq = 1; pq < nq; ++pq) v += part[pq * slab + i];
      v += bias[j];
      part[i] = v;
      const int t = t0 + i / E;
      if (t < T) logits[(size_t)t * E + i % E] = v;
    }
  }
  __syncthreads();
  for (int tt = wave; tt < kProjTokens; tt += kProjThreads / 64)
    if (t0 + tt < T) route_row(part + (size_t)tt * E, t0 + tt, E, top_k, ids, weights);
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                              int top_k, int32_t* __restrict__ ids,
                                                              float* __restrict__ weights) {
  const int t = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  route_token(logits, t, E, top_k, ids, weights);
}

constexpr int kGroupThreadsMax = 1024;

// Exclusive prefix sum of vals[0..n) into out[0..n) by wave 0; returns the
// total to every thread of the block (after the trailing barrier).
__device__ int block_exclusive_scan_wave0(const int* vals, int* out, int n, int* total_slot) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int e = c0 + lane;
      const int x = e < n ? vals[e] : 0;
      int incl = x;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (e < n) out[e] = carry + incl - x;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) *total_slot = carry;
  }
  __syncthreads();
  return *total_slot;
}

// Single workgroup: histogram of experts, exclusive scan into offsets, a
// stable scatter of pair ids into expert order, and the GEMM tile tables: an
// expert with at least big_tokens pairs goes to wide tiles, one with more than
// kStreamTokens pairs to mid tiles, the rest to one streaming tile.
// The scatter walks the pairs in chunks of the block size; inside a wave the lanes with
// the same expert are found by matching the expert id bit by bit with
// ballots, and the per-wave counts are turned into positions wave by wave, so
// pairs keep ascending id order inside every expert.
// With logits != nullptr the block first routes the T tokens itself (one
// wave per token), saving a launch for small batches, and keeps the routed
// ids in LDS for the histogram and the scatter.
template <int kGroupThreads>
__global__ __launch_bounds__(kGroupThreads) void group_kernel(const float* __restrict__ logits, int T, int top_k,
                                                              float* __restrict__ weights,
                                                              int32_t* __restrict__ ids, int P, int E,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_pairs,
                                                              mxfp4moe::TileTables tt) {
  constexpr int kGroupWaves = kGroupThreads / 64;
  extern __shared__ int smem[];
  int* cnt = smem;                 // [E]
  int* base = cnt + E;             // [E]
  int* tile_base = base + E;       // [E]
  int* ntile = tile_base + E;      // [E]
  int* wave_cnt = ntile + E;       // [kGroupWaves][E]
  int* idl = wave_cnt + kGroupWaves * E;  // [P] the routed ids (fused routing only)
  __shared__ int total_slot;

  const int32_t* idsrc = ids;
  if (logits != nullptr) {
    for (int t = threadIdx.x >> 6; t < T; t += kGroupWaves)
      route_row(logits + (size_t)t * E, t, E, top_k, ids, weights, idl);
    idsrc = idl;  // the block reads the ids it routed from LDS
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += kGroupThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kGroupThreads) atomicAdd(&cnt[idsrc[p]], 1);
  __syncthreads();
  block_exclusive_scan_wave0(cnt, base, E, &total_slot);
  for (int e = threadIdx.x; e < E; e += kGroupThreads) offsets[e] = base[e];
  if (threadIdx.x == 0) offsets[E] = P;

  if (tt.big != nullptr) {
    const int bt = tt.big_tokens;
    constexpr int st = mxfp4moe::kStreamTokens;
    // an expert with at least bt pairs: all its pairs in tiles of bt (the
    // last one partial), so its weights are streamed by one kernel only
    for (int e = threadIdx.x; e < E; e += kGroupThreads)
      ntile[e] = (bt > 0 && !tt.no_wide && cnt[e] >= bt) ? (cnt[e] + bt - 1) / bt : 0;
    __syncthreads();
    const int n_big = block_exclusive_scan_wave0(ntile, tile_base, E, &total_slot);
    if (threadIdx.x == 0) *tt.num_big = n_big;
    for (int e = threadIdx.x; e < E; e += kGroupThreads) {
      for (int i = 0; i < ntile[e]; ++i)
        reinterpret_cast<int4*>(tt.big)[tile_base[e] + i] = int4{e, base[e] + i * bt, min(bt, cnt[e] - i * bt), 0};
    }
    __syncthreads();
    // fewer than bt pairs, more than st: mid tiles of at most mt pairs
    constexpr int mt = mxfp4moe::kMidTokens;
    const bool mid_on = bt > 0 || tt.no_wide;  // else everything in streaming tiles
    for (int e = threadIdx.x; e < E; e += kGroupThreads) {
      const int c = cnt[e];
      ntile[e] = (mid_on && c > st && (tt.no_wide || c < bt)) ? (c + mt - 1) / mt : 0;
    }
    __syncthreads();
    const int n_mid = block_exclusive_scan_wave0(ntile, tile_base, E, &total_slot);
    if (threadIdx.x == 0) *tt.num_mid = n_mid;
    for (int e = threadIdx.x; e < E; e += kGroupThreads) {
      for (int i = 0; i < ntile[e]; ++i)
        reinterpret_cast<int4*>(tt.mid)[tile_base[e] + i] = int4{e, base[e] + i * mt, min(mt, cnt[e] - i * mt), 0};
    }
    __syncthreads();
    // at most st pairs: one streaming tile; without full tiles (bt == 0),
    // every pair in streaming tiles of st
    for (int e = threadIdx.x; e < E; e += kGroupThreads) {
      const int c = cnt[e];
      ntile[e] = mid_on ? (c > 0 && c <= st ? 1 : 0) : (c + st - 1) / st;
    }
    __syncthreads();
    const int n_small = block_exclusive_scan_wave0(ntile, tile_base, E, &total_slot);
    if (threadIdx.x == 0) *tt.num_small = n_small;
    for (int e = threadIdx.x; e < E; e += kGroupThreads) {
      for (int i = 0; i < ntile[e]; ++i)
        reinterpret_cast<int4*>(tt.small)[tile_base[e] + i] = int4{e, base[e] + i * st, min(st, cnt[e] - i * st), 0};
    }
  }

  const int wave = threadIdx.x >> 6;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  for (int c0 = 0; c0 < P; c0 += kGroupThreads) {
    for (int i = threadIdx.x; i < kGroupWaves * E; i += kGroupThreads) wave_cnt[i] = 0;
    __syncthreads();
    const int p = c0 + threadIdx.x;
    const bool valid = p < P;
    const int e = valid ? idsrc[p] : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      match &= bit ? ones : ~ones;
    }
    const int rank = mx::lanes_below(match);
    if (valid && rank == 0) wave_cnt[wave * E + e] = __popcll(match);
    __syncthreads();
    for (int ee = threadIdx.x; ee < E; ee += kGroupThreads) {
      int run = base[ee];
      for (int w = 0; w < kGroupWaves; ++w) {
        const int c = wave_cnt[w * E + ee];
        wave_cnt[w * E + ee] = run;
        run += c;
      }
      base[ee] = run;
    }
    __syncthreads();
    if (valid) sorted_pairs[wave_cnt[wave * E + e] + rank] = p;
    __syncthreads();
  }
}

}  // namespace

namespace mxfp4moe {

hipError_t launch_route(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                        hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int per_block = kRouteThreads / 64;
  const unsigned grid = (unsigned)((T + per_block - 1) / per_block);
  ProfileScope prof(kStageRoute, stream);
  route_kernel<<<grid, kRouteThreads, 0, stream>>>(logits, T, E, top_k, ids, weights);
  return hipGetLastError();
}

hipError_t launch_route_proj(const uint16_t* x, const uint16_t* router_w, const uint16_t* router_b, int T, int H,
                             int E, int top_k, float* logits, int32_t* ids, float* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const size_t lds = (size_t)kProjParts * kProjTokens * E * sizeof(float);
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&route_proj_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)((size_t)kProjParts * kProjTokens * MXFP4MOE_MAX_EXPERTS * sizeof(float)));
  if (attr != hipSuccess) return attr;
  ProfileScope prof(kStageRoute, stream);
  route_proj_kernel<<<(unsigned)((T + kProjTokens - 1) / kProjTokens), kProjThreads, lds, stream>>>(
      x, router_w, router_b, T, H, E, top_k, logits, ids, weights);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const TileTables& tt, hipStream_t stream) {
  constexpr int kThreads = kGroupThreadsMax;
  const size_t smem = (size_t)(4 + kThreads / 64) * E * sizeof(int);
  ProfileScope prof(kStageGroup, stream);
  group_kernel<kThreads><<<1, kThreads, smem, stream>>>(nullptr, 0, 1, nullptr, const_cast<int32_t*>(ids), P, E,
                                                   offsets, sorted_pairs, tt);
  return hipGetLastError();
}

hipError_t launch_route_group(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                              int32_t* offsets, int32_t* sorted_pairs, const TileTables& tt, hipStream_t stream) {
  // small batches: four waves (cheaper barriers and scans); the routed ids stay in LDS
  const int P = T * top_k;
  ProfileScope prof(kStageGroup, stream);
  if (P <= 256) {
    const size_t smem = (size_t)(4 + 4) * E * sizeof(int) + (size_t)P * sizeof(int);
    group_kernel<256><<<1, 256, smem, stream>>>(logits, T, top_k, weights, ids, P, E, offsets, sorted_pairs, tt);
  } else {
    const size_t smem = (size_t)(4 + kGroupThreadsMax / 64) * E * sizeof(int) + (size_t)P * sizeof(int);
    group_kernel<kGroupThreadsMax><<<1, kGroupThreadsMax, smem, stream>>>(logits, T, top_k, weights, ids, P, E,
                                                                          offsets, sorted_pairs, tt);
  }
  return hipGetLastError();
}

}  // namespace mxfp4moe
