// Routing data for the MXFP4 experts: top-k with softmax over the selected
// logits, then the pairs grouped by expert ("Restore GPT-OSS's router-masked
// expert-parallel plan", transformers PR #49431, description: the experts
// consume routing data and route their tokens themselves; "feat(gguf): serve
// gpt-oss gguf checkpoints on gpt_oss", FreeToken PR #838, "What it does":
// expert-ordered views of the tokens).
#include "../../include/mxfp4moe.h"
#include "internal.h"
#include "mx_device.h"
#include "route_device.h"

namespace {

using mxroute::route_row;

constexpr int kRouteThreads = 256;  // four tokens per block, one wave each

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

// Mask of the valid lanes of the wave whose expert id equals this lane's,
// matched bit by bit (nbits bits cover every id) with ballots.
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int nbits) {
  uint64_t match = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    match &= bit ? ones : ~ones;
  }
  return match;
}

// Histogram of experts, exclusive scan into offsets, a stable scatter of pair
// ids into expert order, and the GEMM tile tables: an expert with at least
// big_tokens pairs goes to wide tiles, one with more than kStreamTokens pairs
// to mid tiles, the rest to one streaming tile.
// The pairs are cut into chunks of the block size and each block scatters an
// equal run of consecutive chunks (one chunk per block when the grid has one
// block per chunk).  Every block histograms all P ids, counting separately
// those before its first chunk, so it knows where its pairs start inside
// each expert without a second launch or scratch memory.  Inside a chunk the
// lanes of a wave with the same expert are found by matching the expert id
// bit by bit with ballots, and the per-wave counts are turned into positions
// wave by wave, so pairs keep ascending id order inside every expert.
// Wave 0 scans the counts (and, in block 0, the tile counts of the three
// kinds) in one pass of DPP prefix sums; block 0 writes the offsets and the
// tile tables.
// With logits != nullptr (one block only) the block first routes the T
// tokens itself (one wave per token), saving a launch for small batches, and
// keeps the routed ids in LDS for the histogram and the scatter.
template <int kGroupThreads>
__global__ __launch_bounds__(kGroupThreads) void group_kernel(const float* __restrict__ logits, int T, int top_k,
                                                              float* __restrict__ weights,
                                                              int32_t* __restrict__ ids, int P, int E,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_pairs,
                                                              mxfp4moe::TileTables tt) {
  constexpr int kGroupWaves = kGroupThreads / 64;
  constexpr int kRep = kGroupWaves / 2;  // histogram copies per expert
  static_assert(kGroupWaves == 4 || kGroupWaves == 16, "block of 4 or 16 waves");
  extern __shared__ int smem[];
  int* cnt = smem;                 // [E] pairs per expert
  int* base = cnt + E;             // [E] sorted row of this block's next pair of each expert
  int* before = base + E;          // [E] pairs of each expert before this block's chunks
  int* wave_cnt = before + E;      // [E][kGroupWaves]; the histogram copies use it first
  int* idl = wave_cnt + kGroupWaves * E;  // [P] the routed ids (fused routing only)

  const int32_t* idsrc = ids;
  if (logits != nullptr) {
    for (int t = threadIdx.x >> 6; t < T; t += kGroupWaves)
      route_row(logits + (size_t)t * E, t, E, top_k, ids, weights, idl);
    idsrc = idl;  // the block reads the ids it routed from LDS
    __syncthreads();
  }
  const int nchunks = (P + kGroupThreads - 1) / kGroupThreads;
  const int per_block = (nchunks + (int)gridDim.x - 1) / (int)gridDim.x;
  const int p_begin = min(P, (int)blockIdx.x * per_block * kGroupThreads);
  const int p_end = min(P, p_begin + per_block * kGroupThreads);
  const int lane = mx::lane_id();
  const int wave = threadIdx.x >> 6;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;

  // Histogram in kRep copies per expert, lane l adding to copy l % kRep, so
  // fewer lanes of one LDS atomic meet on one address (routing skew puts a
  // popular expert in many lanes); pairs before p_begin in one set of copies,
  // the rest in another.
  int* hist_before = wave_cnt;           // [E][kRep]
  int* hist_rest = wave_cnt + kRep * E;  // [E][kRep]
  for (int i = threadIdx.x; i < 2 * kRep * E; i += kGroupThreads) wave_cnt[i] = 0;
  __syncthreads();
  {
    constexpr int kHistBatch = 8;  // ids in flight per thread before their atomics
    const int copy = lane % kRep;
    for (int p0 = threadIdx.x; p0 < P; p0 += kHistBatch * kGroupThreads) {
      int ev[kHistBatch];
#pragma unroll
      for (int j = 0; j < kHistBatch; ++j) {
        const int p = p0 + j * kGroupThreads;
        ev[j] = p < P ? idsrc[p] : -1;
      }
#pragma unroll
      for (int j = 0; j < kHistBatch; ++j) {
        if (ev[j] >= 0) {
          int* h = p0 + j * kGroupThreads < p_begin ? hist_before : hist_rest;
          atomicAdd(&h[ev[j] * kRep + copy], 1);
        }
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kGroupThreads) {
    int sb = 0, sr = 0;
#pragma unroll
    for (int r = 0; r < kRep; ++r) {
      sb += hist_before[e * kRep + r];
      sr += hist_rest[e * kRep + r];
    }
    before[e] = sb;
    cnt[e] = sb + sr;
  }
  __syncthreads();

  if (wave == 0) {
    const bool tables = tt.big != nullptr && blockIdx.x == 0;
    const int bt = tables ? tt.big_tokens : 0;
    const bool wide_on = bt > 0 && !tt.no_wide;
    const bool mid_on = bt > 0 || tt.no_wide;  // else everything in streaming tiles
    constexpr int st = mxfp4moe::kStreamTokens;
    constexpr int mt = mxfp4moe::kMidTokens;
    int carry = 0, tb = 0, tm = 0, ts = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? cnt[e] : 0;
      const int ic = mx::wave_inclusive_sum(c);
      const int start = carry + ic - c;  // expert e's first sorted row
      if (e < E) {
        base[e] = start + before[e];
        if (blockIdx.x == 0) offsets[e] = start;
      }
      carry += __builtin_amdgcn_readlane(ic, 63);
      if (tables) {
        // an expert with at least bt pairs: all its pairs in tiles of bt (the
        // last one partial), so its weights are streamed by one kernel only;
        // fewer than bt, more than st: ceil(c / mt) mid tiles of near-equal
        // size (the first c % nm one pair larger); at most st: one streaming
        // tile; without full tiles (bt == 0) every pair in streaming tiles of st
        // (no_stream: mid tiles for every expert with pairs)
        const int nb = (wide_on && c >= bt) ? (c + bt - 1) / bt : 0;
        const int nm = (mid_on && c > (tt.no_stream ? 0 : st) && (tt.no_wide || c < bt)) ? (c + mt - 1) / mt : 0;
        const int ns = tt.no_stream ? 0 : mid_on ? (c > 0 && c <= st ? 1 : 0) : (c + st - 1) / st;
        const int ib = mx::wave_inclusive_sum(nb);
        const int im = mx::wave_inclusive_sum(nm);
        const int is = mx::wave_inclusive_sum(ns);
        int4* big = reinterpret_cast<int4*>(tt.big) + tb + ib - nb;
        for (int i = 0; i < nb; ++i) big[i] = int4{e, start + i * bt, min(bt, c - i * bt), 0};
        int4* mid = reinterpret_cast<int4*>(tt.mid) + tm + im - nm;
        if (nm > 0) {
          const int mq = c / nm, mr = c - mq * nm;
          for (int i = 0; i < nm; ++i) mid[i] = int4{e, start + i * mq + min(i, mr), mq + (i < mr ? 1 : 0), 0};
        }
        int4* small = reinterpret_cast<int4*>(tt.small) + ts + is - ns;
        for (int i = 0; i < ns; ++i) small[i] = int4{e, start + i * st, min(st, c - i * st), 0};
        tb += __builtin_amdgcn_readlane(ib, 63);
        tm += __builtin_amdgcn_readlane(im, 63);
        ts += __builtin_amdgcn_readlane(is, 63);
      }
    }
    if (lane == 0 && blockIdx.x == 0) {
      offsets[E] = P;
      if (tables) {
        *tt.num_big = tb;
        *tt.num_mid = tm;
        *tt.num_small = ts;
      }
    }
  }
  __syncthreads();

  for (int c0 = p_begin; c0 < p_end; c0 += kGroupThreads) {
    for (int i = threadIdx.x; i < kGroupWaves * E; i += kGroupThreads) wave_cnt[i] = 0;
    __syncthreads();
    const int p = c0 + threadIdx.x;
    const bool valid = p < p_end;
    const int e = valid ? idsrc[p] : 0;
    const uint64_t match = same_expert_lanes(e, valid, nbits);
    const int rank = mx::lanes_below(match);
    if (valid && rank == 0) wave_cnt[e * kGroupWaves + wave] = __popcll(match);
    __syncthreads();
    // each expert's per-wave counts -> the waves' first sorted rows
    if constexpr (kGroupWaves == 16) {
      // one DPP row per expert: an in-row prefix sum over the 16 waves; the
      // row's last lane advances the expert's base for the next chunk (the
      // row's reads of base[] come first in the wave's LDS order)
      const int n = kGroupWaves * E;
      for (int i0 = 0; i0 < n; i0 += kGroupThreads) {  // uniform trip count: all lanes run the DPP steps
        const int i = i0 + (int)threadIdx.x;
        const int c = i < n ? wave_cnt[i] : 0;
        const int incl = mx::row_inclusive_sum(c);
        if (i < n) {
          const int b = base[i >> 4];
          wave_cnt[i] = b + incl - c;
          if ((i & 15) == 15) base[i >> 4] = b + incl;
        }
      }
    } else {
      for (int ee = threadIdx.x; ee < E; ee += kGroupThreads) {
        int run = base[ee];
        for (int w = 0; w < kGroupWaves; ++w) {
          const int c = wave_cnt[ee * kGroupWaves + w];
          wave_cnt[ee * kGroupWaves + w] = run;
          run += c;
        }
        base[ee] = run;
      }
    }
    __syncthreads();
    if (valid) sorted_pairs[wave_cnt[e * kGroupWaves + wave] + rank] = p;
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
  const size_t smem = (size_t)(3 + kThreads / 64) * E * sizeof(int);
  // one block per chunk of kThreads pairs (one block writes the offsets when P == 0)
  const unsigned grid = P > kThreads ? (unsigned)((P + kThreads - 1) / kThreads) : 1u;
  ProfileScope prof(kStageGroup, stream);
  group_kernel<kThreads><<<grid, kThreads, smem, stream>>>(nullptr, 0, 1, nullptr, const_cast<int32_t*>(ids), P, E,
                                                      offsets, sorted_pairs, tt);
  return hipGetLastError();
}

hipError_t launch_route_group(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                              int32_t* offsets, int32_t* sorted_pairs, const TileTables& tt, hipStream_t stream) {
  // small batches: four waves (cheaper barriers and scans); the routed ids stay in LDS
  const int P = T * top_k;
  ProfileScope prof(kStageGroup, stream);
  if (P <= 256) {
    const size_t smem = (size_t)(3 + 4) * E * sizeof(int) + (size_t)P * sizeof(int);
    group_kernel<256><<<1, 256, smem, stream>>>(logits, T, top_k, weights, ids, P, E, offsets, sorted_pairs, tt);
  } else {
    const size_t smem = (size_t)(3 + kGroupThreadsMax / 64) * E * sizeof(int) + (size_t)P * sizeof(int);
    group_kernel<kGroupThreadsMax><<<1, kGroupThreadsMax, smem, stream>>>(logits, T, top_k, weights, ids, P, E,
                                                                          offsets, sorted_pairs, tt);
  }
  return hipGetLastError();
}

}  // namespace mxfp4moe
