// Device routing of one token: top-k of its logits (descending, ties to the
// lower expert index) and the softmax over the k picks ("Restore GPT-OSS's
// router-masked expert-parallel plan", transformers PR #49431, description:
// the experts consume top-k routing data).  Shared by the routing kernels and
// the decode path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp4moe.h"
#include "mx_device.h"

namespace mxroute {

constexpr int kPerLane = MXFP4MOE_MAX_EXPERTS / 64;

// Selection key of logit v of expert e: larger keys for larger logits and,
// between equal logits, for the lower expert index.  The float bits are
// mapped to an unsigned order (sign flipped for non-negative values, all
// bits for negative ones); -0 takes the key of +0 since the two compare
// equal.  Every real key exceeds 0, the key of an empty slot.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  if ((b << 1) == 0u) b = 0u;
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ float key_logit(uint64_t k) {
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return (int)~(uint32_t)k; }

// Token t, by one wave (all 64 lanes active).  Lane l holds the keys of
// experts l, l+64, ... (kPL of them, kPL * 64 >= E); k rounds of a wave-wide
// key maximum pick the experts by descending logit (ties to the lower expert
// index); lane j keeps the j-th pick.  The softmax runs over the picks
// relative to the largest one.
template <int kPL>
__device__ inline void route_row_keys(const float* row, int t, int E, int top_k, int32_t* __restrict__ ids,
                                      float* __restrict__ weights, int32_t* ids_copy) {
  const int lane = mx::lane_id();
  uint64_t key[kPL];
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(row[e], e) : 0ull;
  }
  float my_v = 0.f, v0 = 0.f;
  int my_e = 0;
  for (int j = 0; j < top_k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPL; ++i) best = mx::max_u64(best, key[i]);
    best = mx::wave_max_u64(best);
    const int be = key_expert(best);
#pragma unroll
    for (int i = 0; i < kPL; ++i)
      if (lane + 64 * i == be) key[i] = 0ull;
    const float bv = key_logit(best);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) v0 = bv;
  }
  const float ex = lane < top_k ? expf(my_v - v0) : 0.f;
  const float sum = mx::wave_sum_f32(ex);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_e;
    weights[(size_t)t * top_k + lane] = ex / sum;
    if (ids_copy != nullptr) ids_copy[t * top_k + lane] = my_e;
  }
}

// route_row_keys with as few keys per lane as E needs (E is uniform).
__device__ inline void route_row(const float* row, int t, int E, int top_k, int32_t* __restrict__ ids,
                                 float* __restrict__ weights, int32_t* ids_copy = nullptr) {
  if (E <= 64)
    route_row_keys<1>(row, t, E, top_k, ids, weights, ids_copy);
  else if (E <= 128)
    route_row_keys<2>(row, t, E, top_k, ids, weights, ids_copy);
  else if (E <= 256)
    route_row_keys<4>(row, t, E, top_k, ids, weights, ids_copy);
  else
    route_row_keys<kPerLane>(row, t, E, top_k, ids, weights, ids_copy);
}

// Routing and grouping of a decode batch (T <= 4 tokens, P = T * top_k <= 64
// pairs: an expert then has at most 4 pairs, one streaming tile) inside one
// block, computed alike in every block of the launch that consumes it, so
// that no launch has to run before that one: wave t routes token t (as
// route_row), then wave 0 groups the pairs.  Lane p takes pair p and, in one
// pass over the pairs, counts the pairs of lower experts (its expert's first
// sorted row), the earlier pairs of its own expert (its place among them) and
// the expert's pairs; in a second pass the distinct lower experts (its
// expert's tile index).  The same ids, weights, stable expert order, offsets
// and tile table as the grouping kernel; block 0 (write) also stores them to
// global memory for the launches that follow.
struct SmallRoute {
  int32_t ids[64];
  float weights[64];
  int32_t sorted[64];
  int4 tiles[64];  // {expert, first sorted row, rows, 0} per active expert, in expert order
  int32_t num_active;
};
constexpr int kSmallRouteTokens = 4;
constexpr int kSmallRoutePairs = 64;

__device__ __forceinline__ void route_group_small(SmallRoute& s, const float* logits, int T, int E, int top_k, bool write,
                                         int32_t* ids, float* weights, int32_t* offsets, int32_t* sorted,
                                         int4* tiles, int32_t* counts) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int P = T * top_k;
  if (wave < T) route_row(logits + (size_t)wave * E, wave, E, top_k, s.ids, s.weights);  // uniform per wave
  __syncthreads();
  if (wave == 0) {
    const bool valid = lane < P;
    const int e = valid ? s.ids[lane] : 0x7fffffff;
    int below = 0, before = 0, cnt = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = __builtin_amdgcn_readlane(e, q);
      below += eq < e ? 1 : 0;
      before += (eq == e && q < lane) ? 1 : 0;
      cnt += eq == e ? 1 : 0;
    }
    const bool first = valid && before == 0;
    const uint64_t firsts = __ballot(first);
    int dbelow = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = __builtin_amdgcn_readlane(e, q);
      dbelow += (((firsts >> q) & 1ull) != 0 && eq < e) ? 1 : 0;
    }
    const int na = __popcll(firsts);
    if (valid) s.sorted[below + before] = lane;
    if (first) s.tiles[dbelow] = int4{e, below, cnt, 0};
    if (lane == 0) s.num_active = na;
    if (write) {
      if (valid) {
        ids[lane] = e;
        weights[lane] = s.weights[lane];
        sorted[below + before] = lane;
      }
      if (first) tiles[dbelow] = int4{e, below, cnt, 0};
      if (lane < 3) counts[lane] = lane == 2 ? na : 0;  // full, mid, streaming tiles
    }
  }
  __syncthreads();
  if (write) {
    for (int i = (int)threadIdx.x; i <= E; i += (int)blockDim.x) {
      int n = 0;
      for (int q = 0; q < P; ++q) n += s.ids[q] < i ? 1 : 0;
      offsets[i] = n;
    }
  }
}

}  // namespace mxroute
