// Host-side declarations shared by the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxfp4moe {

enum Stage : int {
  kStageNone = 0,
  kStageRoute = 1,
  kStageGroup = 2,
  kStageGateUp = 3,
  kStageDown = 4,
  kStageCombine = 5,
  kStageDequant = 6,
  kStageGateUpWide = 7,    // the full-tile launch of gate_up alone
  kStageGateUpStream = 8,  // the remainder-tile launch of gate_up alone
  kStageDownWide = 9,
  kStageDownStream = 10,
  kStageGateUpMid = 11,    // the mid-size remainder launch of gate_up alone
  kStageDownMid = 12,
  kStageActQuant = 13,     // the MXFP8 activation quantizer of the FP4 scaled-MFMA path
  kStageLast = kStageActQuant,
};

// Records a HIP event pair around one launch when the benchmark hook asked for
// this stage (see mxfp4moe_profile_begin); otherwise does nothing.
class ProfileScope {
 public:
  ProfileScope(int stage, hipStream_t stream);
  ~ProfileScope();
  ProfileScope(const ProfileScope&) = delete;
  ProfileScope& operator=(const ProfileScope&) = delete;

 private:
  int slot_;
  hipStream_t stream_;
};

int device_cu_count();

// Token tiles of the expert GEMMs.  An expert with at least kWideTokens pairs
// is cut into tiles of kWideTokens pairs, the last one partial (wide kernel);
// one with more than kStreamTokens pairs into ceil(pairs / kMidTokens) mid
// tiles of near-equal size (mid kernel); one with at most kStreamTokens pairs
// makes a single streaming tile (streaming kernel, which is also the whole
// path for decode-sized batches).  Every expert's weights are streamed by one
// kernel.  With big_tokens == 0 every pair goes to the streaming kernel in
// tiles of kStreamTokens.
constexpr int kWideTokens = 128;
constexpr int kStreamTokens = 4;
constexpr int kMidTokens = 48;
// Batches of kStreamTokens < T <= kMidOnlyTokens take no full tiles, and no
// streaming tiles either when they average at least kMidOnlyPairsPerExpert
// pairs per expert.
constexpr int kMidOnlyTokens = 256;
constexpr int kMidOnlyPairsPerExpert = 16;
constexpr int kMaxHidden = 4096;  // bound on H and I (the GEMMs stage scale rows in LDS)

struct TileTables {
  int32_t* big;        // [max_big][4]   = {expert, first sorted row, rows, 0}
  int32_t* num_big;
  int32_t* mid;        // [max_mid][4]
  int32_t* num_mid;
  int32_t* small;      // [max_small][4]
  int32_t* num_small;
  int big_tokens;      // kWideTokens, or 0 (then: every pair in streaming tiles unless no_wide)
  int no_wide;         // no wide tiles: more than kStreamTokens pairs -> mid tiles, whatever the count
  int no_stream;       // with no_wide: every expert with pairs -> mid tiles (no streaming tiles)
};

// Capacities of the tile tables (bounds the GEMM grids).
struct TileBounds {
  int max_big, max_mid, max_small;
};

// Routing: one wave per token.
hipError_t launch_route(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                        hipStream_t stream);

// Router projection and routing in one launch: logits = x W_r^T + b_r (fp32,
// written to `logits`), then the top-k and softmax as launch_route.
hipError_t launch_route_proj(const uint16_t* x, const uint16_t* router_w, const uint16_t* router_b, int T, int H,
                             int E, int top_k, float* logits, int32_t* ids, float* weights, hipStream_t stream);

// Grouping: counts, offsets, stable expert-ordered pair list, and (when
// tt.big != nullptr) the GEMM tile tables.
hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const TileTables& tt, hipStream_t stream);

// Routing and grouping in one single-block launch, for batches of at most
// kFusedRouteTokens tokens (one wave routes each token).
constexpr int kFusedRouteTokens = 64;
hipError_t launch_route_group(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                              int32_t* offsets, int32_t* sorted_pairs, const TileTables& tt, hipStream_t stream);

struct GemmArgs {
  const uint8_t* wblocks;   // [E, N, K/2]
  const uint8_t* wscales;   // [E, N, K/32]
  const uint16_t* bias;     // [E, N] bf16
  const uint16_t* act;      // gate_up: x [T, K]; down: a [P, K] in expert order
  const int32_t* sorted_pairs;
  const int32_t* tiles;     // [max_tiles][4] = {expert, first sorted row, rows, 0}
  const int32_t* num_tiles;
  const float* topk_weights;  // [P] (down only)
  void* out;                // gate_up: a [P, N/2] bf16 in expert order; down: zw [P, N] bf16 by pair id
  int64_t act_rows;         // rows of `act` (gate_up: T, down: P)
  int N, K, top_k, max_tiles;
  int split_gate_up;        // gate_up only: w13 rows stored [I gate rows; I up rows] instead of interleaved
  const float* scale2;      // NVFP4: [E] second-level scale per expert (scales are E4M3 per 16), else nullptr
  // FP4 scaled-MFMA path for the full tiles (opt-in): the activations of
  // `act` quantized to MXFP8 by launch_act_quant (codes and scale words).
  int act_mode;             // kActBf16, kActMxfp8 or kActMxfp8Split
  const uint8_t* act_codes;
  const uint8_t* act_scales;
  // Decode batches (gate_up streaming launch only): route_logits != nullptr
  // makes every block route and group the batch itself (route_T tokens,
  // route_E experts); block 0 writes the routing data and the tile table
  // that the down and combine launches read: ids, weights (topk_weights),
  // offsets, sorted pairs (sorted_pairs), tiles and the three tile counts.
  const float* route_logits;
  int route_T, route_E;
  int32_t* route_ids;
  float* route_weights;
  int32_t* route_offsets;
  int32_t* route_sorted;
  int32_t* route_tiles;
  int32_t* route_counts;
};
enum ActMode : int { kActBf16 = 0, kActMxfp8 = 1, kActMxfp8Split = 2 };

// Both GEMM stages launch the wide, mid and streaming kernels over their
// tables (each launch skipped when its table has no capacity).
hipError_t launch_gate_up(GemmArgs a, const TileTables& tt, const TileBounds& tb, hipStream_t stream);
hipError_t launch_down(GemmArgs a, const TileTables& tt, const TileBounds& tb, hipStream_t stream);
hipError_t launch_combine(const uint16_t* zw, uint16_t* y, int T, int H, int top_k, hipStream_t stream);

// MXFP8 activations (single or split) in the FP4 GEMM's chunk-interleaved
// layout: per row act_quant_row_bytes(K) code bytes and
// act_quant_scale_row_bytes(K) scale bytes.
size_t act_quant_row_bytes(int K);
size_t act_quant_scale_row_bytes(int K);
hipError_t launch_act_quant(const uint16_t* src, int rows, int K, bool split, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream);

hipError_t launch_dequant(const uint8_t* blocks, const uint8_t* scales, uint16_t* out, int64_t N, int64_t K,
                          hipStream_t stream);

// Dequant-on-copy from host memory through two device staging slots.
int64_t offload_chunk_rows(int64_t K);
size_t offload_staging_bytes(int64_t N, int64_t K);
hipError_t launch_dequant_from_host(const uint8_t* host_blocks, const uint8_t* host_scales, uint16_t* out,
                                    int64_t N, int64_t K, uint8_t* staging, hipStream_t stream);

}  // namespace mxfp4moe
