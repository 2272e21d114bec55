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

// Tile configurations of the expert GEMMs.  Both GEMMs of one call use the
// same token tile (the tile table is shared).
enum GemmConfig : int {
  kGemmSmall = 0,  // 32 token columns per tile: decode-sized expert groups
  kGemmMid = 1,    // 64 token columns per tile
  kGemmWide = 2,   // 256 token columns per tile: prefill-sized expert groups
};
int gemm_tile_tokens(GemmConfig cfg);

// Routing: one wave per token.
hipError_t launch_route(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                        hipStream_t stream);

// Grouping: counts, offsets, stable expert-ordered pair list, and (when
// tiles != nullptr) the GEMM tile table for tiles of `tile_tokens` pairs.
hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        int32_t* tiles, int32_t* num_tiles, int tile_tokens, hipStream_t stream);

struct GemmArgs {
  const uint8_t* wblocks;   // [E, N, K/2]
  const uint8_t* wscales;   // [E, N, K/32]
  const uint16_t* bias;     // [E, N] bf16
  const uint16_t* act;      // gate_up: x [T, K]; down: a [P, K] in expert order
  const int32_t* sorted_pairs;
  const int32_t* tiles;     // [max_tiles][4] = {expert, first sorted row, rows, 0}
  const int32_t* num_tiles;
  const float* topk_weights;  // [P] (down only)
  void* out;                // gate_up: a [P, N/2] bf16 in expert order; down: zw [P, N] f32 by pair id
  int N, K, top_k, max_tiles;
};

hipError_t launch_gate_up(const GemmArgs& a, GemmConfig cfg, hipStream_t stream);
hipError_t launch_down(const GemmArgs& a, GemmConfig cfg, hipStream_t stream);
hipError_t launch_combine(const float* zw, uint16_t* y, int T, int H, int top_k, hipStream_t stream);

hipError_t launch_dequant(const uint8_t* blocks, const uint8_t* scales, uint16_t* out, int64_t N, int64_t K,
                          hipStream_t stream);

}  // namespace mxfp4moe
