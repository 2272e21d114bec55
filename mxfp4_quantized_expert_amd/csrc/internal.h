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

// Token tiles of the expert GEMMs.  Every expert's pairs are cut into full
// tiles of kWideTokens pairs, computed by the wide kernel, and a remainder
// cut into tiles of kStreamTokens pairs, computed by the streaming kernel
// (which is also the whole path for decode-sized batches).
constexpr int kWideTokens = 128;
constexpr int kStreamTokens = 32;

struct TileTables {
  int32_t* big;        // [max_big][4]   = {expert, first sorted row, rows, 0}
  int32_t* num_big;
  int32_t* small;      // [max_small][4]
  int32_t* num_small;
  int big_tokens;      // 0: no full tiles, everything goes to the small table
  int small_tokens;
};

// Routing: one wave per token.
hipError_t launch_route(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                        hipStream_t stream);

// Grouping: counts, offsets, stable expert-ordered pair list, and (when
// tt.big != nullptr) the GEMM tile tables.
hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const TileTables& tt, hipStream_t stream);

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

// Both GEMM stages launch the wide kernel over the full tiles (when there are
// any) and the streaming kernel over the remainder tiles.
hipError_t launch_gate_up(GemmArgs a, const TileTables& tt, int max_big, int max_small, hipStream_t stream);
hipError_t launch_down(GemmArgs a, const TileTables& tt, int max_big, int max_small, hipStream_t stream);
hipError_t launch_combine(const float* zw, uint16_t* y, int T, int H, int top_k, hipStream_t stream);

hipError_t launch_dequant(const uint8_t* blocks, const uint8_t* scales, uint16_t* out, int64_t N, int64_t K,
                          hipStream_t stream);

}  // namespace mxfp4moe
