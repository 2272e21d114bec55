// C ABI of libmxfp4moe.so: argument checks, workspace carving, tile
// configuration choice and the launch sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/mxfp4moe.h"
#include "internal.h"
#include "route_device.h"

namespace mxfp4moe {

// ---------------------------------------------------------------- profiling

namespace {
std::mutex g_prof_mu;
std::atomic<int> g_prof_stage{kStageNone};
int g_prof_next = 0;
std::vector<hipEvent_t> g_prof_start, g_prof_stop;
}  // namespace

ProfileScope::ProfileScope(int stage, hipStream_t stream) : slot_(-1), stream_(stream) {
  if (g_prof_stage.load(std::memory_order_relaxed) == kStageNone) return;  // hook off: no lock
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (stage != g_prof_stage || g_prof_next >= (int)g_prof_start.size()) return;
  slot_ = g_prof_next++;
  (void)hipEventRecord(g_prof_start[slot_], stream_);
}

ProfileScope::~ProfileScope() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof_stop[slot_], stream_);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// ---------------------------------------------------------------- workspace

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t ids, weights, offsets, sorted, counts, big, mid, small, act, zw, logits, xq, xqs, aq, aqs, total;
  int max_big, max_mid, max_small;
};

// Tile table capacities.  An expert gets at most T pairs (a token's k
// experts are distinct).  An expert with at least kWideTokens pairs makes
// ceil(c / kWideTokens) wide tiles (at most P / kWideTokens full ones plus one
// partial per such expert); one with kStreamTokens < c < kWideTokens pairs
// ceil(c / kMidTokens) mid tiles (at most kMidPerExpert, and never more than
// one per kStreamTokens + 1 of its pairs); one with fewer, one streaming tile.
// With no wide tiles an expert with more than kStreamTokens pairs makes
// ceil(c / kMidTokens) mid tiles.  With streaming tiles only, every pair goes
// to tiles of kStreamTokens.
enum TileMode { kTilesWide, kTilesNoWide, kTilesStreamOnly, kTilesMidOnly };
TileBounds tile_bounds(int64_t T, int64_t P, int64_t E, TileMode mode) {
  const int64_t active = E < P ? E : P;
  const int64_t fulls = P / kWideTokens;
  TileBounds b;
  b.max_big = (mode == kTilesWide && T >= kWideTokens) ? (int)(fulls + (active < fulls ? active : fulls)) : 0;
  constexpr int64_t kMidPerExpert = (kWideTokens - 1 + kMidTokens - 1) / kMidTokens;
  const int64_t mids = P / (kStreamTokens + 1);
  if (mode == kTilesWide)
    b.max_mid = T > kStreamTokens ? (int)(kMidPerExpert * active < mids ? kMidPerExpert * active : mids) : 0;
  else if (mode == kTilesNoWide || mode == kTilesMidOnly)
    b.max_mid = T > kStreamTokens ? (int)(P / kMidTokens + active) : 0;
  else
    b.max_mid = 0;
  b.max_small = mode == kTilesStreamOnly ? (int)(P / kStreamTokens + active) : mode == kTilesMidOnly ? 0 : (int)active;
  return b;
}

Layout make_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, bool fp8_act = false) {
  const int64_t P = T * top_k;
  Layout L;
  const TileBounds wide = tile_bounds(T, P, E, kTilesWide), no_wide = tile_bounds(T, P, E, kTilesNoWide),
                   stream_only = tile_bounds(T, P, E, kTilesStreamOnly);
  L.max_big = wide.max_big;
  L.max_mid = wide.max_mid > no_wide.max_mid ? wide.max_mid : no_wide.max_mid;
  L.max_small = stream_only.max_small;  // the largest of the three
  size_t off = 0;
  L.ids = off;       off = align_up(off + (size_t)P * 4);
  L.weights = off;   off = align_up(off + (size_t)P * 4);
  L.offsets = off;   off = align_up(off + (size_t)(E + 1) * 4);
  L.sorted = off;    off = align_up(off + (size_t)P * 4);
  L.counts = off;    off = align_up(off + 12);
  L.big = off;       off = align_up(off + (size_t)L.max_big * 16);
  L.mid = off;       off = align_up(off + (size_t)L.max_mid * 16);
  L.small = off;     off = align_up(off + (size_t)L.max_small * 16);
  L.act = off;       off = align_up(off + (size_t)P * (size_t)I * 2);
  L.zw = off;        off = align_up(off + (size_t)P * (size_t)H * 2);  // bf16 pair outputs
  L.logits = off;    off = align_up(off + (size_t)T * (size_t)E * 4);  // router projection output
  // MXFP8 activations of the FP4 scaled-MFMA path (only with its flag)
  const size_t nx = fp8_act ? (size_t)T : 0, na = fp8_act ? (size_t)P : 0;
  L.xq = off;        off = align_up(off + nx * act_quant_row_bytes((int)H));
  L.xqs = off;       off = align_up(off + nx * act_quant_scale_row_bytes((int)H));
  L.aq = off;        off = align_up(off + na * act_quant_row_bytes((int)I));
  L.aqs = off;       off = align_up(off + na * act_quant_scale_row_bytes((int)I));
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

int check_route_shape(int64_t T, int64_t E, int64_t top_k) {
  if (T < 0 || E < 1 || E > MXFP4MOE_MAX_EXPERTS) return MXFP4MOE_ERR_SHAPE;
  if (top_k < 1 || top_k > E || top_k > MXFP4MOE_MAX_TOPK) return MXFP4MOE_ERR_SHAPE;
  if (T * top_k > (int64_t)0x7fffffff) return MXFP4MOE_ERR_SHAPE;
  return MXFP4MOE_OK;
}

}  // namespace
}  // namespace mxfp4moe

using namespace mxfp4moe;

namespace {

// Scratch of moe_mxfp4_forward_noalloc: a fixed device array, so that callers
// that cannot allocate (graph capture, tight serving loops) need no
// workspace.  Each device holds its own copy for the life of the process.  In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, looked up once per device (noalloc_scratch below).
constexpr size_t kNoAllocScratch = MXFP4MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or nullptr if it cannot be had.
void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

const float kNvQuery = 0.f;  // stands in for the NVFP4 scale pointers of a size query
constexpr uint32_t kForwardFlags =
    MXFP4MOE_GATE_UP_SPLIT | MXFP4MOE_ACT_MXFP8 | MXFP4MOE_ACT_MXFP8_SPLIT | MXFP4MOE_TILES_STREAM;

// The layer.  scale2_13 / scale2_2 != nullptr selects NVFP4 weights (E4M3
// block scales per 16 elements, one second-level scale per expert and
// projection, multiplied before the bias).  router_w != nullptr replaces the
// logits by the router projection of x (router_logits is then unused).
int forward_impl(const uint16_t* x, const float* router_logits, const uint16_t* router_w, const uint16_t* router_b,
                 const uint8_t* w13_blocks, const uint8_t* w13_scales,
                 const float* scale2_13, const uint16_t* w13_bias, const uint8_t* w2_blocks,
                 const uint8_t* w2_scales, const float* scale2_2, const uint16_t* w2_bias, uint16_t* y, int64_t T,
                 int64_t H, int64_t I, int64_t E, int64_t top_k, uint32_t flags, void* workspace,
                 size_t* workspace_bytes, void* stream, bool check_only = false) {
  const bool nv = scale2_13 != nullptr;
  if (workspace_bytes == nullptr) return MXFP4MOE_ERR_ARG;
  int st = check_route_shape(T, E, top_k);
  if (st != MXFP4MOE_OK) return st;
  if (H <= 0 || I <= 0 || (H & 31) != 0 || (I & 31) != 0) return MXFP4MOE_ERR_SHAPE;
  if (H > MXFP4MOE_MAX_HIDDEN || I > MXFP4MOE_MAX_HIDDEN) return MXFP4MOE_ERR_SHAPE;
  static_assert(MXFP4MOE_MAX_HIDDEN == kMaxHidden, "one bound on H and I");
  const int act_mode = (flags & MXFP4MOE_ACT_MXFP8_SPLIT) ? kActMxfp8Split
                       : (flags & MXFP4MOE_ACT_MXFP8)     ? kActMxfp8
                                                          : kActBf16;
  if (act_mode != kActBf16 && nv) return MXFP4MOE_ERR_ARG;  // NVFP4 weights have no FP4 scaled-MFMA path here
  const Layout L = make_layout(T, H, I, E, top_k, act_mode != kActBf16);
  if (workspace == nullptr) {
    *workspace_bytes = L.total;
    return MXFP4MOE_OK;
  }
  if (w13_blocks == nullptr || w13_scales == nullptr || w13_bias == nullptr || w2_blocks == nullptr ||
      w2_scales == nullptr || w2_bias == nullptr)
    return MXFP4MOE_ERR_ARG;
  if (T > 0 && (x == nullptr || y == nullptr)) return MXFP4MOE_ERR_ARG;
  if (T > 0 && router_w == nullptr && router_logits == nullptr) return MXFP4MOE_ERR_ARG;
  if (T > 0 && router_w != nullptr && router_b == nullptr) return MXFP4MOE_ERR_ARG;
  if (T > 0 && router_w != nullptr && !aligned16(router_w)) return MXFP4MOE_ERR_ALIGN;
  if (*workspace_bytes < L.total) return MXFP4MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MXFP4MOE_ERR_ALIGN;
  if (!aligned16(w13_blocks) || !aligned16(w2_blocks)) return MXFP4MOE_ERR_ALIGN;
  // the GEMMs stage scale rows with 16-byte loads and read biases four at a time
  if (!aligned16(w13_scales) || !aligned16(w2_scales)) return MXFP4MOE_ERR_ALIGN;
  if (!aligned8(w13_bias) || !aligned8(w2_bias)) return MXFP4MOE_ERR_ALIGN;
  if (T > 0 && (!aligned16(x) || !aligned16(y))) return MXFP4MOE_ERR_ALIGN;
  if (T == 0 || check_only) return MXFP4MOE_OK;

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* weights = reinterpret_cast<float*>(ws + L.weights);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  uint16_t* zw = reinterpret_cast<uint16_t*>(ws + L.zw);

  const int64_t P = T * top_k;
  TileTables tt;
  tt.big = reinterpret_cast<int32_t*>(ws + L.big);
  tt.num_big = counts;
  tt.mid = reinterpret_cast<int32_t*>(ws + L.mid);
  tt.num_mid = counts + 1;
  tt.small = reinterpret_cast<int32_t*>(ws + L.small);
  tt.num_small = counts + 2;
  // full tiles of kWideTokens pairs take the wide kernel unless the caller
  // asked for streaming tiles only (a check of that kernel on every shape);
  // NVFP4 full tiles read a chunk's scales of a row as one aligned dword, so
  // they need H and I to be multiples of 64 (else mid tiles take those pairs)
  const bool nv_no_wide = nv && ((H & 63) != 0 || (I & 63) != 0);
  // Small prefill batches (kStreamTokens < T <= kMidOnlyTokens, exact bf16
  // activations): no full tiles, since an expert then holds at most two
  // (its pairs take mid tiles of at most kMidTokens instead), and when the
  // batch averages at least kMidOnlyPairsPerExpert pairs per expert no
  // streaming tiles either (an expert with 1..kStreamTokens pairs takes one
  // mid tile).  A launch whose table turns out empty still costs about as
  // much as a launch of a few tiles, and the host cannot know the counts, so
  // the kinds of tile a batch of this size seldom has get no launch at all.
  const bool stream_only = (flags & MXFP4MOE_TILES_STREAM) != 0;
  const bool small = act_mode == kActBf16 && !stream_only && T > kStreamTokens && T <= kMidOnlyTokens;
  const bool mid_only = small && P >= kMidOnlyPairsPerExpert * E;
  tt.no_wide = nv_no_wide || small ? 1 : 0;
  tt.big_tokens = tt.no_wide || stream_only ? 0 : kWideTokens;
  tt.no_stream = mid_only ? 1 : 0;
  const TileBounds tb = tile_bounds(T, P, E,
                                    mid_only             ? kTilesMidOnly
                                    : tt.no_wide         ? kTilesNoWide
                                    : tt.big_tokens > 0  ? kTilesWide
                                                         : kTilesStreamOnly);
  hipStream_t s = (hipStream_t)stream;

  // A decode batch is routed and grouped inside the gate_up launch (every
  // block of it does so alike; one writes the data the later launches read).
  // (With the router projection, from the logits it leaves in the workspace.)
  // (Such a batch has streaming tiles only: its gate_up is one streaming launch.)
  const bool route_in_gate_up = act_mode == kActBf16 && T <= mxroute::kSmallRouteTokens &&
                                P <= mxroute::kSmallRoutePairs && tb.max_big == 0 && tb.max_mid == 0 &&
                                tb.max_small > 0;
  const float* logits = router_w != nullptr ? reinterpret_cast<const float*>(ws + L.logits) : router_logits;
  hipError_t err = hipSuccess;
  if (router_w != nullptr) {
    err = launch_route_proj(x, router_w, router_b, (int)T, (int)H, (int)E, (int)top_k,
                            reinterpret_cast<float*>(ws + L.logits), ids, weights, s);
    if (err == hipSuccess && !route_in_gate_up) err = launch_group(ids, (int)P, (int)E, offsets, sorted, tt, s);
  } else if (route_in_gate_up) {
    // nothing before the gate_up launch
  } else if (T <= kFusedRouteTokens) {
    err = launch_route_group(router_logits, (int)T, (int)E, (int)top_k, ids, weights, offsets, sorted, tt, s);
  } else {
    err = launch_route(router_logits, (int)T, (int)E, (int)top_k, ids, weights, s);
    if (err == hipSuccess) err = launch_group(ids, (int)P, (int)E, offsets, sorted, tt, s);
  }
  GemmArgs g{};
  g.sorted_pairs = sorted;
  g.topk_weights = weights;
  g.top_k = (int)top_k;
  if (err == hipSuccess) {
    g.split_gate_up = (flags & MXFP4MOE_GATE_UP_SPLIT) ? 1 : 0;
    g.scale2 = nv ? scale2_13 : nullptr;
    g.wblocks = w13_blocks;
    g.wscales = w13_scales;
    g.bias = w13_bias;
    g.act = x;
    g.act_rows = T;
    g.out = act;
    g.N = (int)(2 * I);
    g.K = (int)H;
    if (act_mode != kActBf16 && tb.max_big > 0) {
      g.act_mode = act_mode;
      g.act_codes = reinterpret_cast<const uint8_t*>(ws + L.xq);
      g.act_scales = reinterpret_cast<const uint8_t*>(ws + L.xqs);
      err = launch_act_quant(x, (int)T, (int)H, act_mode == kActMxfp8Split, reinterpret_cast<uint8_t*>(ws + L.xq),
                             reinterpret_cast<uint8_t*>(ws + L.xqs), s);
    }
    if (route_in_gate_up) {
      g.route_logits = logits;
      g.route_T = (int)T;
      g.route_E = (int)E;
      g.route_ids = ids;
      g.route_weights = weights;
      g.route_offsets = offsets;
      g.route_sorted = sorted;
      g.route_tiles = tt.small;
      g.route_counts = counts;
    }
    if (err == hipSuccess) err = launch_gate_up(g, tt, tb, s);
    g.route_logits = nullptr;
  }
  if (err == hipSuccess) {
    g.wblocks = w2_blocks;
    g.wscales = w2_scales;
    g.bias = w2_bias;
    g.act = act;
    g.act_rows = P;
    g.out = zw;
    g.N = (int)H;
    g.K = (int)I;
    if (g.act_mode != kActBf16) {
      g.act_codes = reinterpret_cast<const uint8_t*>(ws + L.aq);
      g.act_scales = reinterpret_cast<const uint8_t*>(ws + L.aqs);
      err = launch_act_quant(act, (int)P, (int)I, act_mode == kActMxfp8Split, reinterpret_cast<uint8_t*>(ws + L.aq),
                             reinterpret_cast<uint8_t*>(ws + L.aqs), s);
    }
    g.split_gate_up = 0;
    g.scale2 = nv ? scale2_2 : nullptr;
    if (err == hipSuccess) err = launch_down(g, tt, tb, s);
  }
  if (err == hipSuccess) err = launch_combine(zw, y, (int)T, (int)H, (int)top_k, s);
  return err == hipSuccess ? MXFP4MOE_OK : MXFP4MOE_ERR_HIP;
}

}  // namespace

extern "C" {

const char* mxfp4moe_status_string(int status) {
  switch (status) {
    case MXFP4MOE_OK: return "ok";
    case MXFP4MOE_ERR_ARG: return "invalid argument (NULL pointer)";
    case MXFP4MOE_ERR_SHAPE: return "unsupported shape";
    case MXFP4MOE_ERR_WORKSPACE: return "workspace too small";
    case MXFP4MOE_ERR_ALIGN: return "pointer not aligned as required";
    case MXFP4MOE_ERR_HIP: return "HIP launch error";
    case MXFP4MOE_ERR_SCRATCH: return "layer needs more than the no-allocation scratch";
    default: return "unknown status";
  }
}

int mxfp4_dequantize(const uint8_t* blocks, const uint8_t* scales, uint16_t* out_bf16, int64_t N, int64_t K,
                     void* stream) {
  if (N < 0 || K <= 0 || (K & 31) != 0) return MXFP4MOE_ERR_SHAPE;
  if (N > 0 && K > ((int64_t)1 << 62) / N) return MXFP4MOE_ERR_SHAPE;
  if (N == 0) return MXFP4MOE_OK;
  if (blocks == nullptr || scales == nullptr || out_bf16 == nullptr) return MXFP4MOE_ERR_ARG;
  if (!aligned16(blocks) || !aligned16(out_bf16)) return MXFP4MOE_ERR_ALIGN;
  hipError_t err = launch_dequant(blocks, scales, out_bf16, N, K, (hipStream_t)stream);
  return err == hipSuccess ? MXFP4MOE_OK : MXFP4MOE_ERR_HIP;
}

int mxfp4_dequantize_from_host(const uint8_t* host_blocks, const uint8_t* host_scales, uint16_t* out_bf16,
                               int64_t N, int64_t K, void* staging, size_t* staging_bytes, void* stream) {
  if (staging_bytes == nullptr) return MXFP4MOE_ERR_ARG;
  if (N < 0 || K <= 0 || (K & 31) != 0) return MXFP4MOE_ERR_SHAPE;
  if (N > 0 && K > ((int64_t)1 << 62) / N) return MXFP4MOE_ERR_SHAPE;
  const size_t need = offload_staging_bytes(N, K);
  if (staging == nullptr) {
    *staging_bytes = need;
    return MXFP4MOE_OK;
  }
  if (N == 0) return MXFP4MOE_OK;
  if (host_blocks == nullptr || host_scales == nullptr || out_bf16 == nullptr) return MXFP4MOE_ERR_ARG;
  if (*staging_bytes < need) return MXFP4MOE_ERR_WORKSPACE;
  if (((uintptr_t)staging & (kAlign - 1)) != 0 || !aligned16(out_bf16)) return MXFP4MOE_ERR_ALIGN;
  hipError_t err = launch_dequant_from_host(host_blocks, host_scales, out_bf16, N, K,
                                            static_cast<uint8_t*>(staging), (hipStream_t)stream);
  return err == hipSuccess ? MXFP4MOE_OK : MXFP4MOE_ERR_HIP;
}

int moe_mxfp4_route(const float* router_logits, int64_t T, int64_t E, int64_t top_k, int32_t* topk_ids,
                    float* topk_weights, int32_t* expert_offsets, int32_t* sorted_pairs, void* stream) {
  int st = check_route_shape(T, E, top_k);
  if (st != MXFP4MOE_OK) return st;
  if (expert_offsets == nullptr) return MXFP4MOE_ERR_ARG;
  if (T > 0 && (router_logits == nullptr || topk_ids == nullptr || topk_weights == nullptr ||
                sorted_pairs == nullptr))
    return MXFP4MOE_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_route(router_logits, (int)T, (int)E, (int)top_k, topk_ids, topk_weights, s);
  if (err == hipSuccess)
    err = launch_group(topk_ids, (int)(T * top_k), (int)E, expert_offsets, sorted_pairs, TileTables{}, s);
  return err == hipSuccess ? MXFP4MOE_OK : MXFP4MOE_ERR_HIP;
}

int moe_mxfp4_forward(const uint16_t* x, const float* router_logits, const uint8_t* w13_blocks,
                      const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_blocks,
                      const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* y, int64_t T, int64_t H,
                      int64_t I, int64_t E, int64_t top_k, void* workspace, size_t* workspace_bytes,
                      void* stream) {
  return moe_mxfp4_forward_ex(x, router_logits, w13_blocks, w13_scales, w13_bias, w2_blocks, w2_scales, w2_bias, y,
                              T, H, I, E, top_k, 0u, workspace, workspace_bytes, stream);
}

int moe_mxfp4_forward_noalloc(const uint16_t* x, const float* router_logits, const uint8_t* w13_blocks,
                              const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_blocks,
                              const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* y, int64_t T, int64_t H,
                              int64_t I, int64_t E, int64_t top_k, void* stream) {
  // every host check first, against a stand-in scratch address that nothing
  // dereferences (the check-only pass launches nothing)
  size_t have = kNoAllocScratch;
  int st = forward_impl(x, router_logits, nullptr, nullptr, w13_blocks, w13_scales, nullptr, w13_bias, w2_blocks,
                        w2_scales, nullptr, w2_bias, y, T, H, I, E, top_k, 0u, reinterpret_cast<void*>(kAlign),
                        &have, stream, /*check_only=*/true);
  if (st == MXFP4MOE_ERR_WORKSPACE) return MXFP4MOE_ERR_SCRATCH;
  if (st != MXFP4MOE_OK || T == 0) return st;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return MXFP4MOE_ERR_HIP;
  return forward_impl(x, router_logits, nullptr, nullptr, w13_blocks, w13_scales, nullptr, w13_bias, w2_blocks,
                      w2_scales, nullptr, w2_bias, y, T, H, I, E, top_k, 0u, ws, &have, stream);
}

int moe_mxfp4_forward_ex(const uint16_t* x, const float* router_logits, const uint8_t* w13_blocks,
                         const uint8_t* w13_scales, const uint16_t* w13_bias, const uint8_t* w2_blocks,
                         const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* y, int64_t T, int64_t H,
                         int64_t I, int64_t E, int64_t top_k, uint32_t flags, void* workspace,
                         size_t* workspace_bytes, void* stream) {
  if ((flags & ~kForwardFlags) != 0) return MXFP4MOE_ERR_ARG;
  return forward_impl(x, router_logits, nullptr, nullptr, w13_blocks, w13_scales, nullptr, w13_bias, w2_blocks,
                      w2_scales, nullptr, w2_bias, y, T, H, I, E, top_k, flags, workspace, workspace_bytes, stream);
}

int moe_nvfp4_forward(const uint16_t* x, const float* router_logits, const uint8_t* w13_blocks,
                      const uint8_t* w13_scales, const float* w13_scale2, const uint16_t* w13_bias,
                      const uint8_t* w2_blocks, const uint8_t* w2_scales, const float* w2_scale2,
                      const uint16_t* w2_bias, uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E,
                      int64_t top_k, void* workspace, size_t* workspace_bytes, void* stream) {
  if (workspace != nullptr && (w13_scale2 == nullptr || w2_scale2 == nullptr)) return MXFP4MOE_ERR_ARG;
  if (((uintptr_t)w13_scale2 & 3u) != 0 || ((uintptr_t)w2_scale2 & 3u) != 0) return MXFP4MOE_ERR_ALIGN;
  return forward_impl(x, router_logits, nullptr, nullptr, w13_blocks, w13_scales, w13_scale2 ? w13_scale2 : &kNvQuery,
                      w13_bias,
                      w2_blocks, w2_scales, w2_scale2 ? w2_scale2 : &kNvQuery, w2_bias, y, T, H, I, E, top_k, 0u,
                      workspace, workspace_bytes, stream);
}

int moe_mxfp8_quantize(const uint16_t* src, int64_t rows, int64_t K, int split, uint8_t* codes, uint8_t* scales,
                       void* stream) {
  if (rows < 0 || K <= 0 || (K & 31) != 0 || K > ((int64_t)1 << 30) || rows > ((int64_t)1 << 40) / K)
    return MXFP4MOE_ERR_SHAPE;
  if (rows > (int64_t)0x7fffffff) return MXFP4MOE_ERR_SHAPE;  // the kernel counts rows in int
  if (rows == 0) return MXFP4MOE_OK;
  if (src == nullptr || codes == nullptr || scales == nullptr) return MXFP4MOE_ERR_ARG;
  if (!aligned16(src) || !aligned16(codes) || ((uintptr_t)scales & 3u) != 0) return MXFP4MOE_ERR_ALIGN;
  hipError_t err = launch_act_quant(src, (int)rows, (int)K, split != 0, codes, scales, (hipStream_t)stream);
  return err == hipSuccess ? MXFP4MOE_OK : MXFP4MOE_ERR_HIP;
}

int moe_mxfp4_router(const uint16_t* x, const uint16_t* router_w, const uint16_t* router_b, int64_t T, int64_t H,
                     int64_t E, int64_t top_k, float* logits, int32_t* topk_ids, float* topk_weights, void* stream) {
  int st = check_route_shape(T, E, top_k);
  if (st != MXFP4MOE_OK) return st;
  if (H <= 0 || (H & 31) != 0) return MXFP4MOE_ERR_SHAPE;
  if (T == 0) return MXFP4MOE_OK;
  if (x == nullptr || router_w == nullptr || router_b == nullptr || logits == nullptr || topk_ids == nullptr ||
      topk_weights == nullptr)
    return MXFP4MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(router_w)) return MXFP4MOE_ERR_ALIGN;
  hipError_t err = launch_route_proj(x, router_w, router_b, (int)T, (int)H, (int)E, (int)top_k, logits, topk_ids,
                                     topk_weights, (hipStream_t)stream);
  return err == hipSuccess ? MXFP4MOE_OK : MXFP4MOE_ERR_HIP;
}

int moe_mxfp4_forward_router(const uint16_t* x, const uint16_t* router_w, const uint16_t* router_b,
                             const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                             const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias, uint16_t* y,
                             int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, uint32_t flags,
                             void* workspace, size_t* workspace_bytes, void* stream) {
  if ((flags & ~kForwardFlags) != 0) return MXFP4MOE_ERR_ARG;
  if (workspace != nullptr && T > 0 && router_w == nullptr) return MXFP4MOE_ERR_ARG;
  static const uint16_t kRouterQuery = 0;  // stands in for the router pointers of a size query
  return forward_impl(x, nullptr, router_w ? router_w : &kRouterQuery, router_b, w13_blocks, w13_scales, nullptr,
                      w13_bias, w2_blocks, w2_scales, nullptr, w2_bias, y, T, H, I, E, top_k, flags, workspace,
                      workspace_bytes, stream);
}

int mxfp4moe_profile_begin(int stage, int max_calls) {
  if (stage < kStageRoute || stage > kStageLast || max_calls < 1 || max_calls > 100000)
    return MXFP4MOE_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (hipEvent_t ev : g_prof_start) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : g_prof_stop) (void)hipEventDestroy(ev);
  g_prof_start.assign(max_calls, nullptr);
  g_prof_stop.assign(max_calls, nullptr);
  for (int i = 0; i < max_calls; ++i) {
    if (hipEventCreate(&g_prof_start[i]) != hipSuccess || hipEventCreate(&g_prof_stop[i]) != hipSuccess) {
      g_prof_stage = kStageNone;
      return MXFP4MOE_ERR_HIP;
    }
  }
  g_prof_next = 0;
  g_prof_stage = stage;
  return MXFP4MOE_OK;
}

int mxfp4moe_profile_end(float* ms, int capacity) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int n = g_prof_next;
  int stored = 0;
  int status = MXFP4MOE_OK;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(g_prof_stop[i]) != hipSuccess) {
      status = MXFP4MOE_ERR_HIP;
      break;
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof_start[i], g_prof_stop[i]) != hipSuccess) {
      status = MXFP4MOE_ERR_HIP;
      break;
    }
    if (ms != nullptr && stored < capacity) ms[stored++] = t;
  }
  for (hipEvent_t ev : g_prof_start) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : g_prof_stop) (void)hipEventDestroy(ev);
  g_prof_start.clear();
  g_prof_stop.clear();
  g_prof_stage = kStageNone;
  g_prof_next = 0;
  return status == MXFP4MOE_OK ? stored : status;
}

}  // extern "C"
