// Dequant-on-copy from host memory ("feat(gpt-oss): expert offloading Phase 2
// - MXFP4 dequant-on-copy execution", MoE-Infinity PR #152, Changes: packed
// experts held in host memory are copied to the device and expanded to bf16
// on arrival; "feat(gpt-oss): expert offloading Phase 3", MoE-Infinity PR
// #153, description: the offloaded experts are the six packed components).
//
// The rows move in chunks through two device staging slots.  The copy of
// chunk i+1 runs on the library's copy stream (the DMA engines) while chunk i
// is dequantized on the caller's stream; events hand each slot back and forth.
#include <mutex>

#include "../../include/mxfp4moe.h"
#include "internal.h"

namespace mxfp4moe {
namespace {

constexpr size_t kChunkBytes = (size_t)16 << 20;  // packed bytes per chunk
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct DeviceCopyState {
  hipStream_t copy = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr};
  hipEvent_t freed[2] = {nullptr, nullptr};
  bool ready = false;
};

std::mutex g_mu;
DeviceCopyState g_state[64];

hipError_t device_state(DeviceCopyState** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DeviceCopyState& st = g_state[dev];
  if (!st.ready) {
    // default priority, non-blocking with respect to the null stream
    err = hipStreamCreateWithFlags(&st.copy, hipStreamNonBlocking);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&st.start, hipEventDisableTiming);
    for (int i = 0; i < 2 && err == hipSuccess; ++i) {
      err = hipEventCreateWithFlags(&st.copied[i], hipEventDisableTiming);
      if (err == hipSuccess) err = hipEventCreateWithFlags(&st.freed[i], hipEventDisableTiming);
    }
    if (err != hipSuccess) return err;
    st.ready = true;
  }
  *out = &st;
  return hipSuccess;
}

}  // namespace

int64_t offload_chunk_rows(int64_t K) {
  const int64_t row_bytes = K / 2 + K / 32;
  const int64_t r = (int64_t)kChunkBytes / row_bytes;
  return r > 0 ? r : 1;
}

size_t offload_staging_bytes(int64_t N, int64_t K) {
  int64_t rows = offload_chunk_rows(K);
  if (rows > N) rows = N;
  return 2 * (align_up((size_t)rows * (size_t)(K / 2)) + align_up((size_t)rows * (size_t)(K / 32)));
}

hipError_t launch_dequant_from_host(const uint8_t* host_blocks, const uint8_t* host_scales, uint16_t* out,
                                    int64_t N, int64_t K, uint8_t* staging, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);  // one pipeline at a time per process: the copy state is shared
  DeviceCopyState* st = nullptr;
  hipError_t err = device_state(&st);
  if (err != hipSuccess) return err;
  const int64_t R = offload_chunk_rows(K) < N ? offload_chunk_rows(K) : N;
  const size_t blk_bytes = align_up((size_t)R * (size_t)(K / 2));
  const size_t slot_bytes = blk_bytes + align_up((size_t)R * (size_t)(K / 32));
  // the first copies wait for the caller's earlier work (it may still use the staging slots)
  err = hipEventRecord(st->start, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(st->copy, st->start, 0);
  const int64_t nchunks = (N + R - 1) / R;
  for (int64_t i = 0; i < nchunks && err == hipSuccess; ++i) {
    const int s = (int)(i & 1);
    const int64_t r0 = i * R;
    const int64_t rows = (N - r0) < R ? (N - r0) : R;
    uint8_t* sb = staging + s * slot_bytes;
    uint8_t* ss = sb + blk_bytes;
    if (i >= 2) err = hipStreamWaitEvent(st->copy, st->freed[s], 0);  // slot s dequantized
    if (err == hipSuccess)
      err = hipMemcpyAsync(sb, host_blocks + r0 * (K / 2), (size_t)rows * (size_t)(K / 2), hipMemcpyHostToDevice,
                           st->copy);
    if (err == hipSuccess)
      err = hipMemcpyAsync(ss, host_scales + r0 * (K / 32), (size_t)rows * (size_t)(K / 32), hipMemcpyHostToDevice,
                           st->copy);
    if (err == hipSuccess) err = hipEventRecord(st->copied[s], st->copy);
    if (err == hipSuccess) err = hipStreamWaitEvent(stream, st->copied[s], 0);
    if (err == hipSuccess) err = launch_dequant(sb, ss, out + r0 * K, rows, K, stream);
    if (err == hipSuccess) err = hipEventRecord(st->freed[s], stream);
  }
  return err;
}

}  // namespace mxfp4moe
