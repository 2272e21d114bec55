/*
 * mxfp4moe.h - C ABI of libmxfp4moe.so, the MI355X (gfx950) MXFP4
 * mixture-of-experts expert FFN and the standalone MXFP4 dequant.
 *
 * All tensors are row-major and contiguous.  Every pointer argument that names
 * a tensor is DEVICE memory owned by the caller; the library never allocates,
 * frees or keeps a pointer after a call returns.  `stream` is a hipStream_t
 * (NULL = the default stream).  Every call only enqueues work on `stream` and
 * returns without synchronising; results are valid once the caller has
 * synchronised that stream.  Arguments are checked on the host before any
 * launch: on a non-zero return nothing was launched and nothing was written.
 * Faults inside kernels surface at the caller's next synchronisation.
 *
 * Formats (OCP Microscaling Formats v1.0):
 *   blocks : uint8, two E2M1 codes per byte; element 2i of a row is the low
 *            nibble of byte i, element 2i+1 the high nibble.  E2M1 magnitudes
 *            are 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, bit 3 is the sign.
 *   scales : uint8 E8M0, one per 32 consecutive elements of a row (one
 *            16-byte block); value 2^(s-127).  0xFF means NaN.
 *   bf16   : uint16 bit patterns.
 */
#ifndef MXFP4MOE_H
#define MXFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MXFP4MOE_OK 0
#define MXFP4MOE_ERR_ARG (-1)       /* NULL pointer or otherwise invalid argument          */
#define MXFP4MOE_ERR_SHAPE (-2)     /* sizes out of range or not multiples of 32           */
#define MXFP4MOE_ERR_WORKSPACE (-3) /* workspace smaller than the size the query returned   */
#define MXFP4MOE_ERR_ALIGN (-4)     /* a pointer is not aligned as its call requires        */
#define MXFP4MOE_ERR_HIP (-5)       /* the HIP runtime rejected a launch                   */
#define MXFP4MOE_ERR_SCRATCH (-6)   /* the layer needs more than the no-allocation scratch  */

/* Largest supported expert count and top_k. */
#define MXFP4MOE_MAX_EXPERTS 512
#define MXFP4MOE_MAX_TOPK 32
#define MXFP4MOE_MAX_HIDDEN 4096 /* bound on H and I: the GEMMs stage a tile's scale rows in LDS */

/*
 * mxfp4_dequantize - "dequant-on-copy": expand packed MXFP4 rows to bf16.
 *
 * Defined by "feat(gpt-oss): expert offloading Phase 2 - MXFP4 dequant-on-copy
 * execution" (MoE-Infinity PR #152), Changes: packed experts are dequantized
 * to bf16, bit-exactly (its golden test reports relative error 0.0); the row
 * layout is [N, K//2] (numerical review).  Block layout [E, N, K/32, 16] with
 * one E8M0 byte per block: "Add native GPT-OSS MXFP4 QMoE export" (mobius
 * PR #719), Summary.
 *
 *   blocks   [N, K/2]  uint8, 16-byte aligned
 *   scales   [N, K/32] uint8
 *   out_bf16 [N, K]    uint16 (bf16 bits), 16-byte aligned, must not overlap the inputs
 *   N >= 0 rows (leading dimensions flatten into N: a bank [E, Nr, K/2] passes N = E*Nr);
 *   K > 0, a multiple of 32.
 *
 * out[n, k] = bf16_rne(E2M1(code[n, k]) * 2^(scales[n, k/32] - 127)).  This is
 * exact for scale bytes up to 252; 253 and 254 overflow the largest codes to
 * +-inf; 0xFF writes 0x7FC0 for the whole 32-element group.  N == 0 is a no-op.
 * Returns MXFP4MOE_OK or a negative status.
 */
int mxfp4_dequantize(const uint8_t* blocks, const uint8_t* scales, uint16_t* out_bf16,
                     int64_t N, int64_t K, void* stream);

/*
 * mxfp4_dequantize_from_host - dequant-on-copy of packed rows held in host
 * memory: copy to the device and expand to bf16 on arrival.
 *
 * Defined by "feat(gpt-oss): expert offloading Phase 2 - MXFP4 dequant-on-copy
 * execution" (MoE-Infinity PR #152), Changes: offloaded packed experts are
 * copied to the device and dequantized to bf16 there; and "feat(gpt-oss):
 * expert offloading Phase 3" (MoE-Infinity PR #153), description: the six
 * packed components per layer are what is offloaded.
 *
 *   host_blocks [N, K/2]  uint8 in host memory; page-locked memory (e.g.
 *                         hipHostMalloc) lets the copies run asynchronously
 *   host_scales [N, K/32] uint8 in host memory
 *   out_bf16    [N, K]    bf16 bits, device memory, 16-byte aligned
 *   staging     device scratch of at least *staging_bytes bytes, 256-byte
 *               aligned; with staging == NULL the call only stores the size it
 *               needs (two slots of about 16 MiB of packed rows) and returns
 *               MXFP4MOE_OK.
 * Same values as mxfp4_dequantize.  The rows move in chunks: the copy of
 * chunk i+1 runs on a copy stream the library creates once per device
 * (default priority) while chunk i is dequantized on `stream`.  The call
 * returns after enqueueing; the output and the host buffers' use are complete
 * when `stream` is.  The host buffers must stay valid and unmodified until
 * then.  Calls are serialised inside the process (they share the copy
 * stream); two calls must not share one staging buffer unless ordered on one
 * stream.  N == 0 is a no-op.
 */
int mxfp4_dequantize_from_host(const uint8_t* host_blocks, const uint8_t* host_scales, uint16_t* out_bf16,
                               int64_t N, int64_t K, void* staging, size_t* staging_bytes, void* stream);

/*
 * moe_mxfp4_route - the routing data the MXFP4 experts consume: top-k
 * selection, softmax over the k selected logits, and the tokens grouped by
 * expert.
 *
 * Defined by "Restore GPT-OSS's router-masked expert-parallel plan"
 * (transformers PR #49431), description: MXFP4 experts take routing data and
 * route their tokens themselves; and by "feat(gguf): serve gpt-oss gguf
 * checkpoints on gpt_oss" (FreeToken PR #838), "What it does": the
 * expert-ordered prefill views.
 *
 *   router_logits  [T, E] float32 (post router bias)
 *   topk_ids       [T, top_k] int32 out: experts by descending logit; equal
 *                  logits are ordered by the lower expert index
 *   topk_weights   [T, top_k] float32 out: exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *   expert_offsets [E + 1] int32 out: exclusive prefix sum of tokens per expert
 *   sorted_pairs   [T * top_k] int32 out: pair ids p = t*top_k + j sorted by
 *                  (expert, p); expert e owns sorted_pairs[offsets[e] .. offsets[e+1])
 *   1 <= top_k <= min(E, MXFP4MOE_MAX_TOPK), 1 <= E <= MXFP4MOE_MAX_EXPERTS, T >= 0.
 * T == 0 writes offsets of zeros only.  NaN logits give unspecified ids.
 */
int moe_mxfp4_route(const float* router_logits, int64_t T, int64_t E, int64_t top_k,
                    int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                    int32_t* sorted_pairs, void* stream);

/*
 * moe_mxfp4_forward - one gpt-oss MXFP4 MoE expert layer:
 *
 *   (ids, w) = top-k of router_logits, softmax over the k selected logits
 *   for each pair (t, j), e = ids[t, j]:
 *     h    = x[t] W13_e^T + b13_e                 (bias before the activation)
 *     gate = h[0::2], up = h[1::2]                (interleaved rows)
 *     a    = min(gate,7) * sigmoid(1.702*min(gate,7)) * (clamp(up,-7,7) + 1)
 *     z    = a W2_e^T + b2_e                      (bias before the routing weight)
 *   y[t] = bf16_rne( sum_j bf16_rne(w[t, j] * z_(t,j)) )   (sum in fp32, j ascending)
 *
 * Defined by "feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss"
 * (FreeToken PR #838): "What it does" (alpha 1.702 and limit 7, interleaved
 * gate/up, gate/up bias before the gated activation, down bias before the
 * routing weight, required biases) and review items 3 and 4 (sum w*(s*y + b),
 * router weight applied to the output); "feat(gpt-oss): expert offloading
 * Phase 2" (MoE-Infinity PR #152), numerical review (scales, bias, [N, K//2]
 * layout, gate/up split, clamped SwiGLU, fp32 accumulation); the six packed
 * components per layer of "feat(gpt-oss): expert offloading Phase 3"
 * (MoE-Infinity PR #153), description.
 *
 *   x             [T, H] bf16, 16-byte aligned
 *   router_logits [T, E] float32
 *   w13_blocks    [E, 2I, H/2] uint8, 16-byte aligned   (row 2i = gate i, row 2i+1 = up i)
 *   w13_scales    [E, 2I, H/32] uint8, 16-byte aligned
 *   w13_bias      [E, 2I] bf16, 8-byte aligned
 *   w2_blocks     [E, H, I/2] uint8, 16-byte aligned
 *   w2_scales     [E, H, I/32] uint8, 16-byte aligned
 *   w2_bias       [E, H] bf16, 8-byte aligned
 *   y             [T, H] bf16 out, 16-byte aligned, must not alias any input
 *   H, I multiples of 32 in [32, MXFP4MOE_MAX_HIDDEN]; 1 <= E <= MXFP4MOE_MAX_EXPERTS;
 *   1 <= top_k <= min(E, MXFP4MOE_MAX_TOPK); T >= 0.
 *   workspace     device scratch of at least *workspace_bytes bytes, 256-byte aligned.
 *                 If workspace == NULL the call only stores the required size in
 *                 *workspace_bytes and returns MXFP4MOE_OK without launching anything.
 *
 * Biases are required (a NULL bias is MXFP4MOE_ERR_ARG); there is no mode that
 * applies the routing weight to the input.  Accumulation is fp32; the SwiGLU
 * output is rounded to bf16 before the down GEMM, and each weighted pair
 * output w * z to bf16 before the sum over the k pairs.  T == 0 is a no-op.
 * An expert with at least 128 pairs is cut into tiles of 128 (the last one
 * partial), one with 5..127 pairs into ceil(pairs / 48) tiles of near-equal
 * size, one with at most 4 pairs makes one streaming tile; each kind has a
 * GEMM kernel of its own
 * (with T <= 4 every expert has one streaming tile: the decode path, whose
 * routing runs inside the gate_up launch).  Batches of 5..256 tokens take no
 * full tiles (their experts' pairs take mid tiles), and no streaming tiles
 * either when T * top_k >= 16 * E.  The tiling changes which kernel computes
 * a pair, not what is computed.
 *
 * E8M0 byte 0xFF (NaN) in a weight row makes that row's GEMM output NaN for
 * every token of the expert: a 0xFF in gate_up row r of expert e gives NaN in
 * the whole output row of every token routed to e; a 0xFF in down row n gives
 * NaN in column n of those tokens' outputs.  Nothing else changes.  Scale
 * bytes 253 and 254 with the largest codes overflow the bf16 weights to inf
 * (unspecified outputs); 0..252 are exact.
 */
int moe_mxfp4_forward(const uint16_t* x, const float* router_logits,
                      const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                      const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias,
                      uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                      void* workspace, size_t* workspace_bytes, void* stream);

/*
 * moe_mxfp4_forward_noalloc - moe_mxfp4_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument.  Its scratch is a
 * fixed device array inside the library, MXFP4MOE_NOALLOC_SCRATCH_BYTES bytes
 * per device, held by every device the library runs on until the process
 * ends.  The call allocates nothing: no hipMalloc, hipFree or allocating
 * library routine (the first call on a device looks the array's address up
 * once).  The caller still passes x, the logits, the weights and y.
 *
 * Arguments, checks and results as moe_mxfp4_forward, with the same kernels
 * (bit-identical outputs).  A layer whose workspace (the size
 * moe_mxfp4_forward's query returns) exceeds the scratch returns
 * MXFP4MOE_ERR_SCRATCH before any launch: 32 MiB hold about 700 tokens at
 * H = I = 2880, top_k = 4.  Every call on one device shares that device's
 * array, and a call leaves its contents behind for the next (nothing in it is
 * assumed zero at the start of a call): two calls that overlap on one device
 * race.  Order them on one stream, or use moe_mxfp4_forward with separate
 * workspaces.
 */
#define MXFP4MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_mxfp4_forward_noalloc(const uint16_t* x, const float* router_logits,
                              const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                              const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias,
                              uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                              void* stream);

/*
 * moe_mxfp4_forward_ex - moe_mxfp4_forward with layout flags.
 *
 *   flags = 0                       w13 gate/up rows interleaved (row 2i gate i,
 *                                   row 2i+1 up i; bias likewise), as above
 *   flags = MXFP4MOE_GATE_UP_SPLIT  w13 rows [0, I) are gate, [I, 2I) are up
 *                                   (blocks, scales and bias alike)
 * The split layout is the uninterleaved spelling of the same clamped SwiGLU
 * ("feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss", FreeToken PR #838,
 * "What it does": swigluoai with interleaved=False).  Results are identical
 * to the interleaved call on the correspondingly permuted rows.
 *
 *   flags |= MXFP4MOE_ACT_MXFP8_SPLIT  (opt-in approximation) experts with at
 *           least 128 pairs run both GEMMs on the gfx950 block-scaled MFMA
 *           (v_mfma_scale_f32_32x32x64_f8f6f4): packed E2M1 weights with their
 *           E8M0 scales times activations quantized to MXFP8 (E4M3 in blocks
 *           of 32, one E8M0 scale per block, shared exponent
 *           floor(log2 max) - 7 by this library's own rule, round to
 *           nearest even) plus the MXFP8
 *           quantization of the residual; about 1e-3 normwise from the
 *           exact layer on the test layers.  The SwiGLU output is rounded to
 *           bf16, then quantized the same way.
 *   flags |= MXFP4MOE_ACT_MXFP8        the same with a single MXFP8 tensor
 *           (half the MFMAs; 4 to 20 % normwise from the exact layer on the
 *           test layers, outside the 1e-2 bar: for measurement only).
 * Experts with fewer pairs keep the exact bf16 path.  The two ACT flags are
 * exclusive (SPLIT wins); the workspace query must pass the same flags (the
 * quantized activations live in the workspace).  Not available for NVFP4.
 * How a 0xFF scale byte acts on the ACT paths is unspecified.
 *
 *   flags |= MXFP4MOE_TILES_STREAM   every pair in streaming tiles of at most
 *           4 pairs, whatever the expert loads (the decode kernels on every
 *           shape: a check of those kernels, not a faster path).  Same
 *           results within the tolerance of the layer; with it the ACT
 *           flags find no full tiles and change nothing.
 * Any other flag bit is MXFP4MOE_ERR_ARG.
 */
#define MXFP4MOE_GATE_UP_SPLIT 1u
#define MXFP4MOE_ACT_MXFP8 2u
#define MXFP4MOE_ACT_MXFP8_SPLIT 4u
#define MXFP4MOE_TILES_STREAM 8u
int moe_mxfp4_forward_ex(const uint16_t* x, const float* router_logits,
                         const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                         const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias,
                         uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                         uint32_t flags, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * moe_mxfp8_quantize - the activation quantizer of the MXFP4MOE_ACT_* paths,
 * exposed for tests and callers that keep activations in this form.
 *
 *   src     [rows, K] bf16, 16-byte aligned; K a multiple of 32
 *   codes   [rows, 128 * ceil(K/64)] uint8 out, 16-byte aligned: per 64-wide K
 *           chunk c, the 64 E4M3 codes of K [64c, 64c+64), then the 64 codes
 *           of the residual (zeros unless split)
 *   scales  [rows, 4 * ceil(K/64)] uint8 out, 4-byte aligned: per chunk the
 *           E8M0 bytes of groups 2c, 2c+1, then the residual's (127 unless split)
 * A chunk past K (K % 64 == 32) holds zero codes and scale 127.  Encodings
 * (OCP Microscaling Formats v1.0): E4M3 elements in blocks of 32 sharing one
 * E8M0 scale.  The shared exponent floor(log2(max|v|)) - 7 is this library's
 * own choice (the specification subtracts emax = 8 and clamps at 448; one
 * more keeps every scaled value below 256); 127 for an all-zero block;
 * elements round to nearest, ties to even.
 */
int moe_mxfp8_quantize(const uint16_t* src, int64_t rows, int64_t K, int split, uint8_t* codes,
                       uint8_t* scales, void* stream);

/*
 * moe_mxfp4_router - the router projection fused ahead of the top-k:
 *
 *   logits[t, e] = sum_h x[t, h] * router_w[e, h] + router_b[e]   (fp32 accumulation)
 *   (topk_ids, topk_weights) = top-k of logits[t], softmax over the k selected
 *
 * "feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss" (FreeToken PR
 * #838): the cleanups name the router mlp.router (a linear layer), and
 * "What it does" loads the router bias and requires the router input's bias.
 * One launch: each 16-token tile computes its logits on the MFMA into LDS,
 * writes them out, and routes from LDS (same order and ties as
 * moe_mxfp4_route).
 *
 *   x            [T, H] bf16, 16-byte aligned
 *   router_w     [E, H] bf16, 16-byte aligned
 *   router_b     [E] bf16 (required)
 *   logits       [T, E] float32 out
 *   topk_ids     [T, top_k] int32 out;  topk_weights [T, top_k] float32 out
 *   H a multiple of 32; E, top_k as moe_mxfp4_route.  T == 0 is a no-op.
 */
int moe_mxfp4_router(const uint16_t* x, const uint16_t* router_w, const uint16_t* router_b, int64_t T,
                     int64_t H, int64_t E, int64_t top_k, float* logits, int32_t* topk_ids,
                     float* topk_weights, void* stream);

/*
 * moe_mxfp4_forward_router - moe_mxfp4_forward_ex with the logits computed
 * by the router projection of x (as moe_mxfp4_router) instead of passed in.
 * router_w [E, H] bf16 (16-byte aligned) and router_b [E] bf16 are required
 * when T > 0 and a workspace is given; flags as moe_mxfp4_forward_ex; the
 * workspace query and every other argument as moe_mxfp4_forward.
 */
int moe_mxfp4_forward_router(const uint16_t* x, const uint16_t* router_w, const uint16_t* router_b,
                             const uint8_t* w13_blocks, const uint8_t* w13_scales, const uint16_t* w13_bias,
                             const uint8_t* w2_blocks, const uint8_t* w2_scales, const uint16_t* w2_bias,
                             uint16_t* y, int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                             uint32_t flags, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * moe_nvfp4_forward - the same expert layer over NVFP4 experts.
 *
 * "feat(gguf): serve gpt-oss gguf checkpoints on gpt_oss" (FreeToken PR #838),
 * review item 3: NVFP4 experts carry a second-level scale (weight_scale_2)
 * that multiplies the expert's GEMM output before the bias is added, so the
 * layer is y_t = sum_j w_tj * (s2 * (a W2^T) + b2), never sum_j w_tj * s2 * (y + b2);
 * the gate_up GEMM likewise: h = s2_13 * (x W13^T) + b13.  Element format (the
 * public NVFP4 description; the pages name only the format and its second-
 * level scale): E2M1 codes, two per byte, low nibble first, in blocks of 16
 * elements with one FP8 E4M3 scale byte each.
 *
 *   w13_blocks [E, 2I, H/2] uint8, w13_scales [E, 2I, H/16] uint8 (E4M3),
 *   w13_scale2 [E] float32, w2_blocks [E, H, I/2], w2_scales [E, H, I/16],
 *   w2_scale2 [E] float32 (4-byte aligned); everything else as moe_mxfp4_forward
 *   (gate/up rows interleaved, scales 16-byte and biases 8-byte aligned), and
 *   the same workspace query.  An E4M3 NaN scale byte (0x7F, 0xFF) makes its
 *   weights NaN, with the same effect on the outputs as an E8M0 0xFF.
 * Tiles as moe_mxfp4_forward when H and I are multiples of 64; otherwise
 * every pair runs in mid-size or streaming tiles.  A NULL second-level scale
 * with a workspace is MXFP4MOE_ERR_ARG.
 */
int moe_nvfp4_forward(const uint16_t* x, const float* router_logits,
                      const uint8_t* w13_blocks, const uint8_t* w13_scales, const float* w13_scale2,
                      const uint16_t* w13_bias, const uint8_t* w2_blocks, const uint8_t* w2_scales,
                      const float* w2_scale2, const uint16_t* w2_bias, uint16_t* y, int64_t T, int64_t H,
                      int64_t I, int64_t E, int64_t top_k, void* workspace, size_t* workspace_bytes,
                      void* stream);

/* Short English text for a status code (static storage). */
const char* mxfp4moe_status_string(int status);

/*
 * Kernel timing hook for benchmarks.  mxfp4moe_profile_begin(stage, max_calls)
 * makes the next max_calls launches of one kernel stage record a pair of HIP
 * events around that launch, on the stream the kernel runs on.  Stages:
 * 1 route, 2 group, 3 gate_up GEMM, 4 down GEMM, 5 combine, 6 dequant,
 * then single launches of the GEMM stages: 7 / 11 / 8 the full-tile /
 * mid-remainder / streaming launch of gate_up, 9 / 12 / 10 the same for down,
 * 13 the MXFP8 activation quantizer of the ACT flags.
 * mxfp4moe_profile_end(ms, capacity) synchronises on the recorded events,
 * stores up to `capacity` per-launch durations in milliseconds (host array),
 * releases the events and returns how many were stored (negative on error).
 */
int mxfp4moe_profile_begin(int stage, int max_calls);
int mxfp4moe_profile_end(float* ms, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4MOE_H */
