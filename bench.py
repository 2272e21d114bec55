#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

A step is one moe_mxfp4_forward call (routing, grouping, gate_up GEMM with
bias and clamped SwiGLU, down GEMM with bias and routing weight, combine) over
one batch of synthetic tokens whose inputs are already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  Workloads: 120b_prefill (default: gpt-oss-120b shaped
layer, T=4096 long prefill with Zipf-skewed routing), 20b_prefill, 20b_decode,
tiny, dequant_120b (the standalone dequant of both 120b-shaped expert banks),
dequant_host_120b (the w13 bank dequantized on copy from page-locked host
memory) and copy (a plain 1 GiB device copy: the achievable-bandwidth
reference that also calibrates the HBM byte counters).

The default run (120b_prefill without --only) also times the 20b decode layer
(T=4) and the dequant of the 120b banks, each in a timed region of its own
after the headline one, and reports them under config.decode_20b and
config.dequant_120b; `value` stays the 120b long prefill's tokens/s.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s & prefill MFMA TFLOP/s vs MI355X peak"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(H, I, nvfp4=False):
    """Packed bytes of one expert: (gate_up blocks+scales+bias, down blocks+scales+bias).
    MXFP4: one scale byte per 32 elements; NVFP4: one per 16 plus a float32 second-level scale."""
    g = 16 if nvfp4 else 32
    extra = 4 if nvfp4 else 0
    w13 = 2 * I * (H // 2) + 2 * I * (H // g) + 2 * I * 2 + extra
    w2 = H * (I // 2) + H * (I // g) + H * 2 + extra
    return w13, w2


def tile_kinds(counts, T, H, I, E, k, nvfp4=False, act="bf16"):
    """Which pairs each GEMM kernel takes, by the library's tile policy.

    Returns (full_pairs, mid_pairs, mid_experts): pairs of the experts in
    128-pair tiles, and pairs / experts on mid tiles.  Experts with at least
    128 pairs take full tiles; the rest with more than 4 pairs mid tiles; the
    rest one streaming tile.  Batches of 5..256 tokens with exact bf16
    activations take no full tiles, and when they average at least 16 pairs
    per expert no streaming tiles either; NVFP4 layers take full tiles only
    when H and I are multiples of 64.
    """
    import numpy as np

    counts = np.asarray(counts)
    small = act == "bf16" and 4 < T <= 256
    mid_only = small and T * k >= 16 * E
    wide_tiles = (not nvfp4 or (H % 64 == 0 and I % 64 == 0)) and not small
    full_pairs = int(counts[counts >= 128].sum()) if wide_tiles else 0
    sel = (counts > 0) if mid_only else (counts > 4) & ((counts < 128) | (not wide_tiles))
    return full_pairs, int(counts[sel].sum()), int(sel.sum())


def measured_traffic(workload, kernel_tag):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain copy of
    known size), or None when the GEMM source has changed since they were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    ent = rec["kernels"].get(f"{workload}/{kernel_tag}")
    return None if ent is None else float(ent["bytes"])


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline_moe(layer, spec, nvfp4=False, router=False, budget_s=15.0):
    """Time the float64 CPU oracle on the first tokens of the same layer, on one
    core: the process is pinned to one CPU for the run and BLAS/OpenMP pools
    are limited to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import mxfp4_moe as O

    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    n = 1
    elapsed = 0.0
    try:
        with threadpool_limits(limits=1):
            while True:
                tokens = np.arange(min(n, spec.T))
                t0 = time.perf_counter()
                fwd = O.moe_forward_nvfp4 if nvfp4 else O.moe_forward_router if router else O.moe_forward
                fwd(layer, spec.top_k, tokens=tokens)
                elapsed = time.perf_counter() - t0
                if elapsed >= budget_s / 3 or n >= spec.T:
                    break
                n *= 2
    finally:
        os.sched_setaffinity(0, allowed)
    flops = 6.0 * spec.H * spec.I * spec.top_k * len(tokens)
    return {
        "value": len(tokens) / elapsed,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "gflops": flops / elapsed / 1e9,
        "cpu": f"1 of {os.cpu_count()} host cores ({cpu_model()}), pinned to core {core}",
        "sample": f"first {len(tokens)} of {spec.T} tokens of the same layer through the float64 numpy "
                  f"oracle, one thread, {elapsed:.1f} s",
    }


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth of a plain device copy (read + write bytes / time)."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    stop.synchronize()
    ms = start.elapsed_time(stop) / reps
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9, ms


def per_call_spread(call, n):
    """Median, p10 and p90 (ms) of n calls call(i), each between two HIP events on
    the current stream; an untimed pass after the timed region."""
    import numpy as np
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (ea, eb) in enumerate(evs):
        ea.record()
        call(i)
        eb.record()
    torch.cuda.synchronize()
    t = np.array([ea.elapsed_time(eb) for ea, eb in evs])
    return {"calls": int(t.size), "median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90))}


def run_moe(args):
    import numpy as np
    import torch

    from mxfp4_quantized_expert_amd import binding, workloads

    torch.cuda.synchronize()
    nvfp4 = args.workload.startswith("nvfp4_")
    router = args.workload.startswith("router_")
    base = args.workload[len("nvfp4_"):] if nvfp4 else args.workload[len("router_"):] if router else args.workload
    spec = workloads.LAYERS[base]
    T, H, I, E, k = spec.T, spec.H, spec.I, spec.E, spec.top_k
    P = T * k
    log(f"[bench] generating {args.workload}: T={T} H={H} I={I} E={E} k={k}")
    layer = workloads.make_nvfp4_layer(spec) if nvfp4 else workloads.make_layer(spec)
    if router:  # logits from the router projection of x (the skew rides the router bias)
        layer.update(workloads.make_router(spec))
    dev = binding.layer_to_device(layer, "cuda")
    # Expert loads from the library's own routing (used for the roofline accounting).
    if router:
        dev["router_logits"] = binding.moe_mxfp4_router(dev["x"], dev["router_w"], dev["router_b"], k)[0]
    _, _, offsets, _ = binding.moe_mxfp4_route(dev["router_logits"], k)
    counts = np.diff(offsets.cpu().numpy().astype(np.int64))
    n_active = int((counts > 0).sum())
    full_pairs, mid_pairs, mid_experts = tile_kinds(counts, T, H, I, E, k, nvfp4, args.act)
    w13_b, w2_b = layer_bytes(H, I, nvfp4)
    # Weight copies rotate so that repeated steps cannot be served from the
    # 256 MB Infinity Cache when the active weights would fit in it.
    active_bytes = n_active * (w13_b + w2_b)
    copies = 1 if active_bytes > 512e6 else max(2, int(np.ceil(1.2e9 / (E * (w13_b + w2_b)))))
    weight_sets = [dev]
    for _ in range(copies - 1):
        weight_sets.append({kk: (v.clone() if kk.startswith("w") else v) for kk, v in dev.items()})
    torch.cuda.synchronize()
    if args.act != "bf16" and (nvfp4 or router):
        raise SystemExit("--act applies to the MXFP4 workloads with logits input")
    ws = torch.empty((binding.workspace_bytes(T, H, I, E, k, binding.ACT_FLAGS[args.act]),), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step(i):
        d = weight_sets[i % copies]
        if router:
            binding.moe_mxfp4_forward_router(dev["x"], dev["router_w"], dev["router_b"], d["w13_blocks"],
                                             d["w13_scales"], d["w13_bias"], d["w2_blocks"], d["w2_scales"],
                                             d["w2_bias"], k, out=y, workspace=ws)
        elif nvfp4:
            binding.moe_nvfp4_forward(dev["x"], dev["router_logits"], d["w13_blocks"], d["w13_scales"],
                                      d["w13_scale2"], d["w13_bias"], d["w2_blocks"], d["w2_scales"],
                                      d["w2_scale2"], d["w2_bias"], k, out=y, workspace=ws)
        else:
            binding.moe_mxfp4_forward(dev["x"], dev["router_logits"], d["w13_blocks"], d["w13_scales"],
                                      d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_bias"], k,
                                      out=y, workspace=ws, act=args.act)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Stage breakdown (untimed diagnostics, run before the timed region so that
    # the timed steps also start with the GPU at its steady clock).
    stages = {}
    for st in ["route", "group", "act_quant", "gate_up", "gate_up_wide", "gate_up_mid", "gate_up_stream", "down",
               "down_wide", "down_mid", "down_stream", "combine"]:
        binding.profile_begin(st, 5)
        for i in range(5):
            step(i)
        torch.cuda.synchronize()
        got = binding.profile_end(5)
        stages[st] = float(np.mean(got)) if got else 0.0
    log("[bench] stage ms: " + ", ".join(f"{s}={v:.4f}" for s, v in stages.items()))

    # The dominant kernel: gate_up over full 128-pair tiles when there are any,
    # else gate_up over the streamed tiles.  Its launches inside the timed
    # region are bracketed with HIP events on the stream they run on.
    dominant = "gate_up_wide" if full_pairs > 0 else "gate_up_stream" if T <= 4 else "gate_up_mid"
    if args.graph:
        # One captured step per weight set, replayed in the timed region; the
        # dominant launch is timed on eager steps just before (its events
        # cannot be recorded inside replays).
        binding.profile_begin(dominant, args.steps)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        dom_ms = binding.profile_end(args.steps)
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        binding.profile_begin(dominant, args.steps)
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        dom_ms = binding.profile_end(args.steps)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = T / (ms_per_step / 1e3)
    kms = float(np.mean(dom_ms))

    # per-call spread of eager calls, or of replays with --graph
    per_call = per_call_spread((lambda i: graphs[i % copies].replay()) if args.graph else step, args.steps)

    copy_gbs, _ = copy_bandwidth()

    flops_total = 6.0 * H * I * P
    # The mid launch is priced against whichever roof is lower for its work:
    # its experts' packed w13 once from HBM, or 2*H*2I MFMA FLOPs per pair.
    mid_mfma = (dominant == "gate_up_mid" and
                4.0 * H * I * mid_pairs / (PEAK_BF16_TFLOPS * 1e12) > mid_experts * w13_b / (PEAK_HBM_GBS * 1e9))
    if dominant == "gate_up_wide" or mid_mfma:
        # 2*H*2I FLOPs per pair, over the pairs of the tiles of that launch
        tile_pairs = full_pairs if dominant == "gate_up_wide" else mid_pairs
        work = 4.0 * H * I * tile_pairs
        # the FP4 scaled-MFMA path runs at the FP8 rate (fp4 x fp8 operands)
        peak = PEAK_FP8_TFLOPS if args.act != "bf16" and dominant == "gate_up_wide" else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": work / (kms / 1e3) / 1e12, "peak": peak, "unit": "TFLOP/s"}
        per_unit = (f"{4 * H * I:,} FLOPs per pair (2*H*2I) x {tile_pairs} pairs in "
                    + ("128-pair tiles" if dominant == "gate_up_wide" else "mid tiles of at most 48 pairs"))
    else:
        # packed w13 (blocks, scales, bias) of every active expert + x rows + a rows out
        # (the streaming or the mid launch carries every expert of a small batch)
        if dominant == "gate_up_mid":
            n_exp, rows_in, rows_out = mid_experts, mid_pairs * H * 2, mid_pairs * I * 2
        else:
            n_exp, rows_in, rows_out = n_active, T * H * 2, P * I * 2
        work = n_exp * w13_b + rows_in + rows_out
        per_unit = f"{w13_b} B of packed w13 per expert x {n_exp} + x {rows_in} B + a {rows_out} B"
        roof = {"bound": "hbm", "achieved": work / (kms / 1e3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(args.workload, dominant)
    roof["kernel"] = {"gate_up_wide": ("expert_fp4_kernel" if args.act != "bf16" else "expert_wide_kernel")
                                       + " (gate_up, full 128-pair tiles)",
                      "gate_up_mid": "expert_mid_kernel (gate_up, tiles of at most 48 pairs)",
                      "gate_up_stream": "expert_stream_kernel (gate_up, tiles of at most 4 pairs)"}[dominant]
    roof["kernel_ms"] = kms
    roof["algorithmic"] = per_unit
    layer_tflops = flops_total / (ms_per_step / 1e3) / 1e12
    # active experts' packed weights, scales and biases + x + logits + y
    alg_bytes = active_bytes + T * H * 2 + T * E * 4 + T * H * 2
    log(f"[bench] per call: median {per_call['median']:.4f} ms, p10 {per_call['p10']:.4f}, "
        f"p90 {per_call['p90']:.4f} ({per_call['calls']} calls)")
    log(f"[bench] {args.workload}: {ms_per_step:.4f} ms/step, {value:.1f} tokens/s, "
        f"layer {layer_tflops:.1f} TFLOP/s, active experts {n_active}, weight bytes {active_bytes / 1e6:.1f} MB "
        f"-> {alg_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s; copies {copies}; copy kernel {copy_gbs:.0f} GB/s")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.act == "bf16" else "fp4 x fp8 (full tiles), bf16 (remainder tiles)",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {'NVFP4' if nvfp4 else 'MXFP4'} MoE expert layer T={T} H={H} I={I} E={E} "
                        f"top_k={k}" + (", router projection fused ahead of the top-k" if router else "")
                        + (f", Zipf({spec.zipf_s}) routing skew" if spec.zipf_s else ""),
            "T": T, "H": H, "I": I, "E": E, "top_k": k,
            "weights": ("nvfp4 (e2m1 codes, e4m3 scale per 16, fp32 second-level scale)" if nvfp4 else
                        "mxfp4 (e2m1 codes, e8m0 scale per 32)") + ", bf16 MFMA, fp32 accumulate",
            "activations": {"bf16": "bf16 (exact products)",
                            "mxfp8_split": "experts with >= 128 pairs: MXFP8 + residual MXFP8 on the FP4 x FP8 "
                                           "block-scaled MFMA (opt-in; ~1.7e-3 from the exact layer)",
                            "mxfp8": "experts with >= 128 pairs: one MXFP8 tensor on the FP4 x FP8 block-scaled "
                                     "MFMA (opt-in; up to ~21 % from the exact layer)"}[args.act],
            "active_experts": n_active,
            "pairs_in_full_tiles": full_pairs,
            "weight_copies_rotated": copies,
            "hip_graph": bool(args.graph),
            "layer_tflops": layer_tflops,
            "layer_frac_bf16_peak": layer_tflops / PEAK_BF16_TFLOPS,
            "layer_frac_fp4_peak": layer_tflops / PEAK_FP4_TFLOPS,
            "layer_algorithmic_gbs": alg_bytes / (ms_per_step / 1e3) / 1e9,
            "layer_frac_hbm_peak": alg_bytes / (ms_per_step / 1e3) / 1e9 / PEAK_HBM_GBS,
            "hbm_copy_gbs": copy_gbs,
            "stage_ms": stages,
            "per_call_ms": per_call,
        },
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_moe(layer, spec, nvfp4, router)
    return out


def run_dequant_host(args):
    """Dequant-on-copy of a 120b-shaped w13 bank held in page-locked host memory."""
    import numpy as np
    import torch

    from mxfp4_quantized_expert_amd import binding, workloads

    bank = workloads.DEQUANT_BANK_120B[0]
    blocks, scales = workloads.make_bank(bank)
    hb = torch.from_numpy(blocks).pin_memory()
    hs = torch.from_numpy(scales).pin_memory()
    out = torch.empty(blocks.shape[:-1] + (bank.K,), dtype=torch.bfloat16, device="cuda")
    N = bank.E * bank.N
    staging = torch.empty((binding.offload_staging_bytes(N, bank.K),), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        binding.mxfp4_dequantize_from_host(hb, hs, out=out, staging=staging)
    torch.cuda.synchronize()
    n_chunks = -(-N // max(1, (16 << 20) // (bank.K // 2 + bank.K // 32)))
    binding.profile_begin("dequant", args.steps * n_chunks)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        binding.mxfp4_dequantize_from_host(hb, hs, out=out, staging=staging)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms = binding.profile_end(args.steps * n_chunks)
    ms = (t1 - t0) * 1e3 / args.steps
    host_bytes = blocks.nbytes + scales.nbytes
    chunk_rows = N // n_chunks
    kernel_bytes = chunk_rows * (bank.K // 2 + bank.K // 32 + bank.K * 2)
    kmean = float(np.mean(kms))
    # the plain page-locked host -> device copy of the same packed bytes: the PCIe bound
    db = torch.empty(hb.shape, dtype=torch.uint8, device="cuda")
    ds = torch.empty(hs.shape, dtype=torch.uint8, device="cuda")
    db.copy_(hb, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        db.copy_(hb, non_blocking=True)
        ds.copy_(hs, non_blocking=True)
    torch.cuda.synchronize()
    h2d_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del db, ds
    return {
        "metric": "mxfp4 dequant-on-copy from host memory, host GB/s",
        "value": host_bytes / (ms / 1e3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8->bf16", "data": "synthetic",
        "config": {"workload": f"dequant-on-copy of a gpt-oss-120b shaped w13 bank {list(blocks.shape)} from "
                               f"page-locked host memory, {n_chunks} chunks through two staging slots",
                   "output_gbs": out.numel() * 2 / (ms / 1e3) / 1e9,
                   "plain_h2d_copy_ms": h2d_ms,
                   "plain_h2d_copy_gbs": host_bytes / (h2d_ms / 1e3) / 1e9,
                   "frac_of_plain_h2d": h2d_ms / ms},
        "roofline": {"bound": "hbm", "achieved": kernel_bytes / (kmean / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": kernel_bytes / (kmean / 1e3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "mxfp4_dequant_kernel (one chunk)", "kernel_ms": kmean},
    }


def run_copy(args):
    gbs, ms = copy_bandwidth(reps=args.steps)
    return {"metric": "device copy GB/s", "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": 2, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "u8", "data": "synthetic",
            "config": {"workload": "copy of a 1 GiB device buffer (torch copy kernel), read + write bytes"}}


def run_dequant(args):
    """mxfp4_dequantize of both gpt-oss-120b shaped expert banks (w13 [128, 5760, 2880]
    and w2 [128, 2880, 2880]); a step dequantizes both."""
    import numpy as np
    import torch

    from mxfp4_quantized_expert_amd import binding, workloads

    banks = []
    for bank in workloads.DEQUANT_BANK_120B:
        blocks, scales = workloads.make_bank(bank)
        banks.append((blocks, scales, torch.from_numpy(blocks).cuda(), torch.from_numpy(scales).cuda(),
                      torch.empty(blocks.shape[:-1] + (bank.K,), dtype=torch.bfloat16, device="cuda")))

    def step(_=None):
        for _, _, b, s, out in banks:
            binding.mxfp4_dequantize(b, s, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    binding.profile_begin("dequant", 2 * args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms = 2 * float(np.mean(binding.profile_end(2 * args.steps)))  # both banks, kernel time
    ms = (t1 - t0) * 1e3 / args.steps
    nbytes = sum(bl.nbytes + sc.nbytes + out.numel() * 2 for bl, sc, _, _, out in banks)
    elements = sum(out.numel() for *_, out in banks)
    per_call = per_call_spread(step, args.steps)
    res = {
        "metric": "mxfp4_dequantize HBM GB/s",
        "value": nbytes / (ms / 1e3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8->bf16", "data": "synthetic",
        "config": {"workload": "dequant of both gpt-oss-120b shaped expert banks, w13 "
                               f"{list(banks[0][0].shape)} and w2 {list(banks[1][0].shape)} packed -> bf16",
                   "elements": elements, "bytes_per_step": nbytes, "per_call_ms": per_call},
        "roofline": {"bound": "hbm", "achieved": nbytes / (kms / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (kms / 1e3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "mxfp4_dequant_kernel", "kernel_ms": kms,
                     "algorithmic": "2.53125 B per element (0.5 packed + 1/32 scale + 2 bf16 out) x "
                                    f"{elements} elements"},
    }
    if not args.no_cpu_baseline:
        from oracle import mxfp4_moe as O
        blocks, scales = banks[0][0], banks[0][1]
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 10.0 and n < blocks.shape[0]:
            O.mxfp4_dequantize(blocks[n], scales[n])
            n += 1
        el = time.perf_counter() - t0
        per = (blocks[0].nbytes + scales[0].nbytes + blocks[0].size * 4)
        res["cpu_baseline"] = {"value": n * per / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {blocks.shape[0]} w13 experts, numpy oracle, {el:.1f} s"}
    return res


def compact(res):
    """The figures of a secondary workload that go into the headline line's config."""
    out = {"workload": res["config"]["workload"], "metric": res["metric"], "value": res["value"],
           "unit": res["unit"], "ms_per_step": res["ms_per_step"], "steps": res["steps"]}
    for key in ("per_call_ms", "layer_algorithmic_gbs", "layer_frac_hbm_peak", "active_experts", "stage_ms",
                "weight_copies_rotated"):
        if key in res["config"]:
            out[key] = res["config"][key]
    r = res.get("roofline")
    if r is not None:
        out["roofline"] = {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac", "kernel", "kernel_ms")
                           if k in r}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="120b_prefill",
                    choices=["120b_prefill", "20b_prefill", "20b_decode", "tiny", "nvfp4_20b_decode",
                             "nvfp4_20b_prefill", "nvfp4_120b_prefill", "router_20b_decode", "router_120b_prefill",
                             "dequant_120b", "dequant_host_120b", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="measure the named workload alone (the default run also times the 20b decode layer "
                         "and the 120b dequant after the 120b long prefill)")
    ap.add_argument("--decode-steps", type=int, default=400,
                    help="timed calls of the 20b decode layer in the default run")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of one layer call instead of eager calls")
    ap.add_argument("--act", default="bf16", choices=["bf16", "mxfp8_split", "mxfp8"],
                    help="activations of the full 128-pair tiles: exact bf16 (default) or the opt-in "
                         "FP4 scaled-MFMA path over MXFP8 activations")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload == "dequant_120b":
        res = run_dequant(args)
    elif args.workload == "dequant_host_120b":
        res = run_dequant_host(args)
    elif args.workload == "copy":
        res = run_copy(args)
    else:
        res = run_moe(args)
        if args.workload == "120b_prefill" and not args.only and args.act == "bf16" and not args.graph:
            # the decode half of the metric and the dequant, each in a timed region of its own
            sub = argparse.Namespace(**vars(args))
            sub.workload, sub.steps, sub.warmup, sub.no_cpu_baseline = "20b_decode", args.decode_steps, 10, True
            res["config"]["decode_20b"] = compact(run_moe(sub))
            sub.workload, sub.steps, sub.warmup = "dequant_120b", 5, 2
            res["config"]["dequant_120b"] = compact(run_dequant(sub))
            d = res["config"]["decode_20b"]
            log(f"[bench] 20b decode: {d['ms_per_step'] * 1e3:.1f} us/call, {d['layer_algorithmic_gbs']:.0f} GB/s "
                f"({100 * d['layer_frac_hbm_peak']:.1f} % of HBM peak); dequant "
                f"{res['config']['dequant_120b']['value']:.0f} GB/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
