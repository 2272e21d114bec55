#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

A step is one moe_mxfp4_forward call (routing, grouping, gate_up GEMM with
bias and clamped SwiGLU, down GEMM with bias and routing weight, combine) over
one batch of synthetic tokens whose inputs are already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  Workloads: 120b_prefill (default: gpt-oss-120b shaped
layer, T=4096 long prefill with Zipf-skewed routing), 20b_prefill, 20b_decode,
tiny, and dequant_120b (the standalone dequant of a 120b-shaped w13 bank).
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
W13_BYTES_PER_ROW_PER_K = 0.5 + 1.0 / 32.0  # packed nibbles + one E8M0 byte per 32


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(H, I):
    """Packed bytes of one expert: (gate_up blocks+scales+bias, down blocks+scales+bias)."""
    w13 = 2 * I * (H // 2) + 2 * I * (H // 32) + 2 * I * 2
    w2 = H * (I // 2) + H * (I // 32) + H * 2
    return w13, w2


def cpu_baseline_moe(layer, spec, budget_s=15.0):
    """Time the float64 CPU oracle on the first tokens of the same layer."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import mxfp4_moe as O

    n = 1
    elapsed = 0.0
    while True:
        tokens = np.arange(min(n, spec.T))
        t0 = time.perf_counter()
        O.moe_forward(layer, spec.top_k, tokens=tokens)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s / 3 or n >= spec.T:
            break
        n *= 2
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": len(tokens) / elapsed,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {len(tokens)} of {spec.T} tokens of the same layer, float64 numpy oracle, "
                  f"{elapsed:.1f} s",
    }


def run_moe(args):
    import numpy as np
    import torch

    from mxfp4_quantized_expert_amd import binding, workloads
    from oracle import mxfp4_moe as O

    spec = workloads.LAYERS[args.workload]
    T, H, I, E, k = spec.T, spec.H, spec.I, spec.E, spec.top_k
    log(f"[bench] generating {args.workload}: T={T} H={H} I={I} E={E} k={k}")
    layer = workloads.make_layer(spec)
    ids, _ = O.route(layer["router_logits"], k)
    counts = np.bincount(ids.ravel(), minlength=E)
    n_active = int((counts > 0).sum())
    w13_b, w2_b = layer_bytes(H, I)
    # Weight copies rotate so that repeated steps cannot be served from the
    # 256 MB Infinity Cache when the active weights would fit in it.
    active_bytes = n_active * (w13_b + w2_b)
    copies = 1 if active_bytes > 512e6 else max(2, int(np.ceil(1.2e9 / (E * (w13_b + w2_b)))))
    dev = binding.layer_to_device(layer, "cuda")
    weight_sets = [dev]
    for _ in range(copies - 1):
        weight_sets.append({kk: (v.clone() if kk.startswith("w") else v) for kk, v in dev.items()})
    torch.cuda.synchronize()
    ws = torch.empty((binding.workspace_bytes(T, H, I, E, k),), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step(i):
        d = weight_sets[i % copies]
        binding.moe_mxfp4_forward(dev["x"], dev["router_logits"], d["w13_blocks"], d["w13_scales"],
                                  d["w13_bias"], d["w2_blocks"], d["w2_scales"], d["w2_bias"], k,
                                  out=y, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    binding.profile_begin("gate_up", args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gate_up_ms = binding.profile_end(args.steps)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = T / (ms_per_step / 1e3)
    gu_ms = float(np.mean(gate_up_ms))

    # Stage breakdown (outside the timed region, diagnostics on stderr).
    stages = {}
    for st in ["route", "group", "gate_up", "down", "combine"]:
        binding.profile_begin(st, 5)
        for i in range(5):
            step(i)
        torch.cuda.synchronize()
        stages[st] = float(np.mean(binding.profile_end(5)))
    log("[bench] stage ms: " + ", ".join(f"{s}={v:.4f}" for s, v in stages.items()))

    P = T * k
    flops_total = 6.0 * H * I * P
    gu_flops = 4.0 * H * I * P
    gu_bytes = n_active * w13_b + P * (2 * H + 2 * I)  # weights of active experts + x rows in + a rows out
    if P / max(n_active, 1) >= 64:
        roof = {"bound": "mfma", "achieved": gu_flops / (gu_ms / 1e3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": gu_bytes / (gu_ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "gate_up grouped GEMM (expert_gemm_kernel, gate_up epilogue)"
    roof["kernel_ms"] = gu_ms
    log(f"[bench] {args.workload}: {ms_per_step:.4f} ms/step, {value:.1f} tokens/s, "
        f"layer {flops_total / (ms_per_step / 1e3) / 1e12:.1f} TFLOP/s, "
        f"active experts {n_active}, weight bytes {active_bytes / 1e6:.1f} MB -> "
        f"{active_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s; copies {copies}")

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: MXFP4 MoE expert layer T={T} H={H} I={I} E={E} top_k={k}"
                        + (f", Zipf({spec.zipf_s}) routing skew" if spec.zipf_s else ""),
            "T": T, "H": H, "I": I, "E": E, "top_k": k,
            "weights": "mxfp4 (e2m1 codes, e8m0 scale per 32)",
            "accumulate": "fp32",
            "active_experts": n_active,
            "weight_copies_rotated": copies,
            "layer_tflops": flops_total / (ms_per_step / 1e3) / 1e12,
            "active_weight_gbs": active_bytes / (ms_per_step / 1e3) / 1e9,
            "stage_ms": stages,
        },
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_moe(layer, spec)
    return out


def run_dequant(args):
    import numpy as np
    import torch

    from mxfp4_quantized_expert_amd import binding, workloads

    bank = workloads.DEQUANT_BANK_120B[0]
    blocks, scales = workloads.make_bank(bank)
    b = torch.from_numpy(blocks).cuda()
    s = torch.from_numpy(scales).cuda()
    out = torch.empty(blocks.shape[:-1] + (bank.K,), dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        binding.mxfp4_dequantize(b, s, out=out)
    torch.cuda.synchronize()
    binding.profile_begin("dequant", args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        binding.mxfp4_dequantize(b, s, out=out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms = float(np.mean(binding.profile_end(args.steps)))
    ms = (t1 - t0) * 1e3 / args.steps
    nbytes = blocks.nbytes + scales.nbytes + out.numel() * 2
    res = {
        "metric": "mxfp4_dequantize HBM GB/s",
        "value": nbytes / (ms / 1e3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8->bf16", "data": "synthetic",
        "config": {"workload": f"dequant of a gpt-oss-120b shaped w13 bank {list(blocks.shape)} -> bf16"},
        "roofline": {"bound": "hbm", "achieved": nbytes / (kms / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (kms / 1e3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "mxfp4_dequant_kernel", "kernel_ms": kms},
    }
    if not args.no_cpu_baseline:
        from oracle import mxfp4_moe as O
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 10.0 and n < bank.E:
            O.mxfp4_dequantize(blocks[n], scales[n])
            n += 1
        el = time.perf_counter() - t0
        per = (blocks[0].nbytes + scales[0].nbytes + blocks[0].size * 4)
        res["cpu_baseline"] = {"value": n * per / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {bank.E} experts, numpy oracle, {el:.1f} s"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="120b_prefill",
                    choices=["120b_prefill", "20b_prefill", "20b_decode", "tiny", "dequant_120b"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    res = run_dequant(args) if args.workload == "dequant_120b" else run_moe(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
