"""Benchmark: MoE-LoRA expert layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]

One step is the whole hot path over one batch: route, permute + gather,
grouped gate_up (+LoRA, SwiGLU) and down (+LoRA) GEMMs, combine, and the
backward (combine, route, down and gate_up with SwiGLU', LoRA weight
gradients, unpermute-sum). Inputs are seeded synthetic tensors already
resident in HBM when timing starts. Prints one JSON line.

value    = algorithmic TFLOP/s of the step, F = 12 N H I + 6 N r (2H + 3I)
           (N = T k routed rows; frozen base weights, so no dW; W + B A never
           formed), over the mean step time of the timed region.
roofline = the dominant GEMM kernel's algorithmic FLOPs per launch over its
           mean launch time, timed live with HIP events on the launch stream
           by the library's kernel timer, against the dense bf16 MFMA peak.
cpu_baseline = the CPU oracle (NumPy float32 per-expert loop) on a bounded
           sample of the same workload, on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_F32_TFLOPS = 157.3        # fp32 vector
PEAK_HBM_GBS = 8000.0
METRIC = "MoE-LoRA layer fwd+bwd TFLOP/s and tokens/s on 1 MI355X; % bf16 MFMA peak"

GEMM_KERNELS = ("gate_up_fwd", "down_fwd", "down_bwd", "gate_up_bwd")


def kernel_flops(name, cfg):
    """Algorithmic FLOPs of one launch of a grouped GEMM kernel (all N routed rows)."""
    N, H, I, r = cfg.N, cfg.H, cfg.I, cfg.r
    return {
        "gate_up_fwd": 2 * N * (2 * I) * (H + r),   # X W^T + U B^T over 2I outputs
        "down_fwd": 2 * N * H * (I + r),            # act W^T + U B^T over H outputs
        "down_bwd": 2 * N * I * (H + r),            # G W + GB A over I outputs
        "gate_up_bwd": 2 * N * H * (2 * I + r),     # dH W + dHB A over H outputs
    }[name]


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_lora_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed counter runs, or None if absent or stale."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inp, sample_tokens):
    import numpy as np
    import oracle
    from workloads.synth import to_numpy
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    Ts = min(sample_tokens, cfg.T)
    S = slice(0, Ts)
    h = {n: to_numpy(inp[n]) for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")}
    x, lg, dy = to_numpy(inp["x"][S]), to_numpy(inp["logits"][S]), to_numpy(inp["dy"][S])
    t0 = time.perf_counter()
    oracle.layer_forward_backward(x, lg, dy, h, cfg.k, cfg.router, cfg.lora_scale, np.float32)
    dt = time.perf_counter() - t0
    sub = cfg.with_(T=Ts)
    return {"value": round(sub.flops_fwd_bwd() / dt / 1e12, 4), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "tokens_per_s": round(Ts / dt, 1),
            "sample": f"first {Ts} of {cfg.T} tokens of the same layer (same weights, routing "
                      f"mode and shapes), NumPy float32 per-expert loop, forward+backward",
            "host_cpus": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None)
    ap.add_argument("--seed", type=int, default=3407)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB mebibytes device-to-device once (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is benchmarked on a single MI355X "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calib_copy:
        n = args.calib_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "read_bytes": n, "write_bytes": n}))
        return
    import mixture_experts_lora_amd as mel
    from workloads import BENCH_CONFIG, get_config, make_inputs

    cfg = get_config(args.config or BENCH_CONFIG)
    torch.cuda.set_device(0)
    inp = make_inputs(cfg, args.seed, device="cuda")
    weights = {n: inp[n] for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")}
    shape = mel.Shape.of(cfg)
    torch.cuda.reset_peak_memory_stats()
    layer = mel.MoELoRALayer(shape, cfg.router)
    for _ in range(args.warmup):
        layer.step(inp["x"], inp["logits"], inp["dy"], weights)
    torch.cuda.synchronize()

    # timed region: K steps, kernel timer live (HIP events on the launch stream)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with mel.kernel_timer() as kt:
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            layer.step(inp["x"], inp["logits"], inp["dy"], weights)
        stop.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    kms = {}
    for name in mel._lib.KERNEL_IDS:
        tot, n = kt.read(name)
        if n:
            kms[name] = {"ms_per_step": round(tot / args.steps, 4), "launches": n,
                         "ms_per_launch": round(tot / n, 4)}
    peak_bytes = torch.cuda.max_memory_allocated()

    F = cfg.flops_fwd_bwd()
    tflops = F / (ms / 1e3) / 1e12
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    dom = max((k for k in GEMM_KERNELS if k in kms), key=lambda k: kms[k]["ms_per_step"])
    dom_ms = kms[dom]["ms_per_launch"]
    dom_tf = kernel_flops(dom, cfg) / (dom_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(dom_tf / peak, 4),
                "traffic": traffic_for(dom, cfg.name),
                "flops_per_launch": kernel_flops(dom, cfg), "ms_per_launch": dom_ms}
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}-shaped MoE-LoRA expert layer fwd+bwd",
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k, "r": cfg.r,
                   "router": cfg.router, "lora_scale": cfg.lora_scale, "seed": args.seed},
        "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
        "mfma_peak_frac": round(tflops / peak, 4),
        "flops_per_step": F,
        "peak_hbm_bytes": int(peak_bytes),
        "roofline": roofline,
        "kernels": kms,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
