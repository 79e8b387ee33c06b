"""Benchmark: MoE-LoRA expert layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]

One step is the whole hot path over one batch: route, permute, grouped
gate_up (+LoRA, SwiGLU) and down (+LoRA) GEMMs reading x's rows through the
permutation, combine, and the backward (the combine backward folded into the
down backward, whose GEMMs read dY's rows through the permutation and whose
epilogue gives dw; route, down and gate_up with SwiGLU', LoRA weight
gradients, unpermute-sum). Inputs are seeded synthetic tensors already
resident in HBM when timing starts. Prints one JSON line.

value    = algorithmic TFLOP/s of the step, F = 12 N H I + 6 N r (2H + 3I)
           (N = T k routed rows; frozen base weights, so no dW; W + B A never
           formed), over the mean step time of the timed region.
roofline = the dominant GEMM kernel's algorithmic FLOPs per launch over its
           mean launch time, timed live with HIP events on the launch stream
           by the library's kernel timer, against the dense bf16 (= fp16) MFMA peak.
cpu_baseline = the CPU oracle (NumPy float32 per-expert loop) on a bounded
           sample of the same workload, on the host's cores.
hbm      = the memory-bound kernels' algorithmic bytes per launch over their
           mean launch time, against the 8 TB/s HBM3E peak.
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

GEMM_KERNELS = ("gate_up_fwd", "down_fwd", "down_bwd", "gate_up_bwd", "base_wgrad")
METRIC_FULL_FT = ("MoE expert layer full fine-tuning fwd+bwd (LoRA plus base-weight gradients) "
                  "TFLOP/s and tokens/s on 1 MI355X; % bf16 MFMA peak")


def kernel_flops(name, cfg):
    """Algorithmic FLOPs of one launch of a grouped GEMM kernel (all N routed rows)."""
    N, H, I, r = cfg.N, cfg.H, cfg.I, cfg.r
    return {
        "gate_up_fwd": 2 * N * (2 * I) * (H + r),   # X W^T + U B^T over 2I outputs
        "down_fwd": 2 * N * H * (I + r),            # act W^T + U B^T over H outputs
        "down_bwd": 2 * N * I * (H + r),            # G W + GB A over I outputs
        "gate_up_bwd": 2 * N * H * (2 * I + r),     # dH W + dHB A over H outputs
        "base_wgrad": 3 * N * H * I,                # mean of dW_d = G^T act (2NHI), dW_gu = dH^T X (4NHI)
    }[name]


def kernel_bytes(name, cfg):
    """Algorithmic HBM bytes of one launch of a memory-bound kernel (each tensor once)."""
    T, H, E, k, N = cfg.T, cfg.H, cfg.E, cfg.k, cfg.N
    es = 4 if cfg.dtype == "f32" else 2
    return {
        "route": T * E * 4 + T * k * 8,                        # logits in; ids, weights out
        "permute": N * 4 * 3 + (2 * E + 1) * 4,                # ids in; sorted_pair, inv_pos, counts
        "gather": T * H * es + N * H * es + N * 4,            # x in, X_perm out, sorted_pair
        "combine": N * H * es + T * H * es + N * 8,           # Yexp in, Y out, inv_pos + weights
        "combine_bwd": T * H * es + 2 * N * H * es + N * 12,  # dY, Yexp in; G out; idx, w, dw
        "dy_gather": T * H * es + N * H * es + N * 4,         # dY in, its permuted rows out
        # routing weight per row, w u_d, and the dw partial sums of the down backward
        "dw_sum": N * 12 + 2 * N * cfg.r * es + N * 4 * dw_slots(cfg) + N * 8,
        "row_scale": 2 * N * H * es + N * 4,                  # dY rows scaled in place by w
        "route_bwd": 2 * T * E * 4 + T * k * 8,                # logits in, dlogits out; ids, dw
        "unpermute": N * H * es + T * H * es + N * 4,         # dX_perm in, dX out, inv_pos
        "router_fwd": T * H * es + E * H * es + T * E * 4,    # x, W_r in; logits out
        "router_bwd": T * E * 4 + E * H * es + 2 * T * H * es,  # dlogits, W_r in; dx in and out
        "accumulate": 3 * T * H * es,                          # src, dst in; dst out
    }.get(name)


def dw_slots(cfg):
    """dw partial sums per row that the down backward writes (one per 64-wide
    wave column of its 256-wide column tiles; 64-wide tiles for float32)."""
    return -(-cfg.I // 64) if cfg.dtype == "f32" else -(-cfg.I // 256) * 4


def block_parts(cfg, shared_I):
    """(routed layer, shared expert as a one-expert k = 1 layer or None)."""
    return cfg, (cfg.with_(name=cfg.name + "-shared", E=1, k=1, I=shared_I) if shared_I else None)


def step_flops(cfg, full_ft, shared_I=None, block=False):
    """Algorithmic FLOPs of one step: the routed layer, plus in block mode the
    router projection (2 T E H forward, 2 T E H for dx) and the shared expert
    (the layer formula with E = 1, k = 1, width shared_I)."""
    routed, shared = block_parts(cfg, shared_I)
    F = 0
    for c in (routed, shared) if block else (routed,):
        if c is not None:
            F += c.flops_fwd_bwd() + (6 * c.N * c.H * c.I if full_ft else 0)
    if block:
        F += 4 * cfg.T * cfg.E * cfg.H
    return F


# The sources the counted GEMM kernels are built from (their template, the
# headers it includes, and the build flags); a change to any of them makes
# the recorded traffic stale.
TRAFFIC_SOURCES = ("mixture_experts_lora_amd/csrc/gemm.hip",
                   "mixture_experts_lora_amd/csrc/device_common.h",
                   "mixture_experts_lora_amd/csrc/launch.h",
                   "mixture_experts_lora_amd/build.py")


def source_hash():
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
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


def classify_gemm(kernel_name):
    """Map a profiler kernel name of the 16-bit grouped GEMM to the step it runs."""
    import re
    m = re.search(r"gemm16<([^>]*)>", kernel_name)
    if not m:
        return None
    a = [x.strip() for x in m.group(1).split(",")][1:]     # drop the F16 flag
    bm, bn, mode, epi, b_kc = int(a[0]), int(a[1]), int(a[7]), int(a[8]), a[11] == "true"
    if mode != 0 or bn < 128 or epi > 2:
        return None  # LoRA side products, weight gradients, router projection
    if epi == 1:
        return "gate_up_fwd"
    if epi == 2:
        return "down_bwd"
    return "down_fwd" if b_kc else "gate_up_bwd"


def write_traffic(d, workload):
    """profiles/traffic_<kernel>_<workload>.json from rocprofv3 --pmc runs under d:
    d/fetch and d/write (FETCH_SIZE, WRITE_SIZE of a bench run), d/calib_fetch and
    d/calib_write (the same counters over one device copy of --calib-copy MiB)."""
    import csv
    from collections import defaultdict

    def per_dispatch(sub, counter, pick):
        tot, ids = defaultdict(float), defaultdict(set)
        with open(os.path.join(d, sub, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                k = pick(r["Kernel_Name"])
                if k and r["Counter_Name"] == counter:
                    tot[k] += float(r["Counter_Value"])
                    ids[k].add(r["Dispatch_Id"])
        return {k: (tot[k] / len(ids[k]), len(ids[k])) for k in tot}

    copy = lambda n: "copyBuffer" if "copyBuffer" in n else None  # noqa: E731
    calib = json.load(open(os.path.join(d, "calib.json")))
    cf = calib["read_bytes"] / (per_dispatch("calib_fetch", "FETCH_SIZE", copy)["copyBuffer"][0] * 1024)
    cw = calib["write_bytes"] / (per_dispatch("calib_write", "WRITE_SIZE", copy)["copyBuffer"][0] * 1024)
    fetch = per_dispatch("fetch", "FETCH_SIZE", classify_gemm)
    write = per_dispatch("write", "WRITE_SIZE", classify_gemm)
    if calib.get("source_hash") != source_hash():
        raise SystemExit("counter runs were taken on other kernel sources than these")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for k in sorted(fetch):
        rec = {"kernel": k, "workload": workload, "source_hash": source_hash(),
               "fetch_kib_per_dispatch": round(fetch[k][0], 1),
               "write_kib_per_dispatch": round(write[k][0], 1), "dispatches": fetch[k][1],
               "calib_fetch_factor": round(cf, 4), "calib_write_factor": round(cw, 4),
               "hbm_read_bytes_per_launch": int(fetch[k][0] * 1024 * cf),
               "hbm_write_bytes_per_launch": int(write[k][0] * 1024 * cw)}
        rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
        with open(os.path.join(ROOT, "profiles", f"traffic_{k}_{workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))


def cpu_baseline_block(cfg, inp, sample_tokens, shared_I):
    """The oracle of the whole block (router projection, routed experts, shared
    expert) on the first sample_tokens tokens."""
    import numpy as np
    import oracle
    from workloads.synth import to_numpy
    names = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")
    Ts = min(sample_tokens, cfg.T)
    h = {n: to_numpy(inp[n]) for n in names}
    sh = {n: to_numpy(inp["shared_" + n]) for n in names} if shared_I else None
    x, dy, w_r = to_numpy(inp["x"][:Ts]), to_numpy(inp["dy"][:Ts]), to_numpy(inp["w_r"])
    w = min(256, Ts)
    oracle.layer_with_router_and_shared(x[:w], w_r, dy[:w], h, sh, cfg.k, cfg.router,
                                        cfg.lora_scale)
    t0 = time.perf_counter()
    oracle.layer_with_router_and_shared(x, w_r, dy, h, sh, cfg.k, cfg.router, cfg.lora_scale)
    dt = time.perf_counter() - t0
    flops = step_flops(cfg.with_(T=Ts), False, shared_I, block=True)
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "tokens_per_s": round(Ts / dt, 1),
            "sample": f"first {Ts} of {cfg.T} tokens of the same block (router projection, "
                      f"routed experts, shared expert), NumPy float32, forward+backward"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()
                        if i.get("user_api") == "blas"] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline(cfg, inp, sample_tokens, full_ft=False):
    import numpy as np
    import oracle
    from workloads.synth import to_numpy
    threads = _blas_threads()
    Ts = min(sample_tokens, cfg.T)
    S = slice(0, Ts)
    h = {n: to_numpy(inp[n]) for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")}
    x, lg, dy = to_numpy(inp["x"][S]), to_numpy(inp["logits"][S]), to_numpy(inp["dy"][S])
    w = min(256, Ts)  # warm-up on a few tokens (BLAS threads, page faults)
    oracle.layer_forward_backward(x[:w], lg[:w], dy[:w], h, cfg.k, cfg.router, cfg.lora_scale,
                                  np.float32, base_grads=full_ft)
    t0 = time.perf_counter()
    oracle.layer_forward_backward(x, lg, dy, h, cfg.k, cfg.router, cfg.lora_scale, np.float32,
                                  base_grads=full_ft)
    dt = time.perf_counter() - t0
    sub = cfg.with_(T=Ts)
    flops = sub.flops_fwd_bwd() + (6 * sub.N * sub.H * sub.I if full_ft else 0)
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "tokens_per_s": round(Ts / dt, 1),
            "sample": f"first {Ts} of {cfg.T} tokens of the same layer (same weights, routing "
                      f"mode and shapes), NumPy float32 per-expert loop, forward+backward",
            "host_cpus": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def bench_merge(mel, cfg, args):
    """Merged export W' = W + s B A of every expert's gate_up and down weights:
    HBM-bound (each base weight read once and each merged weight written once;
    the rank-r product is 2 r FLOPs per element)."""
    import torch
    from workloads import make_inputs
    names = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")
    inp = make_inputs(cfg, args.seed, device="cuda", with_dy=False)
    w = {n: inp[n] for n in names}
    shape = mel.Shape.of(cfg)
    ws = torch.empty(max(mel.moe_merge_workspace_bytes(shape), 1), device="cuda",
                     dtype=torch.uint8)
    out_gu, out_d = torch.empty_like(w["w_gu"]), torch.empty_like(w["w_d"])
    for _ in range(args.warmup):
        mel.moe_merge_lora(shape, w, out_gu, out_d, ws)
    torch.cuda.synchronize()
    with mel.kernel_timer() as kt:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            mel.moe_merge_lora(shape, w, out_gu, out_d, ws)
        b.record()
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    kms, n = kt.read("merge")
    es = 4 if cfg.dtype == "f32" else 2
    base = cfg.E * 3 * cfg.I * cfg.H * es                  # W_gu [E, 2I, H] + W_d [E, H, I]
    lora = sum(w[n].numel() for n in ("a_gu", "b_gu", "a_d", "b_d")) * es
    nbytes = 2 * base + lora
    gbs = nbytes / (ms / 1e3) / 1e9
    kgbs = nbytes / (kms / n / 1e3) / 1e9
    print(json.dumps({
        "metric": "MoE-LoRA merged export (W + s B A, every expert, both projections) GB/s "
                  "on 1 MI355X; % HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}-shaped expert weights, merged export",
                   "H": cfg.H, "I": cfg.I, "E": cfg.E, "r": cfg.r, "lora_scale": cfg.lora_scale},
        "roofline": {"bound": "hbm", "kernel": "merge", "achieved": round(kgbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "bytes_per_launch": nbytes,
                     "ms_per_launch": round(kms / n, 4)},
    }), flush=True)


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
    ap.add_argument("--recompute", action="store_true",
                    help="activation-lean mode: h and act recomputed in the backward")
    ap.add_argument("--full-ft", action="store_true",
                    help="full fine-tuning step: also the base-weight gradients (F += 6 N H I)")
    ap.add_argument("--block", action="store_true",
                    help="whole MoE block: router projection from hidden states, routed "
                         "experts, and a shared expert (width --shared-I)")
    ap.add_argument("--shared-I", type=int, default=None,
                    help="shared expert width in --block mode (default I; 0: none)")
    ap.add_argument("--chunks", type=int, default=1,
                    help="run the layer over its tokens in this many chunks sharing one set "
                         "of workspaces (long contexts: lower peak memory)")
    ap.add_argument("--gather-dy", choices=("on", "off"), default="on",
                    help="the backward's GEMMs read dY's rows in token order (on) or from a "
                         "copy in expert order (off)")
    ap.add_argument("--merge", action="store_true",
                    help="only time the merged export W + s B A of both projections")
    ap.add_argument("--write-traffic", metavar="DIR", default=None,
                    help="only write profiles/traffic_*.json from rocprofv3 counter runs in DIR")
    args = ap.parse_args()
    if args.write_traffic:
        from workloads import BENCH_CONFIG
        write_traffic(args.write_traffic, args.config or BENCH_CONFIG)
        return
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
        print(json.dumps({"calib_copy_bytes": n, "read_bytes": n, "write_bytes": n,
                          "source_hash": source_hash()}))
        return
    import mixture_experts_lora_amd as mel
    from workloads import BENCH_CONFIG, get_config, make_block_inputs, make_inputs

    cfg = get_config(args.config or BENCH_CONFIG)
    torch.cuda.set_device(0)
    names = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")
    if args.merge:
        bench_merge(mel, cfg, args)
        return
    shape = mel.Shape.of(cfg)
    shared_I = None
    if args.block:
        shared_I = cfg.I if args.shared_I is None else (args.shared_I or None)
        inp = make_block_inputs(cfg, args.seed, device="cuda", shared_I=shared_I)
        sw = {n: inp["shared_" + n] for n in names} if shared_I else None
    else:
        inp = make_inputs(cfg, args.seed, device="cuda")
    weights = {n: inp[n] for n in names}
    torch.cuda.reset_peak_memory_stats()
    if args.block:
        layer = mel.MoELoRABlock(shape, cfg.router, shared_I, full_ft=args.full_ft,
                                 recompute=args.recompute)
        step = lambda: layer.step(inp["x"], inp["w_r"], inp["dy"], weights, sw)  # noqa: E731
        fwd = lambda: layer.forward(inp["x"], inp["w_r"], weights, sw)  # noqa: E731
        bwd = lambda: layer.backward(inp["dy"], inp["x"], inp["w_r"], weights, sw)  # noqa: E731
        saved = layer.routed.saved_bytes() + (
            sum(v.numel() * v.element_size() for v in layer.shared.saved.values())
            if layer.shared is not None else 0)
    else:
        gdy = args.gather_dy == "on"
        if args.chunks > 1:
            layer = mel.MoELoRAChunkedLayer(shape, cfg.router, args.chunks, full_ft=args.full_ft,
                                            recompute=args.recompute, gather_dy=gdy)
        else:
            layer = mel.MoELoRALayer(shape, cfg.router, full_ft=args.full_ft,
                                     recompute=args.recompute, gather_dy=gdy)
        step = lambda: layer.step(inp["x"], inp["logits"], inp["dy"], weights)  # noqa: E731
        fwd = lambda: layer.forward(inp["x"], inp["logits"], weights)  # noqa: E731
        bwd = lambda: layer.backward(inp["dy"], inp["logits"], weights, x=inp["x"])  # noqa: E731
        saved = layer.saved_bytes()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-kernel times, in a pass of their own: every launch bracketed by HIP
    # events on its stream (about 50 event records per step, which would add
    # ~2% to a timed step).
    kpass = max(1, min(args.steps, 10))
    with mel.kernel_timer() as kt:
        for _ in range(kpass):
            step()
        torch.cuda.synchronize()
    kms = {}
    for name in mel._lib.KERNEL_IDS:
        tot, n = kt.read(name)
        if n:
            kms[name] = {"ms_per_step": round(tot / kpass, 4), "launches": round(n / kpass, 3),
                         "ms_per_launch": round(tot / n, 4)}
    dom = max((k for k in GEMM_KERNELS if k in kms), key=lambda k: kms[k]["ms_per_step"])

    # timed region: K steps, the dominant kernel's launches timed live (HIP
    # events on the launch stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with mel.kernel_timer(only=[dom]) as kt:
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(args.steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    dom_tot, dom_n = kt.read(dom)

    # forward-only and backward-only, after the timed region
    def timed(fn, n=5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    fwd_ms = timed(fwd)
    bwd_ms = timed(bwd)
    peak_bytes = torch.cuda.max_memory_allocated()

    F = step_flops(cfg, args.full_ft, shared_I, args.block)
    tflops = F / (ms / 1e3) / 1e12
    half = cfg.dtype in ("bf16", "f16")      # dense bf16 and fp16 MFMA peaks are equal
    peak = PEAK_BF16_TFLOPS if half else PEAK_F32_TFLOPS
    # FLOPs of the dominant kernel per step over its summed launch time per
    # step, both from the timed region.
    # Every part (the routed layer, or each token chunk; in block mode also the
    # shared expert) launches each GEMM kernel equally often (twice for gate_up_fwd when the
    # backward recomputes h; base_wgrad's figure is the mean of its two launches).
    if args.block:
        parts = [c for c in block_parts(cfg, shared_I) if c is not None]
    elif args.chunks > 1:
        parts = [cfg.with_(T=hi - lo) for lo, hi in layer.bounds]
    else:
        parts = [cfg]
    dom_launches = dom_n / args.steps
    dom_flops_step = dom_launches / len(parts) * sum(kernel_flops(dom, c) for c in parts)
    dom_tf = dom_flops_step / (dom_tot / args.steps / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(dom_tf / peak, 4),
                "traffic": None if args.block else traffic_for(dom, cfg.name),
                "flops_per_launch": int(dom_flops_step / dom_launches),
                "ms_per_launch": round(dom_tot / dom_n, 4)}
    hbm = {}
    for name, kv in kms.items():
        nb = kernel_bytes(name, cfg)
        if nb:
            gbs = nb / (kv["ms_per_launch"] / 1e3) / 1e9
            hbm[name] = {"bytes_per_launch": nb, "GB/s": round(gbs, 1),
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}
    out = {
        "metric": METRIC_FULL_FT if args.full_ft else METRIC, "value": round(tflops, 2),
        "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_median": round(step_ms[len(step_ms) // 2], 4), "ms_min": round(step_ms[0], 4),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}-shaped MoE-LoRA "
                               + ("block (router projection, routed experts"
                                  + (f", shared expert of width {shared_I})" if shared_I else ")")
                                  if args.block else "expert layer")
                               + " fwd+bwd"
                               + (", full fine-tuning" if args.full_ft else "")
                               + (", h and act recomputed in backward" if args.recompute else "")
                               + (f", {args.chunks} token chunks" if args.chunks > 1 else ""),
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k, "r": cfg.r,
                   "router": cfg.router, "lora_scale": cfg.lora_scale, "seed": args.seed},
        "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
        "mfma_peak_frac": round(tflops / peak, 4),
        "flops_per_step": F,
        "peak_hbm_bytes": int(peak_bytes),
        "saved_activation_bytes": int(saved),
        "roofline": roofline,
        "hbm": hbm,
        "kernels": kms,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = (cpu_baseline_block(cfg, inp, args.cpu_tokens, shared_I)
                               if args.block and not args.full_ft
                               else cpu_baseline(cfg, inp, args.cpu_tokens, args.full_ft))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
