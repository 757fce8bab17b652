"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--cf 1.0]

One step is one whole layer forward (router, dispatch with capacity, expert
MLPs, combine) over the workload's batch, inputs and weights already resident
in HBM.  The step runs the C-ABI stage chain moe_route -> moe_dispatch ->
moe_expert_ffn -> moe_combine (the same kernels, in the same order, as
moe_forward) with HIP events between the stages on the launch stream, so the
expert stage's duration is measured live inside the timed region.

Prints one JSON line: tokens/s of the layer, the roofline of the expert stage
(the dominant pair of grouped-GEMM launches: HBM-bound for weight-streaming
workloads, MFMA-bound for large prefill), and the CPU oracle timed on the
host on a bounded sample of the same workload.
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector
METRIC = "MoE layer fwd tokens/s + TFLOP/s (% bf16 MFMA peak) or GB/s (% HBM peak), 1 GPU"

# CPU-baseline sample (tokens) per workload: the oracle in fp64 on the host's
# cores for roughly 5-30 s.  The sample is the first T_s tokens of the same
# batch, with the capacity recomputed for T_s tokens.
CPU_SAMPLE_TOKENS = {"c1": 1024, "c2": 16384, "c3": 2048, "c4": 256, "c5": 128}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", help="c1..c5 (default: c2, the Switch-style layer)")
    ap.add_argument("--cf", type=float, default=None, help="capacity factor override (<0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def expert_stage_work(cfg, counts_kept, used_experts):
    """Algorithmic FLOPs and bytes of the expert stage (fc1+act, fc2).

    FLOPs: 2 per multiply-add over kept rows only: 2*K*D*F per projection
    (two projections, three for SwiGLU).  Bytes: every used expert's weights
    once, plus the kept rows of x read once (bf16/fp32 element size).
    """
    es = 2 if cfg.dtype == "bf16" else 4
    nproj = 3 if cfg.act == "swiglu" else 2
    K = int(counts_kept)
    flops = 2.0 * K * cfg.D * cfg.F * nproj
    w_bytes = used_experts * nproj * cfg.D * cfg.F * es
    if cfg.expert_bias:
        w_bytes += used_experts * (cfg.F + cfg.D) * es
    bytes_ = w_bytes + K * cfg.D * es
    return flops, bytes_


def layer_flops(cfg, counts_kept):
    nproj = 3 if cfg.act == "swiglu" else 2
    return 2.0 * cfg.T * cfg.D * cfg.N + 2.0 * counts_kept * cfg.D * cfg.F * nproj


def cpu_baseline(cfg, inp, key):
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    Ts = min(cfg.T, CPU_SAMPLE_TOKENS.get(key, 1024))
    xs = inp["x"][:Ts]
    C = oracle.capacity(Ts, cfg.k, cfg.N, cfg.cf)
    t0 = time.perf_counter()
    r = oracle.moe_forward(xs, inp, k=cfg.k, act=cfg.act, renorm=cfg.renorm, capacity_slots=C,
                           residual=cfg.residual)
    dt = time.perf_counter() - t0
    del r
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    _ = (np, torch)
    return {"value": Ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {Ts} of {cfg.T} tokens of the same batch (capacity "
                      f"{'none' if C is None else C} for {Ts} tokens), fp64 numpy per-expert loop, "
                      f"{dt:.2f} s on {cpu_model or 'host CPU'}",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_expert_amd import api
    from workloads import generate, get_config

    cf = "keep" if args.cf is None else (None if args.cf < 0 else args.cf)
    cfg = get_config(args.workload, cf=cf)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = generate(cfg)
    g = {k: (None if v is None else v.to(dev).contiguous()) for k, v in inp.items()}
    shape = api.MoeShape.from_config(cfg)
    buf = api.MoeBuffers(shape, device=dev)
    A = cfg.T * cfg.k
    y_perm = torch.empty(A, cfg.D, dtype=shape.torch_dtype, device=dev)
    st = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(st)
        api.route(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, None, st)
        api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped, st)
        if ev is not None:
            ev[1].record(st)
        api.expert_ffn(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], g["w2"],
                       g["b2"], y_perm, buf.ws, st)
        if ev is not None:
            ev[2].record(st)
        api.combine(shape, y_perm, buf.slot, buf.topk_gate, g["x"], buf.out, st)
        if ev is not None:
            ev[3].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(st)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(st)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    route_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ffn_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    comb_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps

    counts = buf.counts.cpu()
    offsets = buf.offsets.cpu()
    kept = int(offsets[-1])
    used = int(((offsets[1:] - offsets[:-1]) > 0).sum())
    n_dropped = int(buf.n_dropped.cpu())
    flops, bytes_ = expert_stage_work(cfg, kept, used)
    lflops = layer_flops(cfg, kept)

    if cfg.dtype == "bf16":
        intensity = flops / bytes_
        ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        bound = "hbm" if intensity < ridge else "mfma"
    else:
        bound = "alu"
    ffn_s = ffn_ms / 1e3
    if bound == "hbm":
        achieved, peak, unit = bytes_ / ffn_s / 1e9, PEAK_HBM_GBS, "GB/s"
    elif bound == "mfma":
        achieved, peak, unit = flops / ffn_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = flops / ffn_s / 1e12, PEAK_FP32_TFLOPS, "TFLOP/s"

    tokens_per_s = cfg.T / (ms_step / 1e3)
    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "D": cfg.D, "F": cfg.F, "experts": cfg.N,
                   "top_k": cfg.k, "act": cfg.act, "capacity_factor": cfg.cf,
                   "capacity": shape.capacity, "renorm": cfg.renorm, "residual": cfg.residual},
        "layer_tflops": lflops / (ms_step / 1e3) / 1e12,
        "layer_tflops_frac_bf16_peak": lflops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "stages_ms": {"route+dispatch": route_ms, "expert_ffn": ffn_ms, "combine": comb_ms},
        "routing": {"kept_assignments": kept, "dropped": n_dropped, "experts_used": used,
                    "max_count": int(counts.max()), "imbalance": float(counts.max()) / (A / cfg.N)},
        "roofline": {
            "kernel": "expert stage: grouped_gemm_kernel fc1(+act) and fc2 launches (moe_expert_ffn)",
            "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": None,
            "algorithmic": {"flops": flops, "bytes": bytes_,
                            "rule": "weights of used experts once + kept x rows once; "
                                    "2 flops per MAC over kept rows"},
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.workload if args.workload in CPU_SAMPLE_TOKENS
                                           else "c2")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
