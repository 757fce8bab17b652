"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--cf 1.0]
                    [--copies 3] [--no-graph] [--no-cpu-baseline]
    python bench.py --copy-calibration     (plain copy of known size, for PMC scaling)

One step is one whole layer forward (router, dispatch with capacity, expert
MLPs, combine) over the workload's batch, inputs and weights already resident
in HBM.  The step runs the C-ABI chain moe_route -> moe_dispatch ->
moe_expert_up -> moe_expert_down -> moe_combine (the kernels of moe_forward,
in the same order) with HIP events between the launches on the launch
stream, so every launch's duration is measured live inside the timed region.
Consecutive steps cycle over --copies separate copies of x and the weights,
so that no step finds its weights in the 256 MB last-level cache from the
step before.

The timed steps are the same chain captured once per input copy into HIP
graphs and replayed (W warm-up replays, then K timed ones between
synchronisations); the eager run before it supplies the per-launch HIP-event
timings and its own step time ("eager").  --no-graph times the eager steps.

Prints one JSON line: tokens/s of the layer, the roofline of the dominant
launch (HBM-bound for weight-streaming workloads, MFMA-bound for large
prefill), and the CPU oracle timed on the host on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 dense MFMA (the fp32 grouped GEMM runs on v_mfma_f32_16x16x4f32)
METRIC = "MoE layer fwd tokens/s + TFLOP/s (% bf16 MFMA peak) or GB/s (% HBM peak), 1 GPU"

# CPU-baseline sample (tokens) per workload: the oracle in fp64 on the host's
# cores for roughly 5-30 s.  The sample is the first T_s tokens of the same
# batch, with the capacity recomputed for T_s tokens.
CPU_SAMPLE_TOKENS = {"c1": 1024, "c2": 16384, "c3": 2048, "c4": 256, "c5": 128, "c6": 512}


# HBM traffic of the dominant launch, from two rocprofv3 --pmc runs of the
# default command of each workload (FETCH_SIZE, then WRITE_SIZE: KiB per
# dispatch, averaged over the dispatches of that launch), each scaled by the
# ratio of known bytes to the counter's reading for a plain copy
# (--copy-calibration).  A figure is used only while the kernel sources hash
# to the value it was measured with; otherwise traffic is null.
PMC_KERNEL_SOURCES = ("mixture_experts_layer_expert_amd/csrc/grouped_gemm.hip",
                      "mixture_experts_layer_expert_amd/csrc/grouped_gemm.h")
PMC_TRAFFIC = {  # workload -> kernel sources hash, then per launch: KiB per dispatch
    "c2": {"sources": "4649bdfacb8eed23",
           "fc1": {"fetch_kib": 309457.2, "write_kib": 91794.2},
           # grouped_gemm_kernel<128, 256, 2, 4, 64, 2, 0, 3>
           "fc2": {"fetch_kib": 341009.7, "write_kib": 22970.5},
           # grouped_gemm_kernel<128, 384, 2, 4, 64, 0, 0, 2>
           },
    "c4": {"sources": "4649bdfacb8eed23",
           "fc1": {"fetch_kib": 3361892.7, "write_kib": 458916.3},
           # grouped_gemm_kernel<256, 256, 2, 4, 64, 3, 0, 2>
           "fc2": {"fetch_kib": 1751301.1, "write_kib": 207205.8},
           # grouped_gemm_kernel<256, 256, 2, 4, 64, 0, 0, 2> + splitk_finish_kernel<256, 256, 2, 4, 64, 0, 0>
           },
    "c5": {"sources": "4649bdfacb8eed23",
           "fc1": {"fetch_kib": 363830.1, "write_kib": 2117.5},
           # grouped_gemm_kernel<32, 256, 1, 4, 64, 3, 0, 4>
           "fc2": {"fetch_kib": 181424.5, "write_kib": 3072.1},
           # grouped_gemm_kernel<32, 256, 1, 4, 64, 0, 0, 4>
           },
    "c3": {"sources": "4649bdfacb8eed23",
           "fc1": {"fetch_kib": 148374.3, "write_kib": 141576.7},
           # grouped_gemm_kernel<256, 256, 2, 4, 64, 1, 1, 2> + splitk_finish_kernel<256, 256, 2, 4, 64, 1, 1>
           "fc2": {"fetch_kib": 212318.8, "write_kib": 89725.9},
           # grouped_gemm_kernel<256, 256, 2, 4, 64, 0, 1, 2> + splitk_finish_kernel<256, 256, 2, 4, 64, 0, 1>
           },
    "c6": {"sources": "4649bdfacb8eed23",
           "fc1": {"fetch_kib": 584125.9, "write_kib": 90145.4},
           # grouped_gemm_kernel<256, 256, 2, 4, 64, 3, 0, 2> + splitk_finish_kernel<256, 256, 2, 4, 64, 3, 0>
           "fc2": {"fetch_kib": 266221.2, "write_kib": 133114.6},
           # grouped_gemm_kernel<256, 256, 2, 4, 64, 0, 0, 2> + splitk_finish_kernel<256, 256, 2, 4, 64, 0, 0>
           },
}
PMC_COPY_FACTOR = {"fetch": 1.99997, "write": 1.0}  # bytes per counter byte


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", help="c1..c5 (default: c2, the Switch-style layer)")
    ap.add_argument("--cf", type=float, default=None, help="capacity factor override (<0: none)")
    ap.add_argument("--priority", choices=("token", "choice"), default="token",
                    help="capacity priority: token order, or (choice, token) (MOE_SLOT_MAJOR)")
    ap.add_argument("--router-stats", action="store_true",
                    help="also compute the router's load statistics (moe_route_stats + moe_router_stats)")
    ap.add_argument("--reroute", type=int, default=0, metavar="R",
                    help="send overflow to the next-best experts with room over R levels "
                         "(moe_route_fallback + moe_dispatch_reroute)")
    ap.add_argument("--expert-shard", type=int, default=1, metavar="G",
                    help="time one GPU's share of an expert-sharded layer: every expert's hidden dim F/G "
                         "(a column block of w1/w3 and the matching row block of w2), all tokens")
    ap.add_argument("--layout", choices=("compact", "padded"), default="compact",
                    help="grouped rows sized by the counts, or N*capacity rows (MOE_PADDED)")
    ap.add_argument("--copies", type=int, default=3,
                    help="copies of x and the weights cycled over consecutive steps")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for PMC counter scaling)")
    return ap.parse_args()


def launch_work(cfg, kept, used):
    """Algorithmic FLOPs and bytes of the two expert launches, per launch.

    FLOPs: 2 per multiply-add over kept rows only (2*K*D*F per projection;
    fc1 of SwiGLU has two).  Bytes: every used expert's weights (and biases)
    once, the launch's activation rows read once and its output rows written
    once: fc1 reads K rows of x (gathered) and writes H[K, F]; fc2 reads H and
    writes y_perm[K, D].  Tile padding, re-reads and the (N/k)x dense work the
    method avoids are not counted.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    K = int(kept)
    up_proj = 2 if cfg.act == "swiglu" else 1
    fc1_w = used * (up_proj * cfg.F * cfg.D + (cfg.F if cfg.expert_bias else 0)) * es
    fc2_w = used * (cfg.D * cfg.F + (cfg.D if cfg.expert_bias else 0)) * es
    return {
        "fc1": {"flops": 2.0 * K * cfg.D * cfg.F * up_proj,
                "bytes": fc1_w + K * cfg.D * es + K * cfg.F * es},
        "fc2": {"flops": 2.0 * K * cfg.F * cfg.D,
                "bytes": fc2_w + K * cfg.F * es + K * cfg.D * es},
    }


def layer_flops(cfg, counts_kept):
    nproj = 3 if cfg.act == "swiglu" else 2
    return 2.0 * cfg.T * cfg.D * cfg.N + 2.0 * counts_kept * cfg.D * cfg.F * nproj


def _code_only(text):
    """Source text without comments, trailing blanks and empty lines: edits to
    comments alone leave the kernel, and so its counters, unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def sources_sha():
    h = hashlib.sha256()
    for rel in PMC_KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, launch):
    rec = PMC_TRAFFIC.get(workload)
    if rec is None or launch not in rec or rec["sources"] != sources_sha():
        return None
    return (rec[launch]["fetch_kib"] * 1024.0 * PMC_COPY_FACTOR["fetch"]
            + rec[launch]["write_kib"] * 1024.0 * PMC_COPY_FACTOR["write"])


def copy_calibration():
    """A plain elementwise copy (torch.neg, out=) of a known size: reads and
    writes COPY_BYTES each.  Under rocprofv3 --pmc its FETCH_SIZE/WRITE_SIZE
    give the scale from counter KiB to HBM bytes."""
    import torch
    n = 1 << 28  # fp32 elements: 1 GiB read, 1 GiB written
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "dispatches": 5}),
          flush=True)


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
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from mixture_experts_layer_expert_amd import api
    from workloads import generate, get_config, scaled_config

    cf = "keep" if args.cf is None else (None if args.cf < 0 else args.cf)
    cfg = get_config(args.workload, cf=cf)
    if args.expert_shard > 1:
        G = args.expert_shard
        if cfg.F % G or (cfg.F // G) % 32:
            raise SystemExit(f"--expert-shard {G}: F={cfg.F} must split into multiples of 32")
        cfg = scaled_config(cfg, F=cfg.F // G, name=f"{cfg.name}_fshare{G}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = generate(cfg)
    g0 = {k: (None if v is None else v.to(dev).contiguous()) for k, v in inp.items()}
    R = max(1, args.copies)
    # copy 0 is the generated tensors; the others are device clones (same
    # values, different addresses)
    gs = [g0] + [{k: (None if v is None else v.clone()) for k, v in g0.items()} for _ in range(R - 1)]
    shape = dataclasses.replace(api.MoeShape.from_config(cfg), slot_major=args.priority == "choice",
                                padded=args.layout == "padded")
    if shape.padded and shape.capacity < 0:
        raise SystemExit("--layout padded needs a capacity factor (--cf >= 0)")
    buf = api.MoeBuffers(shape, device=dev)
    A = cfg.T * cfg.k
    h = torch.empty(shape.group_rows, cfg.F, dtype=shape.torch_dtype, device=dev)
    y_perm = torch.empty(shape.group_rows, cfg.D, dtype=shape.torch_dtype, device=dev)
    st = torch.cuda.current_stream()
    rstats = args.router_stats
    if args.reroute and rstats:
        raise SystemExit("--reroute and --router-stats are separate router variants")
    if args.reroute:
        fb_idx = torch.empty(cfg.T, args.reroute, dtype=torch.int32, device=dev)
        fb_gate = torch.empty(cfg.T, args.reroute, dtype=torch.float32, device=dev)
    if rstats:
        stats_ws = torch.empty(api.stats_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        prob_mean = torch.empty(cfg.N, dtype=torch.float64, device=dev)
        frac = torch.empty(cfg.N, dtype=torch.float64, device=dev)
        summary = torch.empty(3, dtype=torch.float64, device=dev)

    def step(g, s, ev=None):
        if ev is not None:
            ev[0].record(s)
        if rstats:
            api.route_stats(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate,
                            stats_ws, None, s)
        elif args.reroute:
            api.route_fallback(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate,
                               args.reroute, fb_idx, fb_gate, None, s)
        else:
            api.route(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, None, s)
        if args.reroute:
            api.dispatch_reroute(shape, args.reroute, fb_idx, fb_gate, buf.topk_idx, buf.topk_gate, buf.counts,
                                 buf.offsets, buf.perm, buf.slot, buf.n_dropped, s)
        else:
            api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped, s,
                         ws=buf.ws)
        if rstats:
            api.router_stats(shape, stats_ws, buf.counts, buf.n_dropped, prob_mean, frac, summary, s)
        if ev is not None:
            ev[1].record(s)
        api.expert_up(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], h, buf.ws, s)
        if ev is not None:
            ev[2].record(s)
        api.expert_down(shape, h, buf.offsets, g["w2"], g["b2"], y_perm, buf.ws, s)
        if ev is not None:
            ev[3].record(s)
        api.combine(shape, y_perm, buf.slot, buf.topk_gate, g["x"], buf.out, s)
        if ev is not None:
            ev[4].record(s)

    for i in range(args.warmup):
        step(gs[i % R], st)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(st)
    for i in range(args.steps):
        step(gs[i % R], st, evs[i])
    t_end.record(st)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    def mean_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / args.steps

    stages = {"route+dispatch": mean_ms(0, 1), "fc1": mean_ms(1, 2), "fc2": mean_ms(2, 3),
              "combine": mean_ms(3, 4)}

    counts = buf.counts.cpu()
    # useful rows and experts (the padded layout's padding rows are excluded)
    kept_r = counts.clamp(max=shape.capacity) if shape.capacity >= 0 else counts
    if args.reroute:  # rows per expert: kept plus rerouted (compact layout)
        off = buf.offsets.cpu()
        kept_r = off[cfg.n_shared + 1:] - off[cfg.n_shared:-1]
    n_sh = cfg.n_shared if cfg.T > 0 else 0
    kept = cfg.n_shared * cfg.T + int(kept_r.sum())
    used = n_sh + int((kept_r > 0).sum())
    n_dropped = int(buf.n_dropped.cpu())
    work = launch_work(cfg, kept, used)
    lflops = layer_flops(cfg, kept)

    # the dominant launch: the longer of the two grouped-GEMM launches
    launch = "fc1" if stages["fc1"] >= stages["fc2"] else "fc2"
    flops, bytes_ = work[launch]["flops"], work[launch]["bytes"]
    t_s = stages[launch] / 1e3
    # both paths contract on MFMA: bf16 (2.5 PFLOP/s dense) or fp32 (157.3)
    mfma_peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if flops / bytes_ < ridge else "mfma"
    if bound == "hbm":
        achieved, peak, unit = bytes_ / t_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = flops / t_s / 1e12, mfma_peak, "TFLOP/s"
    act_name = {"gelu": "GELU", "relu": "ReLU", "swiglu": "SwiGLU"}[cfg.act]

    graph = None
    if not args.no_graph:
        # the same steps captured once per input copy and replayed; the
        # library allocates nothing and records no memset, so the capture is
        # a plain sequence of kernel nodes
        side = torch.cuda.Stream()
        side.wait_stream(st)
        graphs = []
        with torch.cuda.stream(side):
            for r in range(R):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=side):
                    step(gs[r], side)
                graphs.append(gr)
        st.wait_stream(side)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        g_start = torch.cuda.Event(enable_timing=True)
        g_end = torch.cuda.Event(enable_timing=True)
        g_start.record(st)
        for i in range(args.steps):
            graphs[i % R].replay()
        g_end.record(st)
        torch.cuda.synchronize()
        g_ms = g_start.elapsed_time(g_end) / args.steps
        graph = {"ms_per_step": g_ms, "tokens_per_s": cfg.T / (g_ms / 1e3)}

    # the timed steps: the graph replays (the same launches without the host's
    # per-launch cost, how a serving loop runs the layer), else the eager run
    eager = {"ms_per_step": ms_step, "tokens_per_s": cfg.T / (ms_step / 1e3)}
    if graph is not None:
        ms_step = graph["ms_per_step"]
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
                   "capacity": shape.capacity, "renorm": cfg.renorm, "residual": cfg.residual,
                   "capacity_priority": args.priority, "layout": args.layout,
                   "router_stats": args.router_stats, "reroute_levels": args.reroute,
                   "expert_shard": args.expert_shard, "input_copies": R},
        "layer_tflops": lflops / (ms_step / 1e3) / 1e12,
        "layer_tflops_frac_bf16_peak": lflops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "timed": "hip_graph_replay" if graph is not None else "eager",
        "eager": eager,
        "stages_ms": stages,  # from the eager run, HIP events between the launches
        "graph": graph,
        "routing": {"kept_assignments": kept, "dropped": n_dropped, "experts_used": used,
                    "max_count": int(counts.max()), "imbalance": float(counts.max()) / (A / cfg.N)},
        "router_stats": ({"aux_loss": float(summary[0]), "imbalance": float(summary[1]),
                          "drop_rate": float(summary[2])} if rstats else None),
        "roofline": {
            "kernel": (f"grouped_gemm_kernel, {launch} launch "
                       f"({'fc1 + ' + act_name if launch == 'fc1' else 'fc2'}; "
                       f"moe_expert_{'up' if launch == 'fc1' else 'down'}; with the split-K "
                       f"finishing kernel when its last round of tiles is split)"
                       if cfg.dtype == "bf16" else
                       f"grouped_gemm_f32_kernel, {launch} launch "
                       f"({'fc1 + ' + act_name if launch == 'fc1' else 'fc2'}; "
                       f"moe_expert_{'up' if launch == 'fc1' else 'down'})"),
            "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak,
            "traffic": (measured_traffic(args.workload, launch)
                        if args.cf is None and args.priority == "token" and args.layout == "compact"
                        and args.expert_shard == 1 and not args.reroute else None),
            "launch_ms": stages[launch],
            "algorithmic": {"flops": flops, "bytes": bytes_,
                            "rule": "used experts' weights once + activation rows in once + "
                                    "output rows once; 2 flops per MAC over kept rows"},
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.workload if args.workload in CPU_SAMPLE_TOKENS
                                           else "c2")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
