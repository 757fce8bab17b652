"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--extra c5,c2]
                    [--cf 1.0] [--copies 3] [--no-graph] [--no-cpu-baseline]
    python bench.py --copy-calibration     (plain copy of known size, for PMC scaling)

One step is one whole layer forward (router, dispatch with capacity, expert
MLPs, combine) over the workload's batch, inputs and weights already resident
in HBM.  The step runs the C-ABI chain moe_route -> moe_dispatch ->
moe_expert_up -> moe_expert_down -> moe_combine, each given the workspace
(the kernels of moe_forward, in the same order) with HIP events between the launches on the launch
stream, so every launch's duration is measured live.  Consecutive steps
cycle over --copies separate copies of x and the weights, so that no step
finds its weights in the 256 MB last-level cache from the step before.

The timed steps are the same chain captured once per input copy into HIP
graphs and replayed (W warm-up replays, then K timed ones between
synchronisations); the eager run before it supplies the per-launch HIP-event
timings and its own step time ("eager").  --no-graph times the eager steps.

The headline workload is the Mixtral-shaped prefill layer (c4, 8192 tokens,
MFMA-bound).  The same process then measures the extra workloads (default:
the decode layer c5, HBM-bound, and the Switch layer c2) and reports each
under "workloads" with its own step time, roofline and CPU baseline.  The
decode layer's graph replays are timed over max(K, 200) steps.

Prints one JSON line: tokens/s of the headline layer, the layer's fraction
of its roofline (MFMA for large prefill, HBM for weight streaming), the
roofline of its dominant launch with the sustained core clock measured
during that launch, and the CPU oracle timed on the host on a bounded sample
of the same workload.
"""
from __future__ import annotations

import os
import sys

# The CPU baseline's numpy BLAS takes its thread count when numpy is first
# imported: fix it before anything imports numpy.  A count already set in the
# environment (a box that grants this process a share of its cores) is kept.
_AFFINITY = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
    os.environ.setdefault(_v, str(_AFFINITY))

import argparse  # noqa: E402
import dataclasses  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import re  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA at 2.4 GHz
PEAK_FP32_TFLOPS = 157.3       # fp32 dense MFMA (the fp32 grouped GEMM runs on v_mfma_f32_16x16x4f32)
SPEC_CLOCK_GHZ = 2.4           # the clock the MFMA peaks are quoted at
METRIC = "MoE layer fwd tokens/s + TFLOP/s (% bf16 MFMA peak) or GB/s (% HBM peak), 1 GPU"
DEFAULT_WORKLOAD = "c4"
DEFAULT_EXTRA = "c5,c2"
MIN_STEPS = {"c5": 200}        # graph replays timed for the short decode step

# CPU-baseline sample (tokens) per workload: the oracle in fp64 on the host's
# cores for roughly 5-30 s.  The sample is the first T_s tokens of the same
# batch, with the capacity recomputed for T_s tokens.
CPU_SAMPLE_TOKENS = {"c1": 1024, "c2": 16384, "c3": 2048, "c4": 256, "c5": 128, "c6": 512}


# Counters of each launch, from rocprofv3 --pmc runs of the plain command of
# each workload (bench.py --workload W --extra= --steps 5 --warmup 2
# --no-cpu-baseline --no-clock; profiles/ has the commands and summaries):
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, each pass its own run), scaled
# by the ratio of known bytes to the counter's reading for a plain copy
# (--copy-calibration); and GRBM_GUI_ACTIVE (busy cycles summed over the 8
# XCDs) with SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) and the
# dispatch's duration, which give the sustained core clock and the MFMA pipe's
# busy share.  Values are averaged over the dispatches of the launch (its
# split-K finishing kernel included for the byte counts).  A figure is used
# only while the kernel sources hash to the value it was measured with;
# otherwise it is reported as null.
PMC_KERNEL_SOURCES = {
    "bf16": ("mixture_experts_layer_expert_amd/csrc/grouped_gemm.hip",
             "mixture_experts_layer_expert_amd/csrc/grouped_gemm.h"),
    "fp32": ("mixture_experts_layer_expert_amd/csrc/grouped_gemm_f32.hip",),
}
PMC_TRAFFIC = {
    "c1": {"sources": "49e725d5e2507400",
           "fc1": {"fetch_kib": 20173.7, "write_kib": 8192.0, "grbm": 661032, "mfma_busy": 17825792, "simds": 1024, "dur_ns": 29050},
           "fc2": {"fetch_kib": 40244.6, "write_kib": 2048.0, "grbm": 748271, "mfma_busy": 17301504, "simds": 1024, "dur_ns": 33490}},
    "c2": {"sources": "ed6681ec74ca2f0c",
           "fc1": {"fetch_kib": 309543.8, "write_kib": 92417.9, "grbm": 2765270, "mfma_busy": 75497472, "simds": 1024, "dur_ns": 150877},
           "fc2": {"fetch_kib": 340927.3, "write_kib": 22955.1, "grbm": 2739026, "mfma_busy": 75497472, "simds": 1024, "dur_ns": 146675}},
    "c3": {"sources": "ed6681ec74ca2f0c",
           "fc1": {"fetch_kib": 148745.8, "write_kib": 141793.3, "grbm": 2868067, "mfma_busy": 157286400, "simds": 1024, "dur_ns": 176008},
           "fc2": {"fetch_kib": 212622.9, "write_kib": 90011.0, "grbm": 2488982, "mfma_busy": 157286400, "simds": 1024, "dur_ns": 151083}},
    "c4": {"sources": "ed6681ec74ca2f0c",
           "fc1": {"fetch_kib": 3357288.2, "write_kib": 458877.3, "grbm": 42515886, "mfma_busy": 3992977408, "simds": 1024, "dur_ns": 3320489},
           "fc2": {"fetch_kib": 1904527.8, "write_kib": 208097.4, "grbm": 23433479, "mfma_busy": 1996488704, "simds": 1024, "dur_ns": 1848790}},
    "c5": {"sources": "ed6681ec74ca2f0c",
           "fc1": {"fetch_kib": 365940.4, "write_kib": 2114.0, "grbm": 2610259, "mfma_busy": 23068672, "simds": 1024, "dur_ns": 133482},
           "fc2": {"fetch_kib": 182876.2, "write_kib": 3072.1, "grbm": 1395272, "mfma_busy": 11534336, "simds": 1024, "dur_ns": 68048}},
    "c6": {"sources": "ed6681ec74ca2f0c",
           "fc1": {"fetch_kib": 584096.7, "write_kib": 90165.7, "grbm": 5644770, "mfma_busy": 461373440, "simds": 1024, "dur_ns": 379958},
           "fc2": {"fetch_kib": 270326.3, "write_kib": 135866.8, "grbm": 3769852, "mfma_busy": 230686720, "simds": 1024, "dur_ns": 229206}},
}
PMC_COPY_FACTOR = {"fetch": 1.99997, "write": 1.0}  # bytes per counter byte
# GRBM_GUI_ACTIVE also counts the counter window around the dispatch (about
# 15-20 thousand cycles per XCD, measured on 30-130 us launches): the clock it
# gives is used only for launches long enough for that to be under 1 %.
COUNTER_CLOCK_MIN_NS = 1_000_000


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="headline workload c1..c6 (default: c4, the Mixtral-shaped prefill layer)")
    ap.add_argument("--extra", default=None,
                    help="comma-separated extra workloads measured in the same run and reported under "
                         f"'workloads' (default {DEFAULT_EXTRA!r} with the default headline and options, "
                         "none otherwise; '' for none)")
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
    ap.add_argument("--no-clock", action="store_true", help="skip the clock probe during the dominant launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for PMC counter scaling)")
    return ap.parse_args()


def _es(cfg):
    return 2 if cfg.dtype == "bf16" else 4


def weight_bytes(cfg, used):
    """Bytes of the used experts' weights (and biases), per projection."""
    es = _es(cfg)
    up_proj = 2 if cfg.act == "swiglu" else 1
    fc1 = used * (up_proj * cfg.F * cfg.D + (cfg.F if cfg.expert_bias else 0)) * es
    fc2 = used * (cfg.D * cfg.F + (cfg.D if cfg.expert_bias else 0)) * es
    return fc1, fc2


def launch_work(cfg, kept, used, tokens_in):
    """Algorithmic FLOPs and bytes of the two expert launches.

    FLOPs: 2 per multiply-add over kept rows only (2*K*D*F per projection;
    fc1 of SwiGLU has two).  Bytes: every used expert's weights (and biases)
    once, plus for fc1 the x rows of the tokens it reads, once each
    (tokens_in: tokens with at least one kept row).  The hidden activations H
    that fc1 writes and fc2 reads, y_perm, the split-K partial tiles, tile
    padding, re-reads and the (N/k)x dense work the method avoids are
    implementation bytes: they appear in the counters' traffic, not here.
    """
    es = _es(cfg)
    K = int(kept)
    up_proj = 2 if cfg.act == "swiglu" else 1
    w1, w2 = weight_bytes(cfg, used)
    return {
        "fc1": {"flops": 2.0 * K * cfg.D * cfg.F * up_proj, "bytes": w1 + tokens_in * cfg.D * es},
        "fc2": {"flops": 2.0 * K * cfg.F * cfg.D, "bytes": w2},
    }


def layer_work(cfg, kept, used):
    """Algorithmic FLOPs and bytes of the whole layer: the router's logits
    (2*T*D*N) plus the expert projections over kept rows; the router weights,
    every used expert's weights once, x read once and out written once."""
    es = _es(cfg)
    nproj = 3 if cfg.act == "swiglu" else 2
    flops = 2.0 * cfg.T * cfg.D * cfg.N + 2.0 * kept * cfg.D * cfg.F * nproj
    w1, w2 = weight_bytes(cfg, used)
    bytes_ = cfg.N * cfg.D * es + w1 + w2 + 2 * cfg.T * cfg.D * es
    return flops, bytes_


def _code_only(text):
    """Source text without comments, indentation, trailing blanks and empty
    lines: edits to comments or layout alone leave the kernel, and so its
    counters, unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).strip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def pmc_sources(workload):
    """The GEMM sources whose kernels the workload's expert launches run."""
    from workloads import get_config
    return PMC_KERNEL_SOURCES[get_config(workload).dtype]


def sources_sha(files):
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _pmc(workload, launch):
    rec = PMC_TRAFFIC.get(workload)
    if rec is None or launch not in rec or rec["sources"] != sources_sha(pmc_sources(workload)):
        return None
    return rec[launch]


def measured_traffic(workload, launch):
    r = _pmc(workload, launch)
    if r is None:
        return None
    return (r["fetch_kib"] * 1024.0 * PMC_COPY_FACTOR["fetch"]
            + r["write_kib"] * 1024.0 * PMC_COPY_FACTOR["write"])


def counter_clock(workload, launch):
    """Sustained clock (GHz) and MFMA-busy share of the launch's main kernel
    from the counter run: GRBM_GUI_ACTIVE / 8 XCDs / duration, and
    SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / (GRBM_GUI_ACTIVE / 8)."""
    r = _pmc(workload, launch)
    if r is None or "grbm" not in r or r["dur_ns"] < COUNTER_CLOCK_MIN_NS:
        return None
    cycles = r["grbm"] / 8.0
    return {"ghz": cycles / (r["dur_ns"]), "mfma_busy": r["mfma_busy"] / r["simds"] / cycles,
            "source": "rocprofv3 counters of the same command (profiles/)"}


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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "host CPU"


def cpu_baseline(cfg, inp, key):
    """The oracle as it stands (fp64 numpy per-expert loop) on a bounded
    sample of the same batch, on the host's cores."""
    from threadpoolctl import threadpool_info

    import oracle
    Ts = min(cfg.T, CPU_SAMPLE_TOKENS.get(key, 1024))
    xs = inp["x"][:Ts]
    C = oracle.capacity(Ts, cfg.k, cfg.N, cfg.cf)
    t0 = time.perf_counter()
    r = oracle.moe_forward(xs, inp, k=cfg.k, act=cfg.act, renorm=cfg.renorm, capacity_slots=C,
                           residual=cfg.residual, n_shared=cfg.n_shared)
    dt = time.perf_counter() - t0
    del r
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    nproj = 3 if cfg.act == "swiglu" else 2
    flops = 2.0 * Ts * cfg.D * cfg.N + 2.0 * Ts * (cfg.k + cfg.n_shared) * cfg.D * cfg.F * nproj
    return {"value": Ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "gflops": flops / dt / 1e9, "precision": "fp64",
            "sample": f"first {Ts} of {cfg.T} tokens of the same batch (capacity "
                      f"{'none' if C is None else C} for {Ts} tokens), fp64 numpy per-expert loop, "
                      f"{dt:.2f} s on {_cpu_model()} with {threads} BLAS threads",
            "seconds": dt, "cpu_model": _cpu_model(), "affinity_cores": _AFFINITY}


def run_workload(key, args, *, headline):
    """Times one workload's layer; returns its JSON block.  The headline
    workload takes the command line's options and exactly --steps timed
    steps; an extra workload runs with its defaults."""
    import torch

    from mixture_experts_layer_expert_amd import api
    from workloads import generate, get_config, scaled_config

    if headline:
        opts = args
        cfg = get_config(key) if args.cf is None else get_config(key, cf=None if args.cf < 0 else args.cf)
    else:
        opts = argparse.Namespace(cf=None, priority="token", router_stats=False, reroute=0, expert_shard=1,
                                  layout="compact")
        cfg = get_config(key)
    plain = (opts.cf is None and opts.priority == "token" and not opts.router_stats and not opts.reroute
             and opts.expert_shard == 1 and opts.layout == "compact")
    if opts.expert_shard > 1:
        G = opts.expert_shard
        if cfg.F % G or (cfg.F // G) % 32:
            raise SystemExit(f"--expert-shard {G}: F={cfg.F} must split into multiples of 32")
        cfg = scaled_config(cfg, F=cfg.F // G, name=f"{cfg.name}_fshare{G}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = args.steps if headline else max(args.steps, MIN_STEPS.get(key, 0))

    inp = generate(cfg)
    g0 = {k: (None if v is None else v.to(dev).contiguous()) for k, v in inp.items()}
    R = max(1, args.copies)
    # copy 0 is the generated tensors; the others are device clones (same
    # values, different addresses)
    gs = [g0] + [{k: (None if v is None else v.clone()) for k, v in g0.items()} for _ in range(R - 1)]
    shape = dataclasses.replace(api.MoeShape.from_config(cfg), slot_major=opts.priority == "choice",
                                padded=opts.layout == "padded")
    if shape.padded and shape.capacity < 0:
        raise SystemExit("--layout padded needs a capacity factor (--cf >= 0)")
    buf = api.MoeBuffers(shape, device=dev)
    A = cfg.T * cfg.k
    h = torch.empty(shape.group_rows, cfg.F, dtype=shape.torch_dtype, device=dev)
    y_perm = torch.empty(shape.group_rows, cfg.D, dtype=shape.torch_dtype, device=dev)
    st = torch.cuda.current_stream()
    rstats = opts.router_stats
    if opts.reroute and rstats:
        raise SystemExit("--reroute and --router-stats are separate router variants")
    if opts.reroute:
        fb_idx = torch.empty(cfg.T, opts.reroute, dtype=torch.int32, device=dev)
        fb_gate = torch.empty(cfg.T, opts.reroute, dtype=torch.float32, device=dev)
    if rstats:
        stats_ws = torch.empty(api.stats_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        prob_mean = torch.empty(cfg.N, dtype=torch.float64, device=dev)
        frac = torch.empty(cfg.N, dtype=torch.float64, device=dev)
        summary = torch.empty(3, dtype=torch.float64, device=dev)

    def step(g, s, ev=None, probe=None):
        """One layer forward on stream s.  ev: 5 events recorded between the
        launches; probe(stage, stream) is called right after the launch of
        stage 'fc1' or 'fc2'."""
        if ev is not None:
            ev[0].record(s)
        if rstats:
            api.route_stats(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate,
                            stats_ws, None, s)
        elif opts.reroute:
            api.route_fallback(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate,
                               opts.reroute, fb_idx, fb_gate, None, s)
        else:
            api.route(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, None, s,
                      ws=buf.ws)
        if opts.reroute:
            api.dispatch_reroute(shape, opts.reroute, fb_idx, fb_gate, buf.topk_idx, buf.topk_gate, buf.counts,
                                 buf.offsets, buf.perm, buf.slot, buf.n_dropped, s)
        else:
            api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped, s,
                         ws=buf.ws)
        if rstats:
            api.router_stats(shape, stats_ws, buf.counts, buf.n_dropped, prob_mean, frac, summary, s)
        if ev is not None:
            ev[1].record(s)
        api.expert_up(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], h, buf.ws, s)
        if probe is not None:
            probe("fc1")
        if ev is not None:
            ev[2].record(s)
        api.expert_down(shape, h, buf.offsets, g["w2"], g["b2"], y_perm, buf.ws, s)
        if probe is not None:
            probe("fc2")
        if ev is not None:
            ev[3].record(s)
        api.combine(shape, y_perm, buf.slot, buf.topk_gate, g["x"], buf.out, s)
        if ev is not None:
            ev[4].record(s)

    # ---- eager run: per-launch HIP events on the launch stream
    for i in range(args.warmup):
        step(gs[i % R], st)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(st)
    for i in range(steps):
        step(gs[i % R], st, evs[i])
    t_end.record(st)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps

    def mean_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / steps

    stages = {"route+dispatch": mean_ms(0, 1), "fc1": mean_ms(1, 2), "fc2": mean_ms(2, 3),
              "combine": mean_ms(3, 4)}

    counts = buf.counts.cpu()
    slot = buf.slot.cpu()[:A].view(cfg.T, cfg.k)
    # useful rows and experts (the padded layout's padding rows are excluded)
    kept_r = counts.clamp(max=shape.capacity) if shape.capacity >= 0 else counts
    if opts.reroute:  # rows per expert: kept plus rerouted (compact layout)
        off = buf.offsets.cpu()
        kept_r = off[cfg.n_shared + 1:] - off[cfg.n_shared:-1]
    n_sh = cfg.n_shared if cfg.T > 0 else 0
    kept = cfg.n_shared * cfg.T + int(kept_r.sum())
    used = n_sh + int((kept_r > 0).sum())
    tokens_in = cfg.T if cfg.n_shared else int((slot >= 0).any(dim=1).sum())
    n_dropped = int(buf.n_dropped.cpu())
    work = launch_work(cfg, kept, used, tokens_in)
    lflops, lbytes = layer_work(cfg, kept, used)

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

    # ---- sustained clock during the dominant launch: a probe of one wave
    # per compute unit on a second stream, sharing the GEMM's compute units
    # (it needs a few registers and no LDS), waits a sixth of the launch and
    # counts shader cycles over the next half.  It only counts when its end
    # falls inside the launch (events on both streams).
    clock = None
    if not args.no_clock:
        ps = torch.cuda.Stream()
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        stamps = torch.zeros(4 * n_cu, dtype=torch.int64, device=dev)
        launch_us = stages[launch] * 1e3
        # wait a sixth of the launch, then a chain that lasts about half of
        # it at 2.4 GHz (longer at a lower clock): 4 clocks per add, 1024
        # adds per block
        delay_us = launch_us / 6.0
        iters = max(1, min(1 << 16, int(launch_us * 2400.0 / 2.0 / 4096.0)))
        readings = []
        for i in range(3):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            pe = torch.cuda.Event(enable_timing=True)

            a, b = (1, 2) if launch == "fc1" else (2, 3)

            def probe(stage, _pe=pe, _ev=ev, _a=a):
                if stage == launch:
                    # start with the launch: the probe stream waits for the
                    # event recorded just before it
                    ps.wait_event(_ev[_a])
                    api.clock_probe(n_cu, delay_us, iters, stamps, ps)
                    _pe.record(ps)

            step(gs[i % R], st, ev, probe)
            torch.cuda.synchronize()
            inside = ev[a].elapsed_time(pe) <= ev[a].elapsed_time(ev[b])
            readings.append((api.probe_clock_ghz(stamps), inside))
        good = sorted(c for c, ok in readings if ok)
        if good:
            ghz = good[len(good) // 2]
            clock = {"ghz": ghz, "probes_inside_launch": len(good), "probes": len(readings),
                     "method": "moe_clock_probe: a chain of dependent 32-bit adds (4 shader clocks each) timed "
                               "with the 100 MHz real-time counter, one wave per CU on a second stream, inside "
                               "the dominant launch"}
        else:
            clock = {"ghz": None, "probes_inside_launch": 0, "probes": len(readings),
                     "idle_ghz": [c for c, _ in readings]}

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
        for i in range(steps):
            graphs[i % R].replay()
        g_end.record(st)
        torch.cuda.synchronize()
        g_ms = g_start.elapsed_time(g_end) / steps
        graph = {"ms_per_step": g_ms, "tokens_per_s": cfg.T / (g_ms / 1e3)}
        del graphs

    eager = {"ms_per_step": ms_step, "tokens_per_s": cfg.T / (ms_step / 1e3)}
    if graph is not None:
        ms_step = graph["ms_per_step"]
    step_s = ms_step / 1e3
    lbound = "hbm" if lflops / lbytes < ridge else "mfma"
    layer = {"flops": lflops, "bytes": lbytes, "tflops": lflops / step_s / 1e12, "gbs": lbytes / step_s / 1e9,
             "bound": lbound,
             "frac": (lflops / step_s / 1e12 / mfma_peak) if lbound == "mfma" else (lbytes / step_s / 1e9 / PEAK_HBM_GBS),
             "rule": "router logits + expert projections over kept rows (2 flops per MAC); router weights + "
                     "used experts' weights once + x read once + out written once"}
    roof = {
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
        "traffic": measured_traffic(key, launch) if plain else None,
        "launch_ms": stages[launch],
        "algorithmic": {"flops": flops, "bytes": bytes_,
                        "rule": "used experts' weights once (+ x rows read once for fc1); hidden rows, "
                                "y_perm and partial tiles are implementation bytes; 2 flops per MAC over "
                                "kept rows"},
    }
    cclk = counter_clock(key, launch) if plain else None
    if cclk is not None:
        roof["counters"] = cclk
    ghz = (clock or {}).get("ghz") or (cclk or {}).get("ghz")
    if ghz:
        roof["clock_ghz"] = ghz
        roof["clock_source"] = "moe_clock_probe during the launch" if (clock or {}).get("ghz") else cclk["source"]
        if bound == "mfma":
            roof["peak_at_clock"] = peak * ghz / SPEC_CLOCK_GHZ
            roof["frac_at_clock"] = achieved / roof["peak_at_clock"]
    block = {
        "workload": cfg.name,
        "value": cfg.T / step_s,
        "unit": "tokens/s",
        "ms_per_step": ms_step,
        "steps": steps,
        "timed": "hip_graph_replay" if graph is not None else "eager",
        "dtype": cfg.dtype,
        "config": {"workload": cfg.name, "tokens": cfg.T, "D": cfg.D, "F": cfg.F, "experts": cfg.N,
                   "top_k": cfg.k, "act": cfg.act, "capacity_factor": cfg.cf,
                   "capacity": shape.capacity, "renorm": cfg.renorm, "residual": cfg.residual,
                   "shared_experts": cfg.n_shared,
                   "capacity_priority": opts.priority, "layout": opts.layout,
                   "router_stats": opts.router_stats, "reroute_levels": opts.reroute,
                   "expert_shard": opts.expert_shard, "input_copies": R},
        "layer": layer,
        "layer_tflops": lflops / step_s / 1e12,
        "layer_tflops_frac_bf16_peak": lflops / step_s / 1e12 / PEAK_BF16_TFLOPS,
        "eager": eager,
        "stages_ms": stages,  # from the eager run, HIP events between the launches
        "graph": graph,
        "clock": clock,
        "routing": {"kept_assignments": kept, "dropped": n_dropped, "experts_used": used,
                    "max_count": int(counts.max()), "imbalance": float(counts.max()) / (A / cfg.N)},
        "router_stats": ({"aux_loss": float(summary[0]), "imbalance": float(summary[1]),
                          "drop_rate": float(summary[2])} if rstats else None),
        "roofline": roof,
    }
    del gs, g0, buf, h, y_perm
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        block["cpu_baseline"] = cpu_baseline(cfg, inp, key if key in CPU_SAMPLE_TOKENS else "c2")
    return block


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    plain = (args.cf is None and args.priority == "token" and not args.router_stats
             and not args.reroute and args.expert_shard == 1 and args.layout == "compact")
    extra = args.extra
    if extra is None:
        extra = DEFAULT_EXTRA if (args.workload == DEFAULT_WORKLOAD and plain) else ""
    extras = [w for w in extra.split(",") if w and w != args.workload]

    head = run_workload(args.workload, args, headline=True)
    blocks = {}
    for w in extras:
        b = run_workload(w, args, headline=False)
        blocks[b["workload"]] = b

    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
    }
    for k in ("config", "layer", "layer_tflops", "layer_tflops_frac_bf16_peak", "timed", "eager", "stages_ms",
              "graph", "clock", "routing", "router_stats", "roofline", "cpu_baseline"):
        if k in head:
            res[k] = head[k]
    res["workloads"] = blocks
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
