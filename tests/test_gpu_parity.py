"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Routing (expert indices, counts, offsets, permutation, slots, dropped set)
must match bit-exactly; gates within 1e-6; outputs within the row-relative
tolerance of their dtype (2e-2 bf16, 1e-4 fp32).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_expert_amd import api
from parity import GATE_ATOL, LOGIT_ATOL, TOL, capacity_of, check_outputs, check_routing, oracle_layer, row_rel_err, run_forward, to_gpu
from workloads import CONFIGS, generate, get_config, scaled_config

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# --------------------------------------------------------------- router
@pytest.mark.parametrize("key", sorted(CONFIGS) + ["c5:ws"])
def test_route_full_size(gpu, key):
    """Every workload's router at full size; "c5:ws" gives moe_route the
    workspace, which sends its 128 tokens through the split router."""
    key, _, mode = key.partition(":")
    cfg = CONFIGS[key]
    _say(f"route {cfg.name} {mode}")
    inp = generate(cfg, parts=("x", "router"))
    ref = oracle.route(inp["x"], inp["w_router"], inp["b_router"], cfg.k, cfg.renorm)
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg)
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=gpu)
    gate = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=gpu)
    logits = torch.empty(cfg.T, cfg.N, dtype=torch.float32, device=gpu)
    ws = torch.empty(api.workspace_bytes(shape), dtype=torch.uint8, device=gpu) if mode == "ws" else None
    api.route(shape, g["x"], g["w_router"], g["b_router"], idx, gate, logits, ws=ws)
    torch.cuda.synchronize()
    gerr = np.abs(gate.cpu().numpy() - ref["gate"]).max()
    lerr = np.abs(logits.cpu().numpy() - ref["logits"]).max()
    _say(f"  gate err {gerr:.2e}  logit err {lerr:.2e}")
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    assert gerr <= GATE_ATOL[cfg.dtype]
    assert lerr <= LOGIT_ATOL


def _stats_case(gpu, cfg, inp):
    """moe_route_stats + moe_dispatch + moe_router_stats against the
    oracle's router statistics.  Routing equals moe_route's bit for bit;
    f_e, the imbalance and the drop rate are exact (ratios of integers,
    correctly rounded in fp64 on both sides); P_e is a mean of softmax
    probabilities, so it takes the gates' tolerance, and the loss
    N * sum f_e P_e then moves by at most N * sum f_e * tol = N * k * tol."""
    T, N, k = cfg.T, cfg.N, cfg.k
    shape = api.MoeShape.from_config(cfg)
    g = to_gpu(inp)
    ws = torch.empty(api.stats_workspace_bytes(shape), dtype=torch.uint8, device=gpu)
    buf = api.MoeBuffers(shape)
    api.route_stats(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, ws)
    idx2 = torch.empty_like(buf.topk_idx)
    gate2 = torch.empty_like(buf.topk_gate)
    api.route(shape, g["x"], g["w_router"], g["b_router"], idx2, gate2)
    api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped)
    f64 = dict(dtype=torch.float64, device=gpu)
    outs = []
    for _ in range(2):
        pm, fr, sm = torch.full((N,), -1.0, **f64), torch.full((N,), -1.0, **f64), torch.full((3,), -1.0, **f64)
        api.router_stats(shape, ws, buf.counts, buf.n_dropped, pm, fr, sm)
        outs.append((pm, fr, sm))
    torch.cuda.synchronize()
    assert torch.equal(buf.topk_idx, idx2) and torch.equal(buf.topk_gate, gate2)
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b), "repeated statistics differ"
    pm, fr, sm = (t.cpu().numpy() for t in outs[0])
    r = oracle.route(inp["x"], inp["w_router"], inp["b_router"], k, cfg.renorm)
    assert np.array_equal(buf.topk_idx.cpu().numpy(), r["idx"])
    counts = oracle.expert_counts(r["idx"], N)
    ref = oracle.router_stats(r["idx"], r["probs"], counts, N, capacity_of(cfg))
    tol = GATE_ATOL[cfg.dtype]
    perr = np.abs(pm - ref["prob_mean"]).max()
    aerr = abs(sm[0] - ref["aux_loss"])
    _say(f"  P err {perr:.2e}  aux {sm[0]:.6f} (oracle {ref['aux_loss']:.6f}, err {aerr:.2e})  "
         f"imbalance {sm[1]:.4f}  drop {sm[2]:.4f}")
    assert np.array_equal(fr, ref["frac"])
    assert sm[1] == ref["imbalance"] and sm[2] == ref["drop_rate"]
    assert perr <= tol
    assert aerr <= N * k * tol


@pytest.mark.parametrize("key", sorted(CONFIGS))
def test_router_stats_full_size(gpu, key):
    cfg = CONFIGS[key]
    _say(f"router stats {cfg.name}")
    _stats_case(gpu, cfg, generate(cfg, parts=("x", "router")))


@pytest.mark.parametrize("key,T,N,k", [("c2", 9000, None, None), ("c2", 1000, None, None), ("c2", 1, None, None),
                                       ("c1", 37, None, None), ("c5", 333, None, None), ("c2", 3000, 256, 8)])
def test_router_stats_block_shapes(gpu, key, T, N, k):
    """Other tokens-per-block choices (64, 32, 16 rows), ragged last blocks
    and the widest expert count."""
    base = CONFIGS[key]
    cfg = scaled_config(base, T=T, N=N or base.N, k=k or base.k)
    _say(f"router stats {cfg.name} T={T} N={cfg.N} k={cfg.k}")
    _stats_case(gpu, cfg, generate(cfg, parts=("x", "router")))


def test_router_stats_graph_replay(gpu):
    """route_stats + dispatch + router_stats captured in a HIP graph, the
    second pass forked to another stream: every replay equals the eager
    statistics bit for bit."""
    cfg = scaled_config(CONFIGS["c2"], T=4096)
    shape = api.MoeShape.from_config(cfg)
    g = to_gpu(generate(cfg, parts=("x", "router")))
    ws = torch.empty(api.stats_workspace_bytes(shape), dtype=torch.uint8, device=gpu)
    buf = api.MoeBuffers(shape)
    f64 = dict(dtype=torch.float64, device=gpu)
    pm, fr, sm = torch.empty(cfg.N, **f64), torch.empty(cfg.N, **f64), torch.empty(3, **f64)

    def run(s, aux):
        api.route_stats(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, ws, None, s)
        api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped, s)
        aux.wait_stream(s)
        api.router_stats(shape, ws, buf.counts, buf.n_dropped, pm, fr, sm, aux)
        s.wait_stream(aux)

    st, aux = torch.cuda.current_stream(), torch.cuda.Stream()
    run(st, aux)
    torch.cuda.synchronize()
    want = [t.clone() for t in (pm, fr, sm)]
    side, side_aux = torch.cuda.Stream(), torch.cuda.Stream()
    side.wait_stream(st)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(side, side_aux)
    st.wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (pm, fr, sm):
            t.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((pm, fr, sm), want):
            assert torch.equal(a, b), rep
        run(st, aux)  # eager work between replays
        torch.cuda.synchronize()


def _route_case(gpu, x, w, k, renorm=False, b=None, split=False):
    """moe_route against the oracle.  split: with the workspace, so that bf16
    batches of at most 1024 tokens with D a multiple of 128 take the split
    router (F = 2048 leaves room for its partial tiles in the workspace)."""
    T, D = x.shape
    N = w.shape[0]
    dt = "bf16" if x.dtype == torch.bfloat16 else "fp32"
    shape = api.MoeShape(T=T, D=D, F=2048 if split else 64, N=N, k=k, dtype=dt, act="relu", renorm=renorm,
                         router_bias=b is not None)
    if split:  # the split router's conditions, and room for its partial tiles after y_perm
        assert dt == "bf16" and D % 128 == 0 and T <= 1024
        y_perm_bytes = (shape.group_rows * D * 2 + 255) // 256 * 256
        assert (D // 128) * T * ((N + 15) // 16 * 16) * 4 <= api.workspace_bytes(shape) - y_perm_bytes
    idx = torch.empty(T, k, dtype=torch.int32, device=gpu)
    gate = torch.empty(T, k, dtype=torch.float32, device=gpu)
    logits = torch.empty(T, N, dtype=torch.float32, device=gpu)
    ws = torch.empty(api.workspace_bytes(shape), dtype=torch.uint8, device=gpu) if split else None
    api.route(shape, x.to(gpu), w.to(gpu), None if b is None else b.to(gpu), idx, gate, logits, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.route(x, w, b, k, renorm)
    got = idx.cpu().numpy()
    bad = np.nonzero((got != ref["idx"]).any(axis=1))[0]
    for t in bad[:5]:
        _say(f"token {t}: gpu idx {got[t].tolist()} oracle {ref['idx'][t].tolist()}\n"
             f"  gpu logits {logits[t].cpu().numpy().tolist()}\n  oracle {ref['logits'][t].tolist()}")
    if bad.size:
        _say(f"{bad.size} mismatching tokens of {T}: {bad[:20].tolist()}")
    return got, gate.cpu().numpy(), ref


@pytest.mark.parametrize("dtype,D,split", [(torch.bfloat16, 64, False), (torch.float32, 64, False),
                                           (torch.bfloat16, 256, True)])
def test_route_exact_ties_go_to_lower_index(gpu, dtype, D, split):
    """Small-integer inputs make logits exact integers with many ties; a
    duplicated router row ties two experts on every token.  The split case
    sums two exact partial tiles per logit."""
    g = torch.Generator().manual_seed(0)
    T, N = 333, 8
    x = torch.randint(-2, 3, (T, D), generator=g).to(dtype)
    w = torch.randint(-1, 2, (N, D), generator=g).to(dtype)
    w[7] = w[2]
    for k in (1, 2, 5, N):
        idx, gate, ref = _route_case(gpu, x, w, k, split=split)
        assert np.array_equal(idx, ref["idx"]), k
        assert np.abs(gate - ref["gate"]).max() <= 1e-6  # every token re-ranked in fp64


@pytest.mark.parametrize("N,k", [(1, 1), (2, 2), (16, 8), (40, 3), (64, 6), (200, 3), (256, 8), (256, 1)])
def test_route_shapes(gpu, N, k):
    """Ragged token counts against the 64-, 16- and 4-token blocks, the one-
    and the split router (D = 384: three partial tiles per logit), expert
    counts that fill 16-wide tiles partly."""
    g = torch.Generator().manual_seed(N * 10 + k)
    T, D = 1000, 384
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, D, generator=g) * 0.05).to(torch.bfloat16)
    b = torch.randn(N, generator=g) * 0.1
    for split in (False, True):
        for renorm in (False, True):
            idx, gate, ref = _route_case(gpu, x, w, k, renorm, b, split)
            assert np.array_equal(idx, ref["idx"]), (split, renorm)
            assert np.abs(gate - ref["gate"]).max() <= GATE_ATOL["bf16"]


@pytest.mark.parametrize("N,D,k,bias,renorm,ties", [(128, 768, 1, False, False, False),
                                                     (100, 256, 2, True, True, False),
                                                     (65, 128, 8, True, False, False),
                                                     (128, 768, 2, False, False, True)])
def test_route_two_blocks_per_cu(gpu, N, D, k, bias, renorm, ties):
    """The ring router's mode for 65-128 experts and at least 64 tokens per
    CU (32-token blocks, two to a CU, the Switch layer's): a ragged last
    block, expert counts off the 16-wide tiles, 1, 2 and 6 k steps of 128,
    router bias and renormalisation, and small-integer inputs with a
    duplicated router row, where every token ties and is re-ranked from
    exact products."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = 64 * cus + 45
    g = torch.Generator().manual_seed(N * 100 + D + k)
    if ties:
        x = torch.randint(-2, 3, (T, D), generator=g).to(torch.bfloat16)
        w = torch.randint(-1, 2, (N, D), generator=g).to(torch.bfloat16)
        w[N - 1] = w[3]
    else:
        x = torch.randn(T, D, generator=g).to(torch.bfloat16)
        w = (torch.randn(N, D, generator=g) * 0.02).to(torch.bfloat16)
    b = torch.randn(N, generator=g) * 0.1 if bias else None
    _say(f"router, two blocks per CU: T={T} N={N} D={D} k={k} bias={bias} renorm={renorm} ties={ties}")
    idx, gate, ref = _route_case(gpu, x, w, k, renorm, b)
    assert np.array_equal(idx, ref["idx"])
    assert np.abs(gate - ref["gate"]).max() <= (1e-6 if ties else GATE_ATOL["bf16"])


@pytest.mark.parametrize("T,N,k", [(1, 8, 2), (15, 40, 3), (16, 64, 6), (17, 256, 8), (1024, 1, 1),
                                   (1024, 129, 1)])
def test_route_split_edges(gpu, T, N, k):
    """The split router (moe_route given the workspace) at its edges: fewer
    tokens than one 16-token tile, one tile plus one token, its largest
    batch, expert counts off the 16-wide tiles and the widest expert count
    (four 64-expert groups per token tile)."""
    g = torch.Generator().manual_seed(T * 1000 + N)
    D = 256  # two partial slices per logit
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, D, generator=g) * 0.05).to(torch.bfloat16)
    b = torch.randn(N, generator=g) * 0.1
    for renorm in (False, True):
        idx, gate, ref = _route_case(gpu, x, w, k, renorm, b, split=True)
        assert np.array_equal(idx, ref["idx"]), renorm
        assert np.abs(gate - ref["gate"]).max() <= GATE_ATOL["bf16"]


# ------------------------------------------------------------- dispatch
def _dispatch_case(gpu, idx_np, N, C, priority="token", padded=False):
    """Both dispatch paths against the oracle: one workgroup (no scratch; its
    register mode of 1, 4 or 24 chunks per wave, or none, by batch size) and,
    given the workspace, many workgroups for batches of more than 4096
    assignments."""
    for multi in (False, True):
        _dispatch_once(gpu, idx_np, N, C, priority, padded, multi)


def _dispatch_once(gpu, idx_np, N, C, priority, padded, multi):
    T, k = idx_np.shape
    shape = api.MoeShape(T=T, D=64, F=64, N=N, k=k, capacity=-1 if C is None else C, act="relu",
                         slot_major=(priority == "choice"), padded=padded)
    i32 = dict(dtype=torch.int32, device=gpu)
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(gpu)
    counts = torch.full((N,), -7, **i32)
    offsets = torch.full((N + 1,), -7, **i32)
    perm = torch.full((max(shape.group_rows, 1) + 5,), -7, **i32)
    slot = torch.full((T * k,), -7, **i32)
    nd = torch.full((1,), -7, **i32)
    ws = torch.empty(api.workspace_bytes(shape), dtype=torch.uint8, device=gpu) if multi else None
    api.dispatch(shape, idx, counts, offsets, perm, slot, nd, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx_np, N, C, priority)
    if padded:
        ref = oracle.padded(ref, N, C)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    K = int(ref["offsets"][-1])
    p = perm.cpu().numpy()
    # padding rows (oracle -1) hold assignment 0 on the GPU
    assert np.array_equal(p[:K], np.where(ref["perm"] < 0, 0, ref["perm"]))
    assert np.all(p[K:] == -7), "entries past offsets[N] must stay untouched"
    assert np.array_equal(slot.cpu().numpy(), ref["slot"])
    assert int(nd.item()) == ref["n_dropped"]


def _rand_idx(rng, T, N, k, p=None):
    if p is None and k == 1:
        return rng.integers(0, N, size=(T, 1))
    return np.stack([rng.choice(N, size=k, replace=False, p=p) for _ in range(T)])


@pytest.mark.parametrize("T,N,k,C", [
    (1, 1, 1, None), (1, 4, 4, None), (128, 64, 6, None), (500, 64, 2, 40), (1024, 8, 1, None),
    (777, 8, 2, None), (777, 8, 2, 150), (2000, 128, 1, 15),
    (2000, 128, 1, 0), (3001, 16, 2, 1), (5000, 64, 6, None), (5000, 64, 6, 50), (5000, 64, 6, 480),
    (16384, 128, 1, 128), (40000, 256, 2, 300),
])
def test_dispatch_random(gpu, T, N, k, C):
    rng = np.random.default_rng(T + N + k)
    _dispatch_case(gpu, _rand_idx(rng, T, N, k), N, C)


def test_dispatch_adversarial(gpu):
    rng = np.random.default_rng(1)
    # every token on expert 0 (k=1), and on experts (3, 0) for k=2
    _dispatch_case(gpu, np.zeros((3000, 1), dtype=np.int64), 8, None)
    _dispatch_case(gpu, np.zeros((3000, 1), dtype=np.int64), 8, 100)
    _dispatch_case(gpu, np.tile([3, 0], (2500, 1)), 8, 2000)
    # empty experts: only even ids used
    _dispatch_case(gpu, 2 * _rand_idx(rng, 1500, 8, 2), 16, None)
    # k = N: every expert gets every token
    _dispatch_case(gpu, np.stack([rng.permutation(6) for _ in range(999)]), 6, 500)
    # skewed (Zipf-like) routing
    p = 1.0 / np.arange(1, 17) ** 1.2
    _dispatch_case(gpu, _rand_idx(rng, 4096, 16, 2, p / p.sum()), 16, None)
    # ids outside [0, N) are dropped and not counted
    bad = _rand_idx(rng, 1200, 8, 2)
    bad[::7, 0] = -1
    bad[::11, 1] = 8
    _dispatch_case(gpu, bad, 8, None)
    _dispatch_case(gpu, bad, 8, 120)


@pytest.mark.parametrize("T,N,k,C", [
    (1, 4, 4, None), (777, 8, 2, 150), (3001, 16, 2, 1), (5000, 64, 6, 60), (2000, 128, 1, 15),
    (4096, 16, 2, 300), (40000, 256, 2, 300), (999, 6, 6, 500),
])
def test_dispatch_choice_priority(gpu, T, N, k, C):
    """MOE_SLOT_MAJOR: each expert keeps assignments in (choice, token) order."""
    rng = np.random.default_rng(3 * T + N + k)
    _dispatch_case(gpu, _rand_idx(rng, T, N, k), N, C, "choice")
    p = 1.0 / np.arange(1, N + 1) ** 1.2
    _dispatch_case(gpu, _rand_idx(rng, T, N, k, p / p.sum()), N, C, "choice")


# ----------------------------------------------- scaled layers, every token
SCALED = {
    "c1": get_config("c1"),
    "c2": scaled_config(get_config("c2"), T=2000),
    "c2cf15": scaled_config(get_config("c2", cf=1.5), T=2000),
    "c3": scaled_config(get_config("c3"), T=1500),
    "c4": scaled_config(get_config("c4"), T=700, D=1024, F=2048),
    "c5": get_config("c5"),
    # shared (always-on) experts next to the routed ones
    "c6": scaled_config(get_config("c6"), T=600, D=1024, F=512),
    "c6cf": scaled_config(get_config("c6", cf=1.0), T=300, D=512, F=256, N=16, k=2, n_shared=1),
    "c1sh": scaled_config(get_config("c1"), T=256, init="normal0.02", n_shared=2, name="c1_shared"),
    # fp32 with D and F multiples of 16 but not of 64: the last k step of both
    # projections is partial, and so is the last 64-column tile
    "c1k": scaled_config(get_config("c1"), T=300, D=80, F=208, name="c1_ragged_k"),
    "c1sw": scaled_config(get_config("c1"), T=300, D=112, F=176, act="swiglu", expert_bias=False,
                          init="normal0.02", name="c1_swiglu"),
    # few rows per expert -> fused weight-streaming path
    "c3dec": scaled_config(get_config("c3"), T=64, name="c3_skew_decode"),
    "c2dec": scaled_config(get_config("c2"), T=1000, name="c2_switch_decode"),
    # decode shape with F = 512: the fused kernel's 128-column shards
    "c5f512": scaled_config(get_config("c5"), F=512, name="c5_decode_f512"),
    # decode shapes the fused kernel does not take (D not a multiple of 128;
    # no shard of F among its compiled widths): the flag falls back to the
    # grouped GEMMs
    "c5d192": scaled_config(get_config("c5"), D=192, name="c5_decode_d192"),
    "c5f1600": scaled_config(get_config("c5"), F=1600, name="c5_decode_f1600"),
}


@pytest.fixture(scope="module")
def scaled_cases():
    return {}


def _scaled(key, cache):
    if key not in cache:
        cfg = SCALED[key]
        inp = generate(cfg)
        cache[key] = (cfg, inp, oracle_layer(cfg, inp))
    return cache[key]


FUSED = {"c5", "c3dec", "c2dec", "c5f512", "c5d192", "c5f1600"}  # also run with the fused decode flag


@pytest.mark.parametrize("key", sorted(SCALED) + sorted(k + ":fused" for k in FUSED))
def test_forward_scaled(gpu, key, scaled_cases):
    key, _, mode = key.partition(":")
    cfg, inp, ref = _scaled(key, scaled_cases)
    _say(f"forward scaled {key} {mode}: T={cfg.T} D={cfg.D} F={cfg.F} N={cfg.N} k={cfg.k}")
    g = to_gpu(inp)
    buf = run_forward(cfg, g, fused_decode=(mode == "fused"))
    check_routing(buf, ref, cfg)
    y = buf.out.float().cpu().numpy().astype(np.float64)
    err = check_outputs(y, ref, cfg, inp["x"].double().numpy())
    _say(f"  row-rel err {err:.3e}")
    # a second call gives the same bits (no order-dependent accumulation)
    out1 = buf.out.clone()
    buf.forward(g["x"], g)
    torch.cuda.synchronize()
    assert torch.equal(out1, buf.out)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5", "c6", "c6cf", "c1sh", "c3dec", "c2dec",
                                 "c5:fused", "c3dec:fused"])
def test_stage_chain(gpu, key, scaled_cases):
    """route -> dispatch -> expert_ffn -> combine, each stage also checked
    alone against the oracle with oracle-made inputs."""
    key, _, mode = key.partition(":")
    fused = mode == "fused"
    cfg, inp, ref = _scaled(key, scaled_cases)
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg, fused_decode=fused)
    buf = api.MoeBuffers(shape)
    # given the workspace, the router makes moe_forward's choice of kernels
    api.route(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, ws=buf.ws)
    api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped)
    A = shape.group_rows
    y_perm = torch.empty(A, cfg.D, dtype=shape.torch_dtype, device=gpu)
    api.expert_ffn(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], g["w2"], g["b2"],
                   y_perm, buf.ws)
    out = torch.empty_like(buf.out)
    api.combine(shape, y_perm, buf.slot, buf.topk_gate, g["x"], out)
    torch.cuda.synchronize()
    check_routing(buf, ref, cfg)
    K = int(ref["offsets"][-1])
    yp = y_perm[:K].float().cpu().numpy().astype(np.float64)
    assert row_rel_err(yp, ref["y_perm"]) <= TOL[cfg.dtype]
    # The whole chain equals moe_forward bit for bit on the grouped-GEMM path
    # (same kernels, same order).  With the fused decode kernel moe_forward
    # combines straight from the fp32 shard partials while the stage API
    # rounds y_perm to bf16 first, so the two differ by that one rounding.
    fw = run_forward(cfg, g, fused_decode=fused)
    if fused:
        d = row_rel_err(out.float().cpu().numpy().astype(np.float64),
                        fw.out.float().cpu().numpy().astype(np.float64))
        assert d <= 8e-3, d
    else:
        assert torch.equal(out, fw.out)
    # combine alone on oracle rows rounded to the layer dtype
    yr = torch.from_numpy(ref["y_perm"]).to(shape.torch_dtype)
    y_in = torch.zeros(A, cfg.D, dtype=shape.torch_dtype)
    y_in[:K] = yr
    gate = torch.from_numpy(ref["gate"].astype(np.float32))
    slot = torch.from_numpy(ref["slot"].astype(np.int32))
    out2 = torch.empty_like(buf.out)
    api.combine(shape, y_in.to(gpu), slot.to(gpu), gate.to(gpu), g["x"], out2)
    torch.cuda.synchronize()
    want = oracle.combine_rows(y_in.double().numpy(), ref["slot"], gate.double().numpy(), cfg.k,
                               inp["x"] if cfg.residual else None, n_shared=cfg.n_shared)
    tol = 1e-6 if cfg.dtype == "fp32" else 8e-3  # one final rounding to the layer dtype
    assert row_rel_err(out2.float().cpu().numpy().astype(np.float64), want) <= tol


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5", "c6", "c1sh"])
def test_expert_up_down(gpu, key, scaled_cases):
    """fc1(+act) and fc2 as separate launches: H against the oracle's hidden
    rows, fc2 alone on the oracle's H, and up+down equal to moe_expert_ffn."""
    cfg, inp, ref = _scaled(key, scaled_cases)
    _say(f"expert up/down {key}: T={cfg.T} D={cfg.D} F={cfg.F} N={cfg.N} k={cfg.k} {cfg.act}")
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg)
    buf = api.MoeBuffers(shape)
    # given the workspace, the router makes moe_forward's choice of kernels
    api.route(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, ws=buf.ws)
    api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped)
    A = shape.group_rows
    h = torch.empty(A, cfg.F, dtype=shape.torch_dtype, device=gpu)
    y_ud = torch.empty(A, cfg.D, dtype=shape.torch_dtype, device=gpu)
    y_ffn = torch.empty_like(y_ud)
    # with the workspace (split-K of a partial last round allowed, as in
    # moe_expert_ffn) and without (never split)
    api.expert_up(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], h, buf.ws)
    api.expert_down(shape, h, buf.offsets, g["w2"], g["b2"], y_ud, buf.ws)
    api.expert_ffn(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], g["w2"], g["b2"],
                   y_ffn, buf.ws)
    h_ns = torch.empty_like(h)
    y_ns = torch.empty_like(y_ud)
    api.expert_up(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], h_ns)
    api.expert_down(shape, h_ns, buf.offsets, g["w2"], g["b2"], y_ns)
    torch.cuda.synchronize()
    check_routing(buf, ref, cfg)
    off, perm = ref["offsets"], ref["perm"]
    K = int(off[-1])
    assert torch.equal(y_ud[:K], y_ffn[:K])
    assert row_rel_err(y_ns[:K].float().cpu().numpy().astype(np.float64), ref["y_perm"]) <= TOL[cfg.dtype]
    # oracle hidden rows, expert by expert in grouped order
    h_ref = np.zeros((K, cfg.F))
    for e in range(cfg.n_shared + cfg.N):  # groups = expert weight slots
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            toks = perm[r0:r1] // cfg.k
            sl = lambda n: None if inp.get(n) is None else inp[n][e]  # noqa: E731
            h_ref[r0:r1] = oracle.expert_hidden(inp["x"][toks], cfg.act, sl("w1"), sl("b1"), sl("w3"))
    hg = h[:K].float().cpu().numpy().astype(np.float64)
    assert row_rel_err(hg, h_ref) <= TOL[cfg.dtype]
    # fc2 alone, fed the oracle's H rounded to the layer dtype
    h_in = torch.zeros(A, cfg.F, dtype=shape.torch_dtype)
    h_in[:K] = torch.from_numpy(h_ref).to(shape.torch_dtype)
    y2 = torch.empty_like(y_ud)
    api.expert_down(shape, h_in.to(gpu), buf.offsets, g["w2"], g["b2"], y2, buf.ws)
    torch.cuda.synchronize()
    y2_ref = np.zeros((K, cfg.D))
    h_in64 = h_in[:K].double().numpy()
    for e in range(cfg.n_shared + cfg.N):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            y2_ref[r0:r1] = oracle.expert_output(h_in64[r0:r1], inp["w2"][e],
                                                 None if inp.get("b2") is None else inp["b2"][e])
    assert row_rel_err(y2[:K].float().cpu().numpy().astype(np.float64), y2_ref) <= TOL[cfg.dtype]


def _split_plan(cfg, rows, G, up):
    """Tiles and K chunks per left-over tile of one grouped-GEMM launch, by the
    library's tile rules (for reporting which split a case exercises)."""
    T, k, N = cfg.T, cfg.k, cfg.N
    cap = capacity_of(cfg)
    cap = -1 if cap is None else cap
    expect = -(-T * k // N)
    if cap >= 0:
        expect = min(expect, cap)
    max_rows = T if (cfg.n_shared or cap < 0) else min(cap, T)
    if expect >= 192:
        bm, bn = 256, 256
    elif expect >= 48:
        bm, bn = (128, 256) if (up or max_rows > 128) else (128, 384)
    else:
        bm, bn = 32, 256
    n_out, K = (cfg.F, cfg.D) if up else (cfg.D, cfg.F)
    bn_out = bn // 2 if (up and cfg.act == "swiglu") else bn
    ncol = -(-n_out // bn_out)
    est = (N + cfg.n_shared) * -(-expect // bm) * ncol
    total = sum(-(-int(r) // bm) * ncol for r in rows)
    R = total % G
    S = 1
    allow = bm >= 64 and est < 6 * G and not (max_rows <= bm and est % G == 0)
    if allow and R > 0:
        S = max(1, min(G // R, K // 64, 8))
    return {"tile": f"{bm}x{bn}", "tiles": total, "R": R, "S": S}


SPLIT_CASES = {
    # mid-size groups capped at 128 rows: 128x256 up, 128x384 down (ragged
    # 512 = 384 + 128 output columns, with biases)
    "gelu_bias_S2": scaled_config(get_config("c2", cf=1.0), T=4096, D=512, F=1024, N=64, k=2, act="gelu",
                                  expert_bias=True, residual=False, name="split_gelu_bias_s2"),
    "gelu_bias_S8": scaled_config(get_config("c2", cf=1.0), T=1024, D=512, F=1024, N=16, k=2, act="gelu",
                                  expert_bias=True, residual=False, name="split_gelu_bias_s8"),
    "swiglu_S8": scaled_config(get_config("c2", cf=1.0), T=1024, D=512, F=1024, N=16, k=2, act="swiglu",
                               residual=False, name="split_swiglu_s8"),
    # large groups: 256x256 tiles, few of them (the up projection on the
    # tile whose two waves per SIMD hold 3 and 5 of its 8 token blocks)
    "relu_256": scaled_config(get_config("c2", cf=None), T=1024, D=512, F=1024, N=8, k=2, act="relu",
                              expert_bias=True, residual=False, name="split_relu_256"),
    "swiglu_256": scaled_config(get_config("c2", cf=None), T=1024, D=512, F=1024, N=8, k=2, act="swiglu",
                                residual=False, name="split_swiglu_256"),
}


@pytest.mark.parametrize("key", sorted(SPLIT_CASES))
def test_split_last_round(gpu, key):
    """Layers whose last round of tiles is cut along K into 2..8 chunks (a
    few tiles on a full grid): the expert stage with the workspace (split,
    finished by the second launch) and without (never split) both match the
    oracle; the whole layer twice gives the same bits."""
    cfg = SPLIT_CASES[key]
    inp = generate(cfg)
    ref = oracle_layer(cfg, inp)
    off = ref["offsets"]
    rows = off[1:] - off[:-1]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    G = (cus + 7) // 8 * 8
    plans = [_split_plan(cfg, rows, G, up) for up in (True, False)]
    _say(f"split {key}: T={cfg.T} D={cfg.D} F={cfg.F} N={cfg.N} k={cfg.k} {cfg.act} G={G} up={plans[0]} "
         f"down={plans[1]}")
    if G == 256:  # the cases are sized for a 256-CU part
        assert max(p["S"] for p in plans) >= 2
        if key.endswith("_256"):
            assert plans[0]["S"] >= 2  # the up projection's tile splits too
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg)
    buf = api.MoeBuffers(shape)
    # given the workspace, the router makes moe_forward's choice of kernels
    api.route(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, ws=buf.ws)
    api.dispatch(shape, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.slot, buf.n_dropped)
    A = shape.group_rows
    K = int(off[-1])
    ys = {}
    for mode, ws in (("split", buf.ws), ("plain", None)):
        h = torch.empty(A, cfg.F, dtype=shape.torch_dtype, device=gpu)
        y = torch.empty(A, cfg.D, dtype=shape.torch_dtype, device=gpu)
        api.expert_up(shape, g["x"], buf.perm, buf.offsets, g["w1"], g["b1"], g["w3"], h, ws)
        api.expert_down(shape, h, buf.offsets, g["w2"], g["b2"], y, ws)
        torch.cuda.synchronize()
        ys[mode] = y[:K].float().cpu().numpy().astype(np.float64)
        err = row_rel_err(ys[mode], ref["y_perm"])
        _say(f"  {mode}: y_perm row-rel err {err:.3e}")
        assert err <= TOL[cfg.dtype]
    check_routing(buf, ref, cfg)
    buf.forward(g["x"], g)
    torch.cuda.synchronize()
    out1 = buf.out.clone()
    check_outputs(out1.float().cpu().numpy().astype(np.float64), ref, cfg, inp["x"].double().numpy())
    buf.forward(g["x"], g)
    torch.cuda.synchronize()
    assert torch.equal(out1, buf.out)


@pytest.mark.parametrize("T", [256, 512, 1024])
def test_forward_fp32_tile_heights(gpu, T):
    """The tiny fp32 layer at sizes whose up projection takes 16-, 32- and
    64-row tiles (on a 256-CU part: the tallest tile whose expected count
    fills half of the 4-per-CU grid), against the oracle."""
    cfg = get_config("c1") if T == 1024 else scaled_config(get_config("c1"), T=T, name=f"c1_T{T}")
    inp = generate(cfg)
    ref = oracle_layer(cfg, inp)
    _say(f"fp32 tiles T={T}")
    g = to_gpu(inp)
    buf = run_forward(cfg, g)
    check_routing(buf, ref, cfg)
    check_outputs(buf.out.float().cpu().numpy().astype(np.float64), ref, cfg, inp["x"].double().numpy())


@pytest.mark.parametrize("key,T", [("c3", 1500), ("c5", None), ("c1", None)])
def test_forward_choice_priority(gpu, key, T):
    """Whole layer with MOE_SLOT_MAJOR and a capacity that drops: routing
    bit-exact and outputs within tolerance of the oracle's choice order."""
    base = get_config(key, cf=1.0)
    cfg = base if T is None else scaled_config(base, T=T)
    _say(f"forward choice priority {cfg.name}: T={cfg.T} k={cfg.k} cf={cfg.cf}")
    inp = generate(cfg)
    ref = oracle_layer(cfg, inp, priority="choice")
    assert ref["n_dropped"] > 0
    g = to_gpu(inp)
    buf = run_forward(cfg, g, slot_major=True)
    check_routing(buf, ref, cfg)
    check_outputs(buf.out.float().cpu().numpy().astype(np.float64), ref, cfg, inp["x"].double().numpy())


@pytest.mark.parametrize("T,N,k,C", [
    (1, 1, 1, 0), (1, 4, 4, 1), (777, 8, 2, 150), (777, 8, 2, 400), (2000, 128, 1, 15), (2000, 128, 1, 0),
    (5000, 64, 6, 700), (16384, 128, 1, 192),
])
def test_dispatch_padded(gpu, T, N, k, C):
    rng = np.random.default_rng(T + 3 * N + k)
    _dispatch_case(gpu, _rand_idx(rng, T, N, k), N, C, padded=True)


@pytest.mark.parametrize("key,T,cf", [("c2", 2048, 1.5), ("c3", 1500, 1.0), ("c6", 1024, 1.0),
                                      ("c1", None, 2.0),
                                      # capacity 64: 128x384 down tiles over padded groups
                                      ("c2", 8192, 1.0)])
def test_forward_padded_layout(gpu, key, T, cf):
    """Whole layer in the static capacity layout (MOE_PADDED): routing and
    row layout bit-exact against the oracle's padded dispatch, outputs within
    tolerance, and equal to the compact layout's outputs."""
    base = get_config(key, cf=cf)
    cfg = base if T is None else scaled_config(base, T=T)
    _say(f"forward padded {cfg.name}: T={cfg.T} k={cfg.k} cf={cfg.cf} shared={cfg.n_shared}")
    inp = generate(cfg)
    ref = oracle_layer(cfg, inp, layout="padded")
    g = to_gpu(inp)
    buf = run_forward(cfg, g, padded=True)
    check_routing(buf, ref, cfg)
    y = buf.out.float().cpu().numpy().astype(np.float64)
    check_outputs(y, ref, cfg, inp["x"].double().numpy())
    compact = run_forward(cfg, g)
    y_c = compact.out.float().cpu().numpy().astype(np.float64)
    assert row_rel_err(y, y_c) <= TOL[cfg.dtype]


# ------------------------------------------------ overflow rerouting
FALLBACK_R = {"c1": 3, "c2": 2, "c3": 2, "c4": 2, "c5": 2, "c6": 2}


@pytest.mark.parametrize("key", sorted(CONFIGS))
def test_route_fallback_full_size(gpu, key):
    """moe_route_fallback: the k choices equal moe_route's (gates up to the
    rounding of tokens that the wider near-tie test re-ranks in fp64), the R
    fallback experts equal the oracle's ranks k .. k+R-1 exactly, their gates
    are within the gate tolerance (scaled like the gates with renorm)."""
    cfg = CONFIGS[key]
    R = FALLBACK_R[key]
    _say(f"route fallback {cfg.name} R={R}")
    inp = generate(cfg, parts=("x", "router"))
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg)
    i32 = dict(dtype=torch.int32, device=gpu)
    f32 = dict(dtype=torch.float32, device=gpu)
    idx, gate = torch.empty(cfg.T, cfg.k, **i32), torch.empty(cfg.T, cfg.k, **f32)
    idx2, gate2 = torch.empty_like(idx), torch.empty_like(gate)
    fb_idx, fb_gate = torch.empty(cfg.T, R, **i32), torch.empty(cfg.T, R, **f32)
    api.route_fallback(shape, g["x"], g["w_router"], g["b_router"], idx, gate, R, fb_idx, fb_gate)
    api.route(shape, g["x"], g["w_router"], g["b_router"], idx2, gate2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert (gate - gate2).abs().max().item() <= GATE_ATOL[cfg.dtype]
    r = oracle.route(inp["x"], inp["w_router"], inp["b_router"], cfg.k, cfg.renorm)
    assert np.abs(gate.cpu().numpy() - r["gate"]).max() <= GATE_ATOL[cfg.dtype]
    want_idx, want_gate = oracle.fallback_choices(r["logits"], r["probs"], cfg.k, R, cfg.renorm)
    assert np.array_equal(fb_idx.cpu().numpy(), want_idx)
    assert np.abs(fb_gate.cpu().numpy() - want_gate).max() <= GATE_ATOL[cfg.dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_fallback_hand_example(gpu, dtype, renorm):
    """moe_route_fallback against the hand-derived fixture (integer logits
    with exact ties): the fallbacks are ranks k .. k+R-1 of the router order,
    and their gates follow the closed forms exp(l_f) / sum over all experts
    of exp(l), or over the k chosen experts with renorm.  D is padded with
    zeros to the kernels' multiple, which leaves every logit unchanged."""
    import json
    import math
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "fallback_tiny.json")) as f:
        gold = json.load(f)
    x0 = torch.tensor(gold["x"], dtype=torch.float32)
    w0 = torch.tensor(gold["w_router"], dtype=torch.float32)
    T, N, k = x0.shape[0], w0.shape[0], gold["k"]
    D = 64
    x = torch.zeros(T, D)
    w = torch.zeros(N, D)
    x[:, :x0.shape[1]] = x0
    w[:, :w0.shape[1]] = w0
    dt = "bf16" if dtype == torch.bfloat16 else "fp32"
    shape = api.MoeShape(T=T, D=D, F=64, N=N, k=k, dtype=dt, act="relu", renorm=renorm)
    i32 = dict(dtype=torch.int32, device=gpu)
    f32 = dict(dtype=torch.float32, device=gpu)
    for R, key in ((2, "expected_fallback_R2"), (3, "expected_fallback_R3")):
        _say(f"route fallback hand example {dt} renorm={renorm} R={R}")
        idx, gate = torch.empty(T, k, **i32), torch.empty(T, k, **f32)
        fb_idx, fb_gate = torch.empty(T, R, **i32), torch.empty(T, R, **f32)
        api.route_fallback(shape, x.to(dtype).to(gpu), w.to(dtype).to(gpu), None, idx, gate, R, fb_idx, fb_gate)
        torch.cuda.synchronize()
        assert idx.cpu().tolist() == gold["expected_topk"]
        assert fb_idx.cpu().tolist() == gold[key]
        lg = gold["expected_logits"]
        for t in range(T):
            over = gold["expected_topk"][t] if renorm else range(N)
            den = sum(math.exp(lg[t][c]) for c in over)
            want = [math.exp(lg[t][e]) / den for e in gold[key][t]]
            assert np.abs(fb_gate[t].cpu().numpy() - np.array(want)).max() <= GATE_ATOL["fp32"], (R, t)


def _reroute_case(gpu, T, N, k, C, R, seed, priority="token", n_shared=0, skew=None):
    rng = np.random.default_rng(seed)
    order = np.stack([rng.choice(N, size=k + R, replace=False, p=skew) for _ in range(T)])
    idx_np, fb_np = order[:, :k], order[:, k:]
    gate_np = rng.random((T, k)).astype(np.float32)
    fbg_np = rng.random((T, R)).astype(np.float32)
    shape = api.MoeShape(T=T, D=64, F=64, N=N, k=k, capacity=C, act="relu",
                         slot_major=(priority == "choice"), n_shared=n_shared)
    i32 = dict(dtype=torch.int32, device=gpu)
    idx = torch.from_numpy(idx_np.astype(np.int32)).to(gpu)
    gate = torch.from_numpy(gate_np).to(gpu)
    fb_idx = torch.from_numpy(fb_np.astype(np.int32)).to(gpu)
    fb_gate = torch.from_numpy(fbg_np).to(gpu)
    counts = torch.full((N,), -7, **i32)
    offsets = torch.full((n_shared + N + 1,), -7, **i32)
    perm = torch.full((shape.group_rows,), -7, **i32)
    slot = torch.full((T * k,), -7, **i32)
    nd = torch.full((1,), -7, **i32)
    api.dispatch_reroute(shape, R, fb_idx, fb_gate, idx, gate, counts, offsets, perm, slot, nd)
    torch.cuda.synchronize()
    d = oracle.dispatch(idx_np, N, C, priority)
    ref = oracle.reroute(d, idx_np, gate_np.astype(np.float64), fb_np, fbg_np.astype(np.float64), N, C)
    idx_ref, gate_ref = ref.pop("idx"), ref.pop("gate")
    ref = oracle.with_shared(ref, T, k, n_shared)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    K = int(ref["offsets"][-1])
    p = perm.cpu().numpy()[:K]
    bad = np.nonzero(p != ref["perm"])[0]
    if bad.size:
        _say(f"{bad.size} perm rows differ, first {bad[:8].tolist()}: gpu {p[bad[:8]].tolist()} "
             f"oracle {ref['perm'][bad[:8]].tolist()}; rerouted {ref['n_rerouted']}")
    assert bad.size == 0
    assert np.array_equal(slot.cpu().numpy(), ref["slot"])
    assert int(nd.item()) == ref["n_dropped"]
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.array_equal(gate.cpu().numpy(), gate_ref.astype(np.float32))
    return ref


@pytest.mark.parametrize("T,N,k,C,R", [
    (777, 8, 2, 150, 2), (2000, 128, 1, 15, 3), (3001, 16, 2, 1, 4), (5000, 64, 6, 50, 2),
    (16384, 128, 1, 128, 2), (40000, 256, 2, 300, 2), (2000, 32, 2, 0, 2), (1, 4, 1, 0, 3), (300, 8, 1, 1000, 2),
])
def test_dispatch_reroute(gpu, T, N, k, C, R):
    _reroute_case(gpu, T, N, k, C, R, seed=T + N + k + R)


def test_dispatch_reroute_skewed_choice_and_shared(gpu):
    """Skewed loads (many drops, few experts with room), (choice, token)
    priority for the cut, and shared experts in front of the routed rows."""
    N = 16
    zipf = np.array([1.0 / (e + 1) ** 1.2 for e in range(N)])
    zipf /= zipf.sum()
    ref = _reroute_case(gpu, 4000, N, 2, 300, 3, seed=11, skew=zipf)
    assert ref["n_rerouted"] > 0 and ref["n_dropped"] > 0
    _reroute_case(gpu, 4000, N, 2, 300, 3, seed=12, priority="choice", skew=zipf)
    _reroute_case(gpu, 3000, N, 2, 250, 2, seed=13, n_shared=2, skew=zipf)


@pytest.mark.parametrize("key,T,cf,R", [("c2", 2048, 1.0, 2), ("c3", 1500, 1.0, 2), ("c1", None, 1.0, 3),
                                        ("c6", 1024, 1.0, 2)])
def test_forward_reroute(gpu, key, T, cf, R):
    """Whole layer with rerouting through the stage entry points: routing
    (rewritten idx and gates, rows) exact against the oracle's rerouted
    layer, outputs within tolerance."""
    base = get_config(key, cf=cf)
    cfg = base if T is None else scaled_config(base, T=T)
    _say(f"forward reroute {cfg.name}: T={cfg.T} k={cfg.k} cf={cfg.cf} R={R}")
    inp = generate(cfg)
    C = capacity_of(cfg)
    ref = oracle.moe_forward(inp["x"], inp, k=cfg.k, act=cfg.act, renorm=cfg.renorm, capacity_slots=C,
                             residual=cfg.residual, n_shared=cfg.n_shared, n_fallback=R)
    assert ref["n_rerouted"] > 0
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg)
    buf = api.MoeBuffers(shape)
    i32 = dict(dtype=torch.int32, device=gpu)
    fb_idx = torch.empty(cfg.T, R, **i32)
    fb_gate = torch.empty(cfg.T, R, dtype=torch.float32, device=gpu)
    h = torch.empty(shape.group_rows, cfg.F, dtype=shape.torch_dtype, device=gpu)
    y_perm = torch.empty(shape.group_rows, cfg.D, dtype=shape.torch_dtype, device=gpu)
    api.route_fallback(shape, g["x"], g["w_router"], g["b_router"], buf.topk_idx, buf.topk_gate, R, fb_idx, fb_gate)
    api.dispatch_reroute(shape, R, fb_idx, fb_gate, buf.topk_idx, buf.topk_gate, buf.counts, buf.offsets,
                         buf.perm, buf.slot, buf.n_dropped)
    api.expert_up(shape, g["x"], buf.perm, buf.offsets, g["w1"], g.get("b1"), g.get("w3"), h, buf.ws)
    api.expert_down(shape, h, buf.offsets, g["w2"], g.get("b2"), y_perm, buf.ws)
    api.combine(shape, y_perm, buf.slot, buf.topk_gate, g["x"], buf.out)
    torch.cuda.synchronize()
    check_routing(buf, ref, cfg)
    check_outputs(buf.out.float().cpu().numpy().astype(np.float64), ref, cfg, inp["x"].double().numpy())


# ------------------------------------------ full-size layers, sampled rows
FULL = ["c2", "c2cf15", "c3", "c4", "c5", "c6"]


def _full_cfg(key):
    return get_config("c2", cf=1.5) if key == "c2cf15" else get_config(key)


@pytest.mark.slow
@pytest.mark.parametrize("key", FULL)
def test_forward_full_size(gpu, key):
    cfg = _full_cfg(key)
    _say(f"forward full {cfg.name} cf={cfg.cf}")
    inp = generate(cfg)
    g = to_gpu(inp)
    buf = run_forward(cfg, g)
    rng = np.random.default_rng(123)
    T = cfg.T
    # The sample covers every expert's rows: for each expert with kept rows
    # (from the oracle's own routing), the tokens of its first, last and one
    # random kept row, so that every expert's first and last row tiles get an
    # output check; then the first and last tokens and random ones.
    r = oracle.route(inp["x"], inp["w_router"], inp["b_router"], cfg.k, cfg.renorm)
    d = oracle.dispatch(r["idx"], cfg.N, capacity_of(cfg))
    off, perm = d["offsets"], d["perm"]
    per_expert = []
    for e in range(cfg.N):
        if off[e + 1] > off[e]:
            rows = [off[e], off[e + 1] - 1, rng.integers(off[e], off[e + 1])]
            per_expert += [int(perm[q]) // cfg.k for q in rows]
    sample = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T), np.array(per_expert, dtype=np.int64),
                                       rng.choice(T, size=min(T, 112), replace=False)]))
    covered = {int(e) for t in sample for j, e in enumerate(r["idx"][t]) if d["slot"][t * cfg.k + j] >= 0}
    used = {e for e in range(cfg.N) if off[e + 1] > off[e]}
    assert covered == used, f"experts without a sampled row: {sorted(used - covered)[:10]}"
    ref = oracle_layer(cfg, inp, tokens=sample)
    check_routing(buf, ref, cfg)
    y = buf.out.float().cpu().numpy().astype(np.float64)[sample]
    err = check_outputs(y, ref, cfg, inp["x"].double().numpy()[sample], tokens=sample)
    _say(f"  row-rel err {err:.3e} over {sample.size} sampled tokens covering {len(used)} experts, "
         f"dropped {ref['n_dropped']}")


@pytest.mark.slow
def test_forward_large_batch(gpu):
    """The Switch-shaped layer at 8x its batch (131072 tokens, 128 experts,
    capacity 1024): routing, counts, offsets, perm, slot and drops exact over
    all tokens; outputs on sampled tokens."""
    cfg = scaled_config(get_config("c2"), T=131072)
    _say(f"forward large {cfg.name}: T={cfg.T} cf={cfg.cf}")
    inp = generate(cfg)
    g = to_gpu(inp)
    buf = run_forward(cfg, g)
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([np.arange(4), np.arange(cfg.T - 4, cfg.T),
                                       rng.choice(cfg.T, size=60, replace=False)]))
    ref = oracle_layer(cfg, inp, tokens=sample)
    check_routing(buf, ref, cfg)
    y = buf.out.float().cpu().numpy().astype(np.float64)[sample]
    err = check_outputs(y, ref, cfg, inp["x"].double().numpy()[sample], tokens=sample)
    _say(f"  row-rel err {err:.3e}, dropped {ref['n_dropped']} of {cfg.T}")


# ------------------------------------------ HIP-graph capture of the layer
@pytest.mark.parametrize("key", ["c2", "c5", "c5:fused", "c3dec:fused", "split:gelu_bias_S8", "split:swiglu_S8",
                                 "split:relu_256"])
def test_graph_replay_matches_eager(gpu, key, scaled_cases):
    """moe_forward captured into a HIP graph: every replay, with eager work
    and synchronisations in between, equals the eager result bit for bit.
    The split cases replay layers whose last round of tiles is cut along K
    (partial sums and the tile header in the workspace, a finishing
    launch); the fused cases the fused decode kernel and its shard-summing
    combine."""
    fused = key.endswith(":fused")
    if key.startswith("split:"):
        cfg = SPLIT_CASES[key.split(":", 1)[1]]
        inp = generate(cfg)
    else:
        cfg, inp, _ = _scaled(key.partition(":")[0], scaled_cases)
    _say(f"graph replay {key}: T={cfg.T} D={cfg.D} F={cfg.F} N={cfg.N} k={cfg.k}")
    g = to_gpu(inp)
    shape = api.MoeShape.from_config(cfg, fused_decode=fused)
    eager = api.MoeBuffers(shape)
    eager.forward(g["x"], g)
    torch.cuda.synchronize()
    want = eager.out.clone()
    want_slot = eager.slot.clone()
    cap = api.MoeBuffers(shape)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            cap.forward(g["x"], g, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        cap.out.fill_(0)
        cap.slot.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cap.out, want), rep
        assert torch.equal(cap.slot, want_slot), rep
        eager.forward(g["x"], g)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(eager.out, want)


# ------------------------------------------------ every assignment dropped
@pytest.mark.parametrize("key", ["c2", "c6cf"])
def test_forward_capacity_zero(gpu, key):
    """Capacity 0 drops every routed assignment: the grouped GEMMs see only
    empty routed groups (and the shared groups, if any), and the output is
    the residual plus the shared experts, against the oracle."""
    base = SCALED[key]
    cfg = scaled_config(base, cf=0.0, name=base.name + "_cap0")
    inp = generate(cfg)
    ref = oracle_layer(cfg, inp)
    _say(f"capacity 0 {key}: T={cfg.T} N={cfg.N} k={cfg.k} shared={cfg.n_shared}")
    g = to_gpu(inp)
    buf = run_forward(cfg, g)
    assert int(buf.n_dropped.cpu()) == cfg.T * cfg.k
    check_routing(buf, ref, cfg)
    check_outputs(buf.out.float().cpu().numpy().astype(np.float64), ref, cfg, inp["x"].double().numpy())


# ------------------------------------------------------ one or a few tokens
@pytest.mark.parametrize("key,T,fused", [("c5", 1, False), ("c5", 3, False), ("c4", 1, False), ("c1", 1, False),
                                         ("c6", 2, False), ("c5", 1, True), ("c5", 3, True)])
def test_forward_few_tokens(gpu, key, T, fused):
    """Single-token and few-token batches (decode steps): one row per used
    expert, every tile almost empty, against the oracle; also through the
    fused decode kernel."""
    cfg = scaled_config(SCALED[key], T=T, name=f"{SCALED[key].name}_T{T}")
    inp = generate(cfg)
    ref = oracle_layer(cfg, inp)
    _say(f"few tokens {key}: T={T} D={cfg.D} F={cfg.F} N={cfg.N} k={cfg.k} fused={fused}")
    g = to_gpu(inp)
    buf = run_forward(cfg, g, fused_decode=fused)
    check_routing(buf, ref, cfg)
    check_outputs(buf.out.float().cpu().numpy().astype(np.float64), ref, cfg, inp["x"].double().numpy())
