"""Pins of the oracle's dispatch (counts, stable grouping, capacity drops)."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.cpu


def test_hand_derived_dispatch_example():
    with open(os.path.join(GOLDEN, "dispatch_tiny.json")) as f:
        g = json.load(f)
    idx = np.array(g["idx"])
    T, k = idx.shape
    for case in g["cases"]:
        C = oracle.capacity(T, k, g["N"], case["cf"])
        assert C == case["capacity"]
        d = oracle.dispatch(idx, g["N"], C)
        assert d["counts"].tolist() == case["counts"]
        assert d["offsets"].tolist() == case["offsets"]
        assert d["perm"].tolist() == case["perm"]
        assert d["slot"].tolist() == case["slot"]
        assert d["n_dropped"] == case["n_dropped"]


def test_capacity_truncates_like_the_notebook():
    # switch-style layer: 16384 tokens, top-1, 128 experts
    assert oracle.capacity(16384, 1, 128, 1.0) == 128
    assert oracle.capacity(16384, 1, 128, 1.5) == 192
    # notebook sizes: 1024 tokens, top-2, 8 experts -> 256 and 384 slots
    assert oracle.capacity(1024, 2, 8, 1.0) == 256
    assert oracle.capacity(1024, 2, 8, 1.5) == 384
    # truncation, not rounding: 10*1/3*1.0 = 3.33 -> 3 ; 10*2/3*1.0 = 6.67 -> 6
    assert oracle.capacity(10, 1, 3, 1.0) == 3
    assert oracle.capacity(10, 2, 3, 1.0) == 6
    assert oracle.capacity(10, 2, 3, None) is None
    assert oracle.capacity(10, 2, 3, 0.0) == 0


def _random_idx(rng, T, N, k):
    return np.stack([rng.permutation(N)[:k] for _ in range(T)])


@pytest.mark.parametrize("seed", range(5))
def test_counts_perm_slot_against_library_routines(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 12))
    k = int(rng.integers(1, N + 1))
    T = int(rng.integers(1, 200))
    idx = _random_idx(rng, T, N, k)
    flat = idx.reshape(-1)
    # skew some tokens onto expert 0 when allowed
    d = oracle.dispatch(idx, N, None)
    assert np.array_equal(d["counts"], np.bincount(flat, minlength=N))
    assert d["counts"].sum() == T * k
    assert np.array_equal(d["perm"], np.argsort(flat, kind="stable"))
    assert np.array_equal(d["slot"][d["perm"]], np.arange(T * k))
    for C in (0, 1, 2, 5, T * k):
        dc = oracle.dispatch(idx, N, C)
        stable = np.argsort(flat, kind="stable")
        kept = []
        for e in range(N):
            kept += [a for a in stable if flat[a] == e][:C]
        assert dc["perm"].tolist() == kept
        assert dc["n_dropped"] == int(np.clip(dc["counts"] - C, 0, None).sum())
        assert np.array_equal(np.diff(dc["offsets"]), np.minimum(dc["counts"], C))


def test_rank_brute_force():
    rng = np.random.default_rng(9)
    T, N, k = 40, 5, 2
    idx = _random_idx(rng, T, N, k)
    flat = idx.reshape(-1)
    for C in (3, 8, 16, None):
        d = oracle.dispatch(idx, N, C)
        for a in range(flat.size):
            rank = int((flat[:a] == flat[a]).sum())
            kept = C is None or rank < C
            if kept:
                assert d["slot"][a] == d["offsets"][flat[a]] + rank
            else:
                assert d["slot"][a] == -1


def test_drop_rate_non_increasing_in_capacity_factor():
    rng = np.random.default_rng(11)
    T, N, k = 512, 8, 2
    # skewed routing
    p = np.array([0.4, 0.2, 0.1, 0.1, 0.08, 0.06, 0.04, 0.02])
    idx = np.stack([rng.choice(N, size=k, replace=False, p=p) for _ in range(T)])
    counts = oracle.expert_counts(idx, N)
    prev = None
    for cf in np.linspace(0.0, 4.0, 41):
        C = oracle.capacity(T, k, N, float(cf))
        d = oracle.dispatch(idx, N, C)
        rate = oracle.drop_rate(counts, C)
        assert rate == pytest.approx(d["n_dropped"] / (T * k), abs=0)
        if prev is not None:
            assert rate <= prev
        prev = rate
    # capacity at least the largest count -> no drops
    d = oracle.dispatch(idx, N, int(counts.max()))
    assert d["n_dropped"] == 0


def test_imbalance_and_aux_loss_closed_forms():
    T, N, k = 64, 8, 2
    # round-robin assignment and uniform gates (the notebook's balanced case)
    idx = (np.arange(T * k) % N).reshape(T, k)
    probs = np.full((T, N), 1.0 / N)
    counts = oracle.expert_counts(idx, N)
    assert oracle.imbalance(counts, T, k, N) == 1.0
    # every expert appears in a fraction 2/8 of tokens: loss = N * sum (2/8)(1/8) = k
    assert oracle.switch_aux_loss(idx, probs, N) == pytest.approx(2.0, abs=1e-15)
    # all tokens on experts 0,1 with all probability there: loss = N * (1*0.5 + 1*0.5) = N
    idx2 = np.tile([0, 1], (T, 1))
    probs2 = np.zeros((T, N))
    probs2[:, :2] = 0.5
    assert oracle.switch_aux_loss(idx2, probs2, N) == pytest.approx(N, abs=1e-12)


# --------------------------------------------- choice-major (GShard) priority
def test_choice_priority_hand_example():
    # 4 tokens, top-2, 3 experts, capacity 2.  Expert 0 receives (t0,j0),
    # (t1,j1), (t2,j0), (t3,j1): token order keeps t0,t1; choice order keeps
    # the first choices t0,t2.
    idx = np.array([[0, 1], [2, 0], [0, 2], [1, 0]])
    d = oracle.dispatch(idx, 3, 2, priority="choice")
    assert d["counts"].tolist() == [4, 2, 2]
    assert d["offsets"].tolist() == [0, 2, 4, 6]
    # expert 0: a=0 (t0,j0), a=4 (t2,j0); expert 1: a=6 (t3,j0), a=1 (t0,j1);
    # expert 2: a=2 (t1,j0), a=5 (t2,j1)
    assert d["perm"].tolist() == [0, 4, 6, 1, 2, 5]
    assert d["slot"].tolist() == [0, 3, 4, -1, 1, 5, 2, -1]
    assert d["n_dropped"] == 2
    dt = oracle.dispatch(idx, 3, 2, priority="token")
    assert dt["perm"].tolist()[:2] == [0, 3]


@pytest.mark.parametrize("seed", range(4))
def test_choice_priority_against_lexsort_and_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(2, 10))
    k = int(rng.integers(1, min(N, 4) + 1))
    T = int(rng.integers(1, 120))
    idx = _random_idx(rng, T, N, k)
    C = int(rng.integers(0, T))
    d = oracle.dispatch(idx, N, C, priority="choice")
    flat = idx.reshape(-1)
    a = np.arange(flat.size)
    # library: sort by (expert, choice, token); keep each expert's first C
    order = np.lexsort((a // k, a % k, flat))
    want = []
    for e in range(N):
        mine = [x for x in order if flat[x] == e]
        want += mine[:C]
    assert d["perm"].tolist() == want
    # brute force rank of every assignment
    for x in range(flat.size):
        t, j = divmod(x, k)
        rank = sum(1 for y in range(flat.size) if flat[y] == flat[x] and (y % k, y // k) < (j, t))
        assert (d["slot"][x] >= 0) == (rank < C)
    # k = 1: choice order is token order
    i1 = idx[:, :1]
    d1c, d1t = oracle.dispatch(i1, N, C, "choice"), oracle.dispatch(i1, N, C, "token")
    for key in ("counts", "offsets", "perm", "slot"):
        assert np.array_equal(d1c[key], d1t[key])


def test_choice_priority_keeps_first_choices_first():
    # GShard guarantee: an expert never keeps a second choice while it drops a
    # first choice; under token order it can
    rng = np.random.default_rng(7)
    T, N, k = 400, 6, 2
    p = np.array([0.5, 0.2, 0.1, 0.1, 0.05, 0.05])
    idx = np.stack([rng.choice(N, size=k, replace=False, p=p) for _ in range(T)])
    C = oracle.capacity(T, k, N, 1.0)
    d = oracle.dispatch(idx, N, C, priority="choice")
    flat = idx.reshape(-1)
    for e in range(N):
        mine = np.nonzero(flat == e)[0]
        j_kept = mine[d["slot"][mine] >= 0] % k
        j_drop = mine[d["slot"][mine] < 0] % k
        if j_drop.size and j_kept.size:
            assert j_drop.min() >= j_kept.max()
    # more first choices survive than under token order
    dt = oracle.dispatch(idx, N, C, priority="token")
    first = np.arange(T) * k
    assert (d["slot"][first] >= 0).sum() > (dt["slot"][first] >= 0).sum()


def test_choice_priority_layer_matches_brute_force():
    from workloads import generate, get_config, scaled_config
    cfg = scaled_config(get_config("c1"), T=48, D=32, F=64, N=4, k=2)
    inp = generate(cfg)
    C = oracle.capacity(cfg.T, cfg.k, cfg.N, 0.75)
    ref = oracle.moe_forward(inp["x"], inp, k=cfg.k, act=cfg.act, capacity_slots=C, priority="choice")
    y_b = oracle.brute_forward(inp["x"], inp, k=cfg.k, act=cfg.act, capacity_slots=C, priority="choice")
    assert np.allclose(ref["y"], y_b, rtol=1e-12, atol=1e-12)
    assert ref["n_dropped"] > 0


# ------------------------------------------------- static padded layout
def test_padded_layout_hand_example_and_invariants():
    # same hand case as the choice test: 4 tokens, top-2, 3 experts, C = 2
    idx = np.array([[0, 1], [2, 0], [0, 2], [1, 0]])
    d = oracle.padded(oracle.dispatch(idx, 3, 2), 3, 2)
    assert d["offsets"].tolist() == [0, 2, 4, 6]
    # token order: expert 0 keeps a=0,3; expert 1 a=1,6; expert 2 a=2,5
    assert d["perm"].tolist() == [0, 3, 1, 6, 2, 5]
    rng = np.random.default_rng(5)
    T, N, k = 300, 7, 2
    idx = _random_idx(rng, T, N, k)
    for C in (0, 10, 90, 200):
        dc = oracle.dispatch(idx, N, C)
        dp = oracle.padded(dc, N, C)
        assert dp["offsets"].tolist() == [e * C for e in range(N + 1)]
        assert np.array_equal(dp["counts"], dc["counts"]) and dp["n_dropped"] == dc["n_dropped"]
        kept = np.minimum(dc["counts"], C)
        for e in range(N):
            rows = dp["perm"][e * C:(e + 1) * C]
            assert np.array_equal(rows[:kept[e]], dc["perm"][dc["offsets"][e]:dc["offsets"][e + 1]])
            assert (rows[kept[e]:] == -1).all()
        # every kept assignment's slot points at its own row
        k_a = np.nonzero(dp["slot"] >= 0)[0]
        assert np.array_equal(dp["perm"][dp["slot"][k_a]], k_a)
        assert np.array_equal(dp["slot"] >= 0, dc["slot"] >= 0)


def test_padded_layout_layer_equals_compact():
    from workloads import generate, get_config, scaled_config
    cfg = scaled_config(get_config("c1"), T=64, D=32, F=48, N=4, k=2)
    inp = generate(cfg)
    for cf in (0.5, 1.0, 2.0):
        C = oracle.capacity(cfg.T, cfg.k, cfg.N, cf)
        a = oracle.moe_forward(inp["x"], inp, k=cfg.k, act=cfg.act, capacity_slots=C)
        b = oracle.moe_forward(inp["x"], inp, k=cfg.k, act=cfg.act, capacity_slots=C, layout="padded")
        assert np.allclose(a["y"], b["y"], rtol=1e-14, atol=1e-14)


def test_router_stats_closed_forms_and_invariants():
    """f sums to k and P to 1 on any batch; equal logits give P = 1/N and a
    loss of exactly k; all tokens on one expert with all probability there
    gives a loss of N; the hand case below is worked out on paper."""
    rng = np.random.default_rng(5)
    T, N, k = 50, 6, 2
    logits = rng.standard_normal((T, N))
    probs = oracle.softmax(logits)
    idx = oracle.select_topk(logits, k)
    counts = oracle.expert_counts(idx, N)
    st = oracle.router_stats(idx, probs, counts, N, oracle.capacity(T, k, N, 1.0))
    assert st["frac"].sum() == pytest.approx(k, abs=1e-12)
    assert st["prob_mean"].sum() == pytest.approx(1.0, abs=1e-12)
    assert np.array_equal(st["frac"], counts / T)  # distinct choices: any() == count
    assert st["aux_loss"] == pytest.approx(oracle.switch_aux_loss(idx, probs, N), abs=0)
    # equal logits: P = 1/N, loss = N * sum f / N = k
    flat = np.zeros((T, N))
    st = oracle.router_stats(oracle.select_topk(flat, k), oracle.softmax(flat),
                             oracle.expert_counts(oracle.select_topk(flat, k), N), N, None)
    assert np.allclose(st["prob_mean"], 1.0 / N, atol=1e-15)
    assert st["aux_loss"] == pytest.approx(k, abs=1e-12)
    # ties go to the lowest indices: every token on experts 0..k-1
    assert st["imbalance"] == T / (T * k / N) and st["drop_rate"] == 0.0
    # hand case: T=4, N=4, k=1, tokens on experts 0, 0, 0, 2; probabilities
    # 0.7 on the chosen expert and 0.1 elsewhere; capacity 2
    idx = np.array([[0], [0], [0], [2]])
    probs = np.full((4, 4), 0.1)
    probs[np.arange(4), idx[:, 0]] = 0.7
    counts = oracle.expert_counts(idx, 4)
    st = oracle.router_stats(idx, probs, counts, 4, 2)
    assert np.allclose(st["frac"], [0.75, 0.0, 0.25, 0.0])
    assert np.allclose(st["prob_mean"], [0.55, 0.1, 0.25, 0.1])
    # 4 * (0.75*0.55 + 0.25*0.25) = 4 * 0.475 = 1.9
    assert st["aux_loss"] == pytest.approx(1.9, abs=1e-12)
    assert st["imbalance"] == 3.0      # 3 / (4*1/4)
    assert st["drop_rate"] == 0.25     # one of four over capacity 2


def _reroute_case(idx, fb, N, C):
    idx = np.asarray(idx)
    fb = np.asarray(fb)
    T, k = idx.shape
    gate = np.full((T, k), 0.5)
    fb_gate = np.tile(np.arange(1, fb.shape[1] + 1) * 0.01, (T, 1))
    d = oracle.dispatch(idx, N, C)
    return oracle.reroute(d, idx, gate, fb, fb_gate, N, C)


def test_reroute_hand_examples():
    """Worked on paper.  (1) Switch-like k=1, C=1: tokens 1 and 2 overflow
    expert 0; token 1's fallbacks (1, 2) find expert 1 full and, one level
    later, expert 2 already taken at level 0 by token 2.  (2) Level order
    beats token order: token 1 fails at level 0 and its level-1 expert went to
    token 3 at level 0.  (3) k=2: both of token 1's choices overflow and come
    back on two levels, lowest j first."""
    r = _reroute_case([[0], [0], [0], [1]], [[1, 2], [1, 2], [2, 1], [0, 2]], N=3, C=1)
    assert r["offsets"].tolist() == [0, 1, 2, 3]
    assert r["perm"].tolist() == [0, 3, 2]
    assert r["slot"].tolist() == [0, -1, 2, 1]
    assert r["idx"].ravel().tolist() == [0, 0, 2, 1]
    assert r["gate"].ravel().tolist() == [0.5, 0.5, 0.01, 0.5]
    assert (r["n_dropped"], r["n_rerouted"]) == (1, 1)
    assert r["counts"].tolist() == [3, 1, 0]  # routed counts before the cut
    r = _reroute_case([[0], [0], [1], [0]], [[1, 2], [1, 2], [0, 2], [2, 1]], N=3, C=1)
    assert r["perm"].tolist() == [0, 2, 3] and r["slot"].tolist() == [0, -1, 1, 2]
    assert (r["n_dropped"], r["n_rerouted"]) == (1, 1)
    r = _reroute_case([[0, 1], [0, 1]], [[2, 3], [2, 3]], N=4, C=1)
    assert r["offsets"].tolist() == [0, 1, 2, 3, 4]
    assert r["perm"].tolist() == [0, 1, 2, 3]
    assert r["idx"].tolist() == [[0, 1], [2, 3]]
    assert r["gate"].tolist() == [[0.5, 0.5], [0.01, 0.02]]
    assert r["n_dropped"] == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_reroute_invariants(seed):
    """No level or no capacity changes nothing; no expert exceeds C; a
    rerouted choice is one of the token's fallbacks and never repeats one of
    its experts; rows + drops = T*k; slot and perm agree; expert rows hold
    their kept assignments first, in dispatch order."""
    rng = np.random.default_rng(seed)
    T, N, k, R = 300, 8, 2, 3
    logits = rng.standard_normal((T, N)) + np.linspace(1.5, 0, N)  # skewed
    probs = oracle.softmax(logits)
    idx = oracle.select_topk(logits, k)
    gate = oracle.gate_values(probs, idx, False)
    fb_idx, fb_gate = oracle.fallback_choices(logits, probs, k, R, False)
    C = oracle.capacity(T, k, N, 1.0)
    d = oracle.dispatch(idx, N, C)
    for none in (oracle.reroute(d, idx, gate, fb_idx[:, :0], fb_gate[:, :0], N, C),
                 oracle.reroute(oracle.dispatch(idx, N, None), idx, gate, fb_idx, fb_gate, N, None)):
        base = d if none["n_dropped"] else oracle.dispatch(idx, N, None)
        for key in ("offsets", "perm", "slot"):
            assert np.array_equal(none[key], base[key])
        assert np.array_equal(none["idx"], idx) and none["n_rerouted"] == 0
    r = oracle.reroute(d, idx, gate, fb_idx, fb_gate, N, C)
    assert r["n_rerouted"] > 0 and r["n_dropped"] < d["n_dropped"]
    assert r["n_dropped"] + r["perm"].size == T * k
    assert (np.diff(r["offsets"]) <= C).all()
    for t in range(T):
        assert len(set(r["idx"][t])) == k
        for j in range(k):
            if r["idx"][t, j] != idx[t, j]:
                rr = list(fb_idx[t]).index(r["idx"][t, j])
                assert r["gate"][t, j] == fb_gate[t, rr]
                assert d["slot"][t * k + j] < 0 <= r["slot"][t * k + j]
    assert np.array_equal(r["slot"][r["perm"]], np.arange(r["perm"].size))
    for e in range(N):
        kept = d["perm"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.array_equal(r["perm"][r["offsets"][e]:r["offsets"][e] + kept.size], kept)
        rows = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert (r["idx"].reshape(-1)[rows] == e).all()


def test_reroute_layer_matches_dense_gates():
    """The layer with rerouting equals the dense formulation of its final
    routing: y[t] = sum over assignments that end in a row of
    gate[t, j] * MLP_{idx[t, j]}(x[t]), every expert run on every token."""
    from workloads import get_config, generate, scaled_config
    cfg = scaled_config(get_config("c1"), T=96)
    inp = generate(cfg)
    C = oracle.capacity(cfg.T, cfg.k, cfg.N, 1.0)
    out = oracle.moe_forward(inp["x"], inp, k=cfg.k, act=cfg.act, capacity_slots=C, n_fallback=2)
    assert out["n_rerouted"] > 0 and out["n_dropped"] > 0
    X = oracle.f64(inp["x"])
    Yall = np.stack([oracle.expert_mlp(X, cfg.act, w1=inp["w1"][e], b1=inp["b1"][e], w2=inp["w2"][e],
                                       b2=inp["b2"][e]) for e in range(cfg.N)])
    y = np.zeros_like(X)
    for t in range(cfg.T):
        for j in range(cfg.k):
            if out["slot"][t * cfg.k + j] >= 0:
                y[t] += out["gate"][t, j] * Yall[out["idx"][t, j], t]
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-12)


def _golden_fallback():
    with open(os.path.join(GOLDEN, "fallback_tiny.json")) as f:
        return json.load(f)


def _exp_gate(logits_row, e, over):
    """exp(l_e) / sum of exp(l) over the experts in ``over`` (exact-arithmetic
    form of a softmax probability, or of one renormalised over ``over``)."""
    return math.exp(logits_row[e]) / sum(math.exp(logits_row[c]) for c in over)


def test_fallback_choices_hand_example():
    """Ranks k .. k+R-1 of the router order, checked against the hand-derived
    fixture; the renormalised gate divides by the k chosen probabilities
    only (its closed form after the softmax denominator cancels)."""
    g = _golden_fallback()
    x = np.array(g["x"], dtype=np.float64)
    w = np.array(g["w_router"], dtype=np.float64)
    k = g["k"]
    logits = oracle.router_logits(x, w)
    assert np.array_equal(logits, np.array(g["expected_logits"], dtype=np.float64))
    probs = oracle.softmax(logits)
    assert np.array_equal(oracle.select_topk(logits, k), np.array(g["expected_topk"]))
    for R, key in ((2, "expected_fallback_R2"), (3, "expected_fallback_R3")):
        for renorm in (False, True):
            fb_idx, fb_gate = oracle.fallback_choices(logits, probs, k, R, renorm)
            assert np.array_equal(fb_idx, np.array(g[key])), (R, renorm)
            for t in range(x.shape[0]):
                chosen = g["expected_topk"][t]
                over = chosen if renorm else range(w.shape[0])
                want = [_exp_gate(g["expected_logits"][t], e, over) for e in g[key][t]]
                assert np.allclose(fb_gate[t], want, rtol=1e-14, atol=0), (R, renorm, t)
    _, fb_gate = oracle.fallback_choices(logits, probs, k, 2, True)
    assert np.allclose(fb_gate[0], g["renorm_gate_x0_R2"]["value"], rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fallback_choices_against_sorted_with_ties(seed):
    """Small-integer logits with many exact ties and duplicated router rows:
    the fallbacks equal Python's sorted() of (-logit, expert) cut at
    [k, k+R), for every k + R <= N including k + R = N."""
    rng = np.random.default_rng(seed)
    N, D, T = 7, 3, 60
    w = rng.integers(-2, 3, size=(N, D)).astype(np.float64)
    w[4] = w[1]  # duplicated rows force exact ties on every token
    w[6] = w[2]
    x = rng.integers(-2, 3, size=(T, D)).astype(np.float64)
    l = oracle.router_logits(x, w)
    p = oracle.softmax(l)
    n_ties = sum(len(set(row)) < N for row in l.tolist())
    assert n_ties == T
    for k in range(1, N):
        for R in range(1, N - k + 1):
            fb_idx, fb_gate = oracle.fallback_choices(l, p, k, R, renorm=True)
            _, fb_plain = oracle.fallback_choices(l, p, k, R, renorm=False)
            for t in range(T):
                order = sorted(range(N), key=lambda e: (-l[t, e], e))
                assert fb_idx[t].tolist() == order[k:k + R], (k, R, t)
                want = [_exp_gate(l[t], e, order[:k]) for e in order[k:k + R]]
                assert np.allclose(fb_gate[t], want, rtol=1e-12, atol=0), (k, R, t)
                want = [_exp_gate(l[t], e, range(N)) for e in order[k:k + R]]
                assert np.allclose(fb_plain[t], want, rtol=1e-12, atol=0), (k, R, t)


def test_out_of_range_ids_are_neither_counted_nor_kept():
    """An id outside [0, N) names no expert: it is not counted, never gets a
    row and is dropped (the GPU dispatch treats it the same way)."""
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 8, size=(300, 2))
    idx[::7, 0] = -1
    idx[::11, 1] = 8
    flat = idx.reshape(-1)
    inside = flat[(flat >= 0) & (flat < 8)]
    for C in (None, 30):
        d = oracle.dispatch(idx, 8, C)
        assert np.array_equal(d["counts"], np.bincount(inside, minlength=8))
        bad = np.nonzero((flat < 0) | (flat >= 8))[0]
        assert (d["slot"][bad] == -1).all()
        assert not np.isin(bad, d["perm"]).any()
