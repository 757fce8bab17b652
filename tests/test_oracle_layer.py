"""Pins of the oracle's expert MLPs and combine against library routines,
closed forms and a second (dense, brute-force) formulation."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle

pytestmark = pytest.mark.cpu


def _params(rng, N, D, F, act, bias, scale=0.3):
    p = {
        "w_router": rng.standard_normal((N, D)),
        "b_router": None,
        "w1": rng.standard_normal((N, F, D)) * scale,
        "b1": rng.standard_normal((N, F)) * scale if bias else None,
        "w3": rng.standard_normal((N, F, D)) * scale if act == "swiglu" else None,
        "w2": rng.standard_normal((N, D, F)) * scale,
        "b2": rng.standard_normal((N, D)) * scale if bias else None,
    }
    return p


def test_gelu_erf_special_values_and_library():
    z = np.array([0.0, 1.0, -1.0, 3.0, -3.0, 10.0, -10.0])
    g = oracle.gelu_erf(z)
    assert g[0] == 0.0
    # Phi(1) = 0.841344746068543 (standard normal table)
    assert g[1] == pytest.approx(0.841344746068543, rel=1e-14)
    # odd-even identity: gelu(z) - gelu(-z) = z
    assert np.allclose(g[1::2] - g[2::2], z[1::2], atol=1e-15)
    assert g[5] == pytest.approx(10.0, rel=1e-15)
    assert abs(g[6]) < 1e-20
    zz = np.linspace(-6, 6, 1001)
    ref = Fnn.gelu(torch.from_numpy(zz), approximate="none").numpy()
    assert np.allclose(oracle.gelu_erf(zz), ref, rtol=1e-13, atol=1e-15)
    # the tanh approximation differs measurably, so the erf form is pinned
    tanh = Fnn.gelu(torch.from_numpy(zz), approximate="tanh").numpy()
    assert np.abs(oracle.gelu_erf(zz) - tanh).max() > 1e-5


def test_silu_and_relu_library():
    z = np.linspace(-20, 20, 801)
    assert np.allclose(oracle.silu(z), Fnn.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)
    assert np.array_equal(oracle.relu(z), Fnn.relu(torch.from_numpy(z)).numpy())
    assert oracle.silu(np.array([0.0]))[0] == 0.0


@pytest.mark.parametrize("act,bias", [("gelu", True), ("relu", False), ("relu", True), ("swiglu", False)])
def test_single_expert_equals_torch_modules(act, bias):
    """N = 1, k = 1: every gate is exactly 1, so the layer is one expert."""
    rng = np.random.default_rng(7)
    T, D, F = 23, 12, 20
    p = _params(rng, 1, D, F, act, bias)
    x = rng.standard_normal((T, D))
    r = oracle.moe_forward(x, p, k=1, act=act)
    assert np.all(r["gate"] == 1.0)
    xt = torch.from_numpy(x)
    fc1 = torch.nn.Linear(D, F, bias=bias).double()
    fc2 = torch.nn.Linear(F, D, bias=bias).double()
    with torch.no_grad():
        fc1.weight.copy_(torch.from_numpy(p["w1"][0]))
        fc2.weight.copy_(torch.from_numpy(p["w2"][0]))
        if bias:
            fc1.bias.copy_(torch.from_numpy(p["b1"][0]))
            fc2.bias.copy_(torch.from_numpy(p["b2"][0]))
        if act == "gelu":
            ref = fc2(Fnn.gelu(fc1(xt)))
        elif act == "relu":
            ref = fc2(Fnn.relu(fc1(xt)))
        else:
            up = torch.nn.Linear(D, F, bias=False).double()
            up.weight.copy_(torch.from_numpy(p["w3"][0]))
            ref = fc2(Fnn.silu(fc1(xt)) * up(xt))
    assert np.allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_identical_experts_closed_forms(act):
    rng = np.random.default_rng(8)
    T, D, F, N, k = 31, 10, 14, 6, 3
    p = _params(rng, 1, D, F, act, act == "gelu")
    for name in ("w1", "b1", "w3", "w2", "b2"):
        if p[name] is not None:
            p[name] = np.repeat(p[name], N, axis=0)
    p["w_router"] = rng.standard_normal((N, D))
    x = rng.standard_normal((T, D))
    ffn = oracle.expert_mlp(x, act, p["w1"][0], None if p["b1"] is None else p["b1"][0],
                            None if p["w3"] is None else p["w3"][0], p["w2"][0],
                            None if p["b2"] is None else p["b2"][0])
    rn = oracle.moe_forward(x, p, k=k, act=act, renorm=True)
    assert np.allclose(rn["y"], ffn, rtol=1e-12, atol=1e-12)
    r = oracle.moe_forward(x, p, k=k, act=act, renorm=False)
    assert np.allclose(r["y"], r["gate"].sum(1, keepdims=True) * ffn, rtol=1e-12, atol=1e-12)


def test_zero_w2_unique_bias_pins_unpermute():
    """W2 = 0: each expert outputs its own constant b2_e, so the layer output
    is sum_j g[t,j] * b2[idx[t,j]], which exposes any slot/row mix-up."""
    rng = np.random.default_rng(12)
    T, D, F, N, k = 57, 6, 9, 7, 3
    p = _params(rng, N, D, F, "gelu", True)
    p["w2"][:] = 0.0
    p["b2"] = np.arange(N * D, dtype=np.float64).reshape(N, D) + 1.0
    x = rng.standard_normal((T, D))
    for C in (None, 9, 3, 0):
        r = oracle.moe_forward(x, p, k=k, act="gelu", capacity_slots=C)
        want = np.zeros((T, D))
        flat = r["idx"].reshape(-1)
        for a in range(T * k):
            t, j = divmod(a, k)
            rank = int((flat[:a] == flat[a]).sum())
            if C is None or rank < C:
                want[t] += r["gate"][t, j] * p["b2"][flat[a]]
        assert np.allclose(r["y"], want, rtol=1e-14, atol=1e-13)


def test_k_equals_N_is_the_dense_softmax_mixture():
    rng = np.random.default_rng(13)
    T, D, F, N = 19, 8, 11, 4
    p = _params(rng, N, D, F, "relu", True)
    x = rng.standard_normal((T, D))
    r = oracle.moe_forward(x, p, k=N, act="relu")
    probs = r["probs"]
    dense = sum(probs[:, e:e + 1] * oracle.expert_mlp(x, "relu", p["w1"][e], p["b1"][e], None,
                                                      p["w2"][e], p["b2"][e]) for e in range(N))
    assert np.allclose(r["y"], dense, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("act", ["gelu", "relu", "swiglu"])
def test_per_expert_loop_matches_dense_brute_force(seed, act):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 16))
    N = int(rng.integers(1, 6))
    k = int(rng.integers(1, N + 1))
    D, F = 5, 7
    p = _params(rng, N, D, F, act, act != "swiglu")
    if seed % 2:
        p["b_router"] = rng.standard_normal(N)
    x = rng.standard_normal((T, D))
    for C in (None, 0, 1, 2, 4):
        for renorm in (False, True):
            for residual in (False, True):
                a = oracle.moe_forward(x, p, k=k, act=act, renorm=renorm, capacity_slots=C,
                                       residual=residual)["y"]
                b = oracle.brute_forward(x, p, k=k, act=act, renorm=renorm, capacity_slots=C,
                                         residual=residual)
                assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_dropped_tokens_are_exact_zero_or_exact_residual():
    rng = np.random.default_rng(14)
    T, D, F, N, k = 40, 6, 8, 4, 1
    p = _params(rng, N, D, F, "relu", False)
    x = rng.standard_normal((T, D))
    r0 = oracle.moe_forward(x, p, k=k, act="relu", capacity_slots=0, residual=True)
    assert np.array_equal(r0["y"], x)
    r1 = oracle.moe_forward(x, p, k=k, act="relu", capacity_slots=3, residual=False)
    dropped_tokens = np.nonzero(r1["slot"].reshape(T, k).max(1) < 0)[0]
    assert dropped_tokens.size > 0
    assert np.all(r1["y"][dropped_tokens] == 0.0)


def test_sampled_tokens_equal_full_forward():
    rng = np.random.default_rng(15)
    T, D, F, N, k = 64, 8, 12, 5, 2
    p = _params(rng, N, D, F, "swiglu", False)
    x = rng.standard_normal((T, D))
    full = oracle.moe_forward(x, p, k=k, act="swiglu", capacity_slots=20, residual=True)
    toks = [0, 5, 17, 63, 40]
    part = oracle.moe_forward(x, p, k=k, act="swiglu", capacity_slots=20, residual=True, tokens=toks)
    assert np.allclose(part["y"], full["y"][toks], rtol=1e-13, atol=1e-13)


def test_active_parameter_fraction_is_k_over_N():
    """Each token touches exactly k distinct experts, so with no drops the
    executed expert FLOPs are k/N of evaluating every expert on every token."""
    rng = np.random.default_rng(16)
    T, D, F, N, k = 200, 8, 16, 8, 2
    p = _params(rng, N, D, F, "gelu", True)
    x = rng.standard_normal((T, D))
    r = oracle.moe_forward(x, p, k=k, act="gelu")
    assert all(len(set(row)) == k for row in r["idx"].tolist())
    assert r["counts"].sum() == T * k
    executed = sum(2 * 2 * D * F * (r["offsets"][e + 1] - r["offsets"][e]) for e in range(N))
    dense = 2 * 2 * D * F * T * N
    assert executed / dense == pytest.approx(k / N, abs=0)
    assert math.isclose(r["perm"].size / (T * N), k / N)


def test_combine_rows_hand_example_and_consistency():
    # two tokens, k=2: token 0 keeps both choices, token 1 lost choice 1
    y_perm = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    slot = np.array([2, 0, 1, -1])
    gate = np.array([[0.5, 0.25], [0.75, 0.125]])
    out = oracle.combine_rows(y_perm, slot, gate, 2)
    assert out.tolist() == [[0.5 * 100 + 0.25 * 1, 0.5 * 200 + 0.25 * 2], [0.75 * 10, 0.75 * 20]]
    x = np.array([[1.0, 1.0], [2.0, 2.0]])
    assert np.array_equal(oracle.combine_rows(y_perm, slot, gate, 2, x), out + x)
    # equals the per-expert loop on a random layer
    rng = np.random.default_rng(17)
    T, D, F, N, k = 30, 6, 10, 5, 2
    p = _params(rng, N, D, F, "gelu", True)
    xx = rng.standard_normal((T, D))
    r = oracle.moe_forward(xx, p, k=k, act="gelu", capacity_slots=9, residual=True)
    y = oracle.combine_rows(r["y_perm"], r["slot"], r["gate"], k, xx)
    assert np.allclose(y, r["y"], rtol=1e-13, atol=1e-13)


# ------------------------------------------------ shared (always-on) experts
def _shared_params(rng, S, N, D, F, act, bias):
    """Stacks of S shared experts followed by N routed ones; router over N."""
    p = _params(rng, S + N, D, F, act, bias)
    p["w_router"] = rng.standard_normal((N, D))
    return p


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("act", ["gelu", "relu", "swiglu"])
def test_shared_experts_match_dense_brute_force(seed, act):
    rng = np.random.default_rng(300 + seed)
    T = int(rng.integers(1, 16))
    N = int(rng.integers(1, 6))
    S = int(rng.integers(1, 3))
    k = int(rng.integers(1, N + 1))
    D, F = 5, 7
    p = _shared_params(rng, S, N, D, F, act, act != "swiglu")
    x = rng.standard_normal((T, D))
    for C in (None, 0, 2):
        for residual in (False, True):
            a = oracle.moe_forward(x, p, k=k, act=act, capacity_slots=C, residual=residual, n_shared=S)["y"]
            b = oracle.brute_forward(x, p, k=k, act=act, capacity_slots=C, residual=residual, n_shared=S)
            assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_one_routed_one_shared_equals_torch_modules():
    """N = 1, k = 1: the routed gate is exactly 1, so the layer is the sum of
    two plain MLPs (torch CPU Linear + GELU), the routed one in slot 1."""
    rng = np.random.default_rng(17)
    T, D, F = 23, 12, 20
    p = _shared_params(rng, 1, 1, D, F, "gelu", True)
    x = rng.standard_normal((T, D))
    r = oracle.moe_forward(x, p, k=1, act="gelu", n_shared=1)
    xt = torch.from_numpy(x)

    def mlp(e):
        fc1 = torch.nn.Linear(D, F).double()
        fc2 = torch.nn.Linear(F, D).double()
        with torch.no_grad():
            fc1.weight.copy_(torch.from_numpy(p["w1"][e])); fc1.bias.copy_(torch.from_numpy(p["b1"][e]))
            fc2.weight.copy_(torch.from_numpy(p["w2"][e])); fc2.bias.copy_(torch.from_numpy(p["b2"][e]))
            return fc2(Fnn.gelu(fc1(xt))).numpy()
    assert np.allclose(r["gate"], 1.0)
    assert np.allclose(r["y"], mlp(0) + mlp(1), rtol=1e-12, atol=1e-12)


def test_shared_rows_and_gate_one_pinned_by_unique_biases():
    """W2 = 0: every expert outputs its own b2, so y[t] = sum over shared s of
    b2[s] + sum over kept choices of g[t,j] * b2[S + idx[t,j]], exactly."""
    rng = np.random.default_rng(18)
    T, D, F, N, S, k = 41, 6, 9, 5, 2, 2
    p = _shared_params(rng, S, N, D, F, "gelu", True)
    p["w2"][:] = 0.0
    p["b2"] = np.arange((S + N) * D, dtype=np.float64).reshape(S + N, D) + 1.0
    x = rng.standard_normal((T, D))
    for C in (None, 7, 0):
        r = oracle.moe_forward(x, p, k=k, act="gelu", capacity_slots=C, n_shared=S)
        want = np.tile(p["b2"][:S].sum(0), (T, 1))
        flat = r["idx"].reshape(-1)
        for a in range(T * k):
            t, j = divmod(a, k)
            rank = int((flat[:a] == flat[a]).sum())
            if C is None or rank < C:
                want[t] += r["gate"][t, j] * p["b2"][S + flat[a]]
        assert np.allclose(r["y"], want, rtol=1e-14, atol=1e-13)
        # rows: shared expert s, token t at s*T + t; routed rows after S*T
        assert r["offsets"][:S + 1].tolist() == [s * T for s in range(S + 1)]
        assert (r["perm"][:S * T] == np.tile(np.arange(T) * k, S)).all()
        kept = r["slot"] >= 0
        assert (r["slot"][kept] >= S * T).all()
        # combine_rows over the same rows reproduces the layer output
        y2 = oracle.combine_rows(r["y_perm"], r["slot"], r["gate"], k, None, n_shared=S)
        assert np.allclose(y2, r["y"], rtol=1e-13, atol=1e-12)
