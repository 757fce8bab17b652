"""Pins of the oracle's router (selection, gates, margin) against facts that
do not come from the oracle itself: a hand-derived example, brute-force
sorting, exact ties, closed forms of the softmax."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.cpu


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_hand_derived_router_example():
    g = _load("route_tiny.json")
    x = np.array(g["x"], dtype=np.float64)
    w = np.array(g["w_router"], dtype=np.float64)
    l = oracle.router_logits(x, w)
    assert np.array_equal(l, np.array(g["expected_logits"], dtype=np.float64))
    assert oracle.expert_order(l).tolist() == g["expected_order"]
    idx = oracle.select_topk(l, 2)
    assert idx.tolist() == [row[:2] for row in g["expected_order"]]
    assert oracle.expert_counts(idx, 4).tolist() == g["expected_counts_top2"]["counts"]
    assert oracle.topk_margin(l, 2).tolist() == g["expected_margin_top2"]["margin"]


def test_router_has_no_hidden_bias_and_adds_given_bias():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((3, 7))
    b = np.array([0.5, -1.0, 2.0])
    # logits are linear in x: l(2x) = 2 l(x) exactly for power-of-two scaling
    assert np.array_equal(oracle.router_logits(2 * x, w), 2 * oracle.router_logits(x, w))
    # zero input gives exactly the bias
    assert np.array_equal(oracle.router_logits(np.zeros((2, 7)), w, b), np.tile(b, (2, 1)))


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_python_sorted(seed):
    rng = np.random.default_rng(seed)
    T, N = 13, int(rng.integers(1, 9))
    # small integers give many exact ties
    l = rng.integers(-2, 3, size=(T, N)).astype(np.float64)
    for k in range(1, N + 1):
        idx = oracle.select_topk(l, k)
        for t in range(T):
            want = sorted(range(N), key=lambda e: (-l[t, e], e))[:k]
            assert idx[t].tolist() == want


def test_ties_go_to_lower_index_with_duplicate_router_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 16))
    w = rng.standard_normal((6, 16))
    w[4] = w[1]  # experts 1 and 4 always tie exactly
    l = oracle.router_logits(x, w)
    assert np.array_equal(l[:, 1], l[:, 4])
    order = oracle.expert_order(l)
    for t in range(50):
        pos = order[t].tolist()
        assert pos.index(1) < pos.index(4)


def test_k_equals_N_returns_every_expert_in_decreasing_logit_order():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((20, 5))
    idx = oracle.select_topk(l, 5)
    for t in range(20):
        assert sorted(idx[t].tolist()) == list(range(5))
        v = l[t, idx[t]]
        assert np.all(v[:-1] >= v[1:])


def test_softmax_closed_forms():
    # equal logits -> uniform
    p = oracle.softmax(np.zeros((3, 8)))
    assert np.allclose(p, 1 / 8, rtol=0, atol=1e-15)
    # two experts: p0 = 1 / (1 + exp(l1 - l0))  (logistic function)
    l = np.array([[0.3, -1.2], [5.0, 5.0], [-2.0, 1.0]])
    p = oracle.softmax(l)
    for t in range(3):
        assert p[t, 0] == pytest.approx(1 / (1 + math.exp(l[t, 1] - l[t, 0])), rel=1e-14)
    # shift invariance and ratio property p_a / p_b = exp(l_a - l_b)
    rng = np.random.default_rng(2)
    l = rng.standard_normal((10, 6)) * 3
    p = oracle.softmax(l)
    assert np.allclose(p.sum(1), 1.0, atol=1e-14)
    assert np.allclose(oracle.softmax(l + 7.25), p, atol=1e-15)
    assert np.allclose(p[:, 2] / p[:, 5], np.exp(l[:, 2] - l[:, 5]), rtol=1e-12)
    # probabilities are ordered as the logits are
    o_p = np.argsort(-p, axis=1, kind="stable")
    assert np.array_equal(o_p, oracle.expert_order(l))


def test_gate_values_plain_and_renormalised():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((30, 8))
    r = oracle.route(rng.standard_normal((30, 4)), rng.standard_normal((8, 4)), None, 2, False)
    p, idx, g = r["probs"], r["idx"], r["gate"]
    for t in range(30):
        for j in range(2):
            assert g[t, j] == p[t, idx[t, j]]
    # not renormalised: chosen gates sum to less than one unless k == N
    assert np.all(g.sum(1) < 1.0)
    rr = oracle.route(rng.standard_normal((30, 4)), rng.standard_normal((8, 4)), None, 2, True)
    assert np.allclose(rr["gate"].sum(1), 1.0, atol=1e-15)
    # renormalised top-2 gate equals the logistic function of the logit gap
    gap = np.take_along_axis(rr["logits"], rr["idx"], 1)
    assert np.allclose(rr["gate"][:, 0], 1 / (1 + np.exp(gap[:, 1] - gap[:, 0])), rtol=1e-13)
    # top-1 without renorm: the gate is the largest probability, not 1
    r1 = oracle.route(rng.standard_normal((10, 4)), rng.standard_normal((8, 4)), None, 1, False)
    assert np.allclose(r1["gate"][:, 0], r1["probs"].max(1), rtol=0, atol=0)
    del l


def test_margin_brute_force():
    rng = np.random.default_rng(5)
    for N in (1, 2, 3, 7):
        l = rng.standard_normal((9, N))
        for k in range(1, N + 1):
            m = oracle.topk_margin(l, k)
            for t in range(9):
                s = sorted(l[t].tolist(), reverse=True)
                gaps = [s[r] - s[r + 1] for r in range(min(k, N - 1))]
                assert m[t] == (min(gaps) if gaps else np.inf)
