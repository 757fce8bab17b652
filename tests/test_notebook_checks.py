"""The self-checks of the notebook "Mixture-of-experts and expert
parallelism" (sections "Dispatch and gather", "Capacity factor" and "Switch
Transformer auxiliary loss"), restated and run through the oracle on the
tiny layer with the notebook's sizes and distributions (1024 tokens, D=256,
8 experts, top-2, Linear+GELU+Linear experts)."""
import numpy as np
import pytest

import oracle
from workloads import generate, get_config

pytestmark = pytest.mark.cpu


@pytest.fixture(scope="module")
def c1_run():
    cfg = get_config("c1")
    inp = generate(cfg)
    r = oracle.moe_forward(inp["x"], inp, k=cfg.k, act=cfg.act)
    return cfg, inp, r


def test_output_shape_and_finite(c1_run):
    cfg, inp, r = c1_run
    assert r["y"].shape == tuple(inp["x"].shape)
    assert np.isfinite(r["y"]).all()


def test_higher_capacity_reduces_drops(c1_run):
    cfg, inp, r = c1_run
    d10 = oracle.drop_rate(r["counts"], oracle.capacity(cfg.T, cfg.k, cfg.N, 1.0))
    d15 = oracle.drop_rate(r["counts"], oracle.capacity(cfg.T, cfg.k, cfg.N, 1.5))
    assert d15 <= d10


def test_untrained_router_has_measurable_imbalance(c1_run):
    cfg, inp, r = c1_run
    assert oracle.imbalance(r["counts"], cfg.T, cfg.k, cfg.N) >= 1.05


def test_aux_loss_imbalanced_higher_than_balanced(c1_run):
    cfg, inp, r = c1_run
    imb = oracle.switch_aux_loss(r["idx"], r["probs"], cfg.N)
    # a perfectly balanced router: token t takes experts t, t+1, ..., t+k-1
    # (mod N), so each expert holds T*k/N assignments, and every
    # probability is 1/N
    bal_idx = (np.arange(cfg.T)[:, None] + np.arange(cfg.k)[None, :]) % cfg.N
    assert (oracle.expert_counts(bal_idx, cfg.N) == cfg.T * cfg.k // cfg.N).all()
    bal = oracle.switch_aux_loss(bal_idx, np.full((cfg.T, cfg.N), 1.0 / cfg.N), cfg.N)
    assert imb > bal


def test_active_params_equal_k_over_N(c1_run):
    """Measured, not restated: each token's row of idx holds k distinct
    experts and the counts sum to T*k, so per-token expert use is k/N."""
    cfg, inp, r = c1_run
    rows = r["idx"].tolist()
    assert all(len(set(row)) == cfg.k for row in rows)
    frac = r["counts"].sum() / (cfg.T * cfg.N)
    assert frac == cfg.k / cfg.N
