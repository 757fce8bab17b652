"""Input generators: determinism, bf16 rounding, and the near-tie rule."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, expert_slice, generate, get_config, scaled_config

pytestmark = pytest.mark.cpu

MIN_MARGIN = 1e-6


def test_same_seed_same_bytes():
    cfg = scaled_config(get_config("c3"), T=64, D=32, F=48)
    a, b = generate(cfg), generate(cfg)
    for name in a:
        if a[name] is None:
            assert b[name] is None
        else:
            assert torch.equal(a[name], b[name]), name


def test_expert_slice_matches_full_draw():
    cfg = scaled_config(get_config("c4"), T=16, D=64, F=96)
    full = generate(cfg)
    for name in ("w1", "w3", "w2"):
        for e in (0, cfg.N - 1):
            assert torch.equal(full[name][e], expert_slice(cfg, name, e))


def test_bf16_is_round_to_nearest_even_of_fp32():
    cfg = scaled_config(get_config("c2"), T=256, D=64, F=32, N=4)
    g = torch.Generator().manual_seed(0)
    v = torch.randn(10000, generator=g)
    b = v.to(torch.bfloat16)
    bits = v.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = b.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(got, rne)
    x = generate(cfg, parts=("x",))["x"]
    assert x.dtype == torch.bfloat16


def test_notebook_recipe_shapes_and_ranges():
    cfg = get_config("c1")
    inp = generate(cfg)
    assert inp["x"].shape == (1024, 256)
    assert inp["w_router"].shape == (8, 256)
    assert inp["w1"].shape == (8, 1024, 256) and inp["w2"].shape == (8, 256, 1024)
    # default nn.Linear init is U(+-1/sqrt(fan_in)) for weights and biases
    assert inp["w1"].abs().max() <= 1 / 16 and inp["b1"].abs().max() <= 1 / 16
    assert inp["w2"].abs().max() <= 1 / 32 and inp["b2"].abs().max() <= 1 / 32
    assert abs(float(inp["w_router"].std()) - 0.1) < 0.01


def test_zipf_bias_makes_expert_zero_hot():
    cfg = get_config("c3")
    inp = generate(cfg, parts=("x", "router"))
    b = inp["b_router"].double().numpy()
    assert b[0] == 0.0 and np.all(np.diff(b) < 0)
    r = oracle.route(inp["x"], inp["w_router"], inp["b_router"], cfg.k, cfg.renorm)
    share = oracle.expert_counts(r["idx"], cfg.N)[0] / (cfg.T * cfg.k)
    assert 0.4 < share <= 0.5


@pytest.mark.parametrize("key", sorted(CONFIGS))
def test_instance_has_no_near_ties(key):
    cfg = CONFIGS[key]
    inp = generate(cfg, parts=("x", "router"))
    l = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
    m = oracle.topk_margin(l, cfg.k)
    assert m.min() >= MIN_MARGIN, (key, float(m.min()))
