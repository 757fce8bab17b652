"""The shader-clock probe (moe_clock_probe) on the GPU: the chain's length is
recorded and the clock it reports is a plausible core clock."""
import pytest
import torch

from mixture_experts_layer_expert_amd import api

pytestmark = pytest.mark.gpu


def test_clock_probe_idle(gpu):
    blocks, iters = 64, 200
    stamps = torch.zeros(4 * blocks, dtype=torch.int64, device=gpu)
    api.clock_probe(blocks, 10.0, iters, stamps)
    torch.cuda.synchronize()
    s = stamps.view(-1, 4).cpu()
    assert (s[:, 2] == 1024 * iters).all()
    assert (s[:, 1] > s[:, 0]).all()
    ghz = api.probe_clock_ghz(stamps)
    print(f"idle clock {ghz:.3f} GHz", flush=True)
    assert 0.3 <= ghz <= 3.0
