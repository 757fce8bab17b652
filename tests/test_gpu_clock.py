"""The shader-clock probe (moe_clock_probe) on the GPU: its real-time window
matches the request and the clock it reports is a plausible core clock."""
import pytest
import torch

from mixture_experts_layer_expert_amd import api

pytestmark = pytest.mark.gpu


def test_clock_probe_idle(gpu):
    blocks = 64
    stamps = torch.zeros(4 * blocks, dtype=torch.int64, device=gpu)
    api.clock_probe(blocks, 10.0, 200.0, stamps)
    torch.cuda.synchronize()
    s = stamps.view(-1, 4).cpu()
    ticks = (s[:, 1] - s[:, 0]).tolist()
    cycles = (s[:, 3] - s[:, 2]).tolist()
    # 200 us of the 100 MHz counter, plus the few ticks one loop turn takes
    assert all(20000 <= t <= 20000 + 2000 for t in ticks), ticks[:4]
    assert all(c > 0 for c in cycles)
    ghz = api.probe_clock_ghz(stamps)
    print(f"idle clock {ghz:.3f} GHz", flush=True)
    assert 0.3 <= ghz <= 3.0
