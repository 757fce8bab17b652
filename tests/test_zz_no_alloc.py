"""moe_forward_noalloc (the workspace in the library's own device scratch)
against moe_forward with a caller workspace: identical routing tensors and
outputs, on two calls in a row, the second with fewer tokens; and a layer
whose workspace exceeds the scratch is rejected before any launch."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_expert_amd import _lib as L
from mixture_experts_layer_expert_amd import api
from workloads import generate, get_config, scaled_config

pytestmark = pytest.mark.gpu

FIELDS = ("out", "topk_idx", "topk_gate", "counts", "offsets", "perm", "slot", "n_dropped")


def _noalloc(shape, g, buf):
    api.forward_noalloc(shape, g["x"], g["w_router"], g.get("b_router"), g["w1"], g.get("b1"), g.get("w3"),
                        g["w2"], g.get("b2"), buf.out, buf.topk_idx, buf.topk_gate, buf.counts, buf.offsets,
                        buf.perm, buf.slot, buf.n_dropped)


def _poison(buf):
    for f in FIELDS:
        t = getattr(buf, f)
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _case(gpu, cfg, fused=False):
    print(f"no-alloc forward {cfg.name}: T={cfg.T} fused_decode={fused}", flush=True)
    inp = generate(cfg)
    g = {k: (None if v is None else v.to(gpu).contiguous()) for k, v in inp.items()}
    shape = api.MoeShape.from_config(cfg, fused_decode=fused)
    assert api.workspace_bytes(shape) <= L.MOE_NOALLOC_SCRATCH_BYTES
    ref = api.MoeBuffers(shape, device=gpu)
    got = api.MoeBuffers(shape, device=gpu)
    _poison(got)
    ref.forward(g["x"], g)
    _noalloc(shape, g, got)
    torch.cuda.synchronize()
    K = int(ref.offsets[-1].item())
    for f in FIELDS:
        a, b = getattr(ref, f), getattr(got, f)
        if f == "perm":
            a, b = a[:K], b[:K]
        assert torch.equal(a, b), f
    assert np.isfinite(got.out.float().cpu().numpy()).all()


def test_noalloc_matches_forward_twice_second_smaller(gpu):
    base = get_config("c5")
    _case(gpu, base)
    _case(gpu, scaled_config(base, T=40, name="c5_decode_bf16_T40"))


def test_noalloc_fused_decode_twice_second_smaller(gpu):
    """The fused decode kernel's fp32 shard partials in the scratch."""
    base = get_config("c5")
    _case(gpu, base, fused=True)
    _case(gpu, scaled_config(base, T=40, name="c5_decode_bf16_T40"), fused=True)


def test_noalloc_fp32_layer_then_smaller(gpu):
    base = get_config("c1")
    _case(gpu, scaled_config(base, T=700, name="c1_tiny_fp32_T700"))
    _case(gpu, scaled_config(base, T=90, name="c1_tiny_fp32_T90"))


def test_noalloc_rejects_a_layer_beyond_the_scratch(gpu):
    cfg = get_config("c4")
    shape = api.MoeShape.from_config(cfg)
    assert api.workspace_bytes(shape) > L.MOE_NOALLOC_SCRATCH_BYTES
    sc = shape.c()
    import ctypes
    st = L.load().moe_forward_noalloc(ctypes.byref(sc), *([None] * 16), None)
    assert st == L.MOE_ERR_WORKSPACE
