"""Seeded random draws for one MoE layer instance (inputs only).

Two recipes:

* ``"linear_default"``, the distributions of the notebook "Mixture-of-experts
  and expert parallelism" (sections "Top-k router" and "Dispatch and
  gather"): x ~ N(0, 1); router weights ~ N(0, 0.1^2) and no router bias;
  every expert weight and bias ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)) with
  fan_in = D for fc1 and F for fc2 (PyTorch's default for a Linear layer).
  The tensors are drawn from the same per-(tensor, expert) generators as the
  other recipe, not in the notebook's order of draws.
* ``"normal0.02"``: x ~ N(0, 1); router, expert weights and (when present)
  expert biases ~ N(0, 0.02^2).  Every (tensor, expert) pair has its own
  ``torch.Generator`` so that one expert can be regenerated alone and the
  draws can run on several threads.  The optional "zipf1.2" router bias is
  b[e] = -1.2 * ln(e + 1), the logarithm of a Zipf(s=1.2) weight over expert
  rank, stored in fp32.

bf16 tensors are drawn in fp32 and rounded to nearest-even.  All tensors are
CPU tensors in the layouts of the C ABI: x[T,D], w_router[N,D], b_router[N],
w1[S+N,F,D], b1[S+N,F], w3[S+N,F,D], w2[S+N,D,F], b2[S+N,D]; with S shared
(always-on) experts they take the first S expert slots and routed expert r
is slot S + r.
"""
from __future__ import annotations

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional

import torch

from .configs import MoeConfig

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}
_STD_W = 0.02
_ALL_PARTS = ("x", "router", "experts")


def _stream_seed(base: int, tensor: str, e: int) -> int:
    return (base * 1_000_003 + zlib.crc32(tensor.encode()) * 65_537 + e * 7_919) % (2**62)


def _normal(shape, seed: int, std: float, dtype: torch.dtype, out: Optional[torch.Tensor] = None):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    v = v.to(dtype)
    if out is not None:
        out.copy_(v)
        return out
    return v


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def zipf_router_bias(N: int, s: float = 1.2) -> torch.Tensor:
    return torch.tensor([-s * math.log(e + 1.0) for e in range(N)], dtype=torch.float32)


def _expert_tensor_specs(cfg: MoeConfig):
    """(name, per-expert shape) of each expert parameter the config has."""
    specs = [("w1", (cfg.F, cfg.D))]
    if cfg.act == "swiglu":
        specs.append(("w3", (cfg.F, cfg.D)))
    specs.append(("w2", (cfg.D, cfg.F)))
    if cfg.expert_bias:
        specs += [("b1", (cfg.F,)), ("b2", (cfg.D,))]
    return specs


def expert_slice(cfg: MoeConfig, tensor: str, e: int) -> torch.Tensor:
    """Regenerate one expert's parameter alone ("normal0.02" recipe only)."""
    if cfg.init != "normal0.02":
        raise ValueError("expert_slice is defined for the normal0.02 recipe")
    shape = dict(_expert_tensor_specs(cfg))[tensor]
    return _normal(shape, _stream_seed(cfg.seed, tensor, e), _STD_W, _TORCH_DTYPE[cfg.dtype])


def _uniform(shape, seed: int, bound: float) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.rand(shape, generator=g, dtype=torch.float32).mul_(2.0 * bound).sub_(bound)


def _gen_linear_default(cfg: MoeConfig, parts: Iterable[str]) -> dict:
    if cfg.dtype != "fp32":
        raise ValueError("the linear_default recipe is fp32")
    if cfg.act == "swiglu":
        raise ValueError("the linear_default recipe has fc1 and fc2 only")
    out: dict = {}
    if "x" in parts:
        out["x"] = _normal((cfg.T, cfg.D), _stream_seed(cfg.seed, "x", cfg.x_seed), 1.0, torch.float32)
    if "router" in parts:
        out["w_router"] = _normal((cfg.N, cfg.D), _stream_seed(cfg.seed, "router", 0), 0.1, torch.float32)
        out["b_router"] = None
    if "experts" in parts:
        bound1, bound2 = 1.0 / math.sqrt(cfg.D), 1.0 / math.sqrt(cfg.F)
        for name, shape, bound in (("w1", (cfg.F, cfg.D), bound1), ("b1", (cfg.F,), bound1),
                                   ("w2", (cfg.D, cfg.F), bound2), ("b2", (cfg.D,), bound2)):
            out[name] = torch.stack([_uniform(shape, _stream_seed(cfg.seed, name, e), bound)
                                     for e in range(cfg.n_slots)]).contiguous()
        out["w3"] = None
    return out


def _gen_normal(cfg: MoeConfig, parts: Iterable[str]) -> dict:
    dt = _TORCH_DTYPE[cfg.dtype]
    out: dict = {}
    if "x" in parts:
        out["x"] = _normal((cfg.T, cfg.D), _stream_seed(cfg.seed, "x", cfg.x_seed), 1.0, dt)
    if "router" in parts:
        out["w_router"] = _normal((cfg.N, cfg.D), _stream_seed(cfg.seed, "router", 0), _STD_W, dt)
        if cfg.router_bias is None:
            out["b_router"] = None
        elif cfg.router_bias == "zipf1.2":
            out["b_router"] = zipf_router_bias(cfg.N, 1.2)
        else:
            raise ValueError(f"unknown router bias recipe {cfg.router_bias!r}")
    if "experts" in parts:
        specs = _expert_tensor_specs(cfg)
        jobs = []
        for name, shape in specs:
            t = torch.empty((cfg.n_slots,) + shape, dtype=dt)
            out[name] = t
            for e in range(cfg.n_slots):
                jobs.append((t[e], shape, _stream_seed(cfg.seed, name, e)))
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(lambda j: _normal(j[1], j[2], _STD_W, dt, out=j[0]), jobs))
        for name in ("w3", "b1", "b2"):
            out.setdefault(name, None)
    return out


def generate(cfg: MoeConfig, parts: Iterable[str] = _ALL_PARTS) -> dict:
    """Draw the tensors of one instance; ``parts`` may omit "experts"."""
    parts = tuple(parts)
    if cfg.init == "linear_default":
        return _gen_linear_default(cfg, parts)
    if cfg.init == "normal0.02":
        return _gen_normal(cfg, parts)
    raise ValueError(f"unknown init recipe {cfg.init!r}")
