"""Workload registry: the five MoE layer shapes and their input recipes.

Each entry names a synthetic instance shaped like the workloads the pages
discuss.  The pages measure on language-modelling and machine-translation
MoE models and on encoder-based MoE models ("Towards MoE Deployment:
Mitigating Inefficiencies in Mixture-of-Expert (MoE) Inference", abstract;
"Accelerating MoE Model Inference with Expert Sharding", abstract).  Those
models and their data are not available, so seeded random tensors of these
shapes stand in for them.

``x_seed`` values were found by ``tests/golden/find_seeds.py``: the x stream
is advanced until every token's top-(k+1) router logits are separated by at
least 1e-6 in exact arithmetic, so the routing decision of the instance is
well defined.  ``tests/test_workloads.py`` re-checks that rule with the
oracle.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int            # tokens
    D: int            # model dim
    F: int            # expert hidden dim (d_ff)
    N: int            # experts
    k: int            # experts per token
    act: str          # "gelu" (erf form) | "relu" | "swiglu"
    dtype: str        # "fp32" | "bf16": x, weights and output
    expert_bias: bool  # fc1/fc2 carry biases b1[N,F], b2[N,D]
    renorm: bool      # gates renormalised over the chosen k
    router_bias: Optional[str]  # None | "zipf1.2"
    cf: Optional[float]         # capacity factor; None = no limit
    residual: bool    # y = x + sum of kept expert outputs
    init: str         # "linear_default" (the notebook's distributions) | "normal0.02"
    seed: int         # base seed for every stream of this config
    x_seed: int = 0   # x stream seed offset (near-tie rule)
    n_shared: int = 0  # always-on experts, applied to every token with gate 1
    description: str = ""

    @property
    def A(self) -> int:
        """Number of (token, choice) assignments, T*k."""
        return self.T * self.k

    @property
    def n_slots(self) -> int:
        """Expert weight slots: the shared experts first, then the N routed."""
        return self.n_shared + self.N

    def with_cf(self, cf: Optional[float]) -> "MoeConfig":
        return dataclasses.replace(self, cf=cf)


CONFIGS: dict[str, MoeConfig] = {
    "c1": MoeConfig(
        name="c1_tiny_fp32", T=1024, D=256, F=1024, N=8, k=2, act="gelu", dtype="fp32",
        expert_bias=True, renorm=False, router_bias=None, cf=None, residual=False,
        init="linear_default", seed=0, x_seed=0,
        description="Tiny fp32 layer with the notebook's distributions: 1024 tokens, D=256, "
                    "8 experts, top-2 softmax router, Linear+GELU+Linear experts"),
    "c2": MoeConfig(
        name="c2_switch_bf16", T=16384, D=768, F=3072, N=128, k=1, act="relu", dtype="bf16",
        expert_bias=False, renorm=False, router_bias=None, cf=1.0, residual=True,
        init="normal0.02", seed=2, x_seed=0,
        description="Switch-style encoder layer: 32x512 tokens, D=768, d_ff=3072, 128 experts, "
                    "top-1, ReLU, capacity factor 1.0 (or 1.5), dropped tokens pass through"),
    "c3": MoeConfig(
        name="c3_skew_bf16", T=8192, D=1024, F=4096, N=16, k=2, act="gelu", dtype="bf16",
        expert_bias=True, renorm=False, router_bias="zipf1.2", cf=None, residual=False,
        init="normal0.02", seed=3, x_seed=0,
        description="Skewed routing: 8192 tokens, D=1024, d_ff=4096, 16 experts, top-2, "
                    "Zipf(1.2) router bias so expert 0 is in nearly every token's pair"),
    "c4": MoeConfig(
        name="c4_mixtral_bf16", T=8192, D=4096, F=14336, N=8, k=2, act="swiglu", dtype="bf16",
        expert_bias=False, renorm=True, router_bias=None, cf=None, residual=False,
        init="normal0.02", seed=4, x_seed=0,
        description="Mixtral-shaped prefill: 8192 tokens, D=4096, d_ff=14336, 8 experts, "
                    "top-2 renormalised, SwiGLU experts"),
    "c5": MoeConfig(
        name="c5_decode_bf16", T=128, D=2048, F=1408, N=64, k=6, act="swiglu", dtype="bf16",
        expert_bias=False, renorm=False, router_bias=None, cf=None, residual=False,
        init="normal0.02", seed=5, x_seed=0,
        description="Decode-regime fine-grained MoE: 128 tokens, D=2048, d_ff=1408, 64 experts, "
                    "top-6, SwiGLU experts; weight-streaming"),
    "c6": MoeConfig(
        name="c6_shared_bf16", T=4096, D=2048, F=1408, N=64, k=6, act="swiglu", dtype="bf16",
        expert_bias=False, renorm=False, router_bias=None, cf=None, residual=False,
        init="normal0.02", seed=6, x_seed=1, n_shared=2,
        description="Fine-grained MoE with always-on experts (the notebook's shared-experts "
                    "exercise, DeepSeek-V2-Lite-shaped): 4096 tokens, D=2048, d_ff=1408, 2 shared "
                    "+ 64 routed experts, top-6, SwiGLU"),
}


def get_config(key: str, cf: Optional[float] = "keep") -> MoeConfig:
    """Look up a config by short key (c1..c5) or full name."""
    cfg = CONFIGS.get(key)
    if cfg is None:
        for c in CONFIGS.values():
            if c.name == key:
                cfg = c
                break
    if cfg is None:
        raise KeyError(f"unknown workload {key!r}; known: {sorted(CONFIGS)}")
    if cf != "keep":
        cfg = cfg.with_cf(cf)
    return cfg


def scaled_config(base: MoeConfig, **changes) -> MoeConfig:
    """A reduced-size variant of a config (for oracle-sized parity cases)."""
    name = changes.pop("name", None) or (base.name + "_scaled")
    return dataclasses.replace(base, name=name, **changes)
