"""Search the x-stream seed offset of each workload so that no token has two
of its top-(k+1) router logits within 1e-6 of each other.

Run:  python tests/golden/find_seeds.py
Prints, for every config, the first offset that satisfies the rule and the
instance's smallest margin.  The offsets are recorded in
workloads/configs.py (field ``x_seed``).  Only the oracle and the input
generators are used.
"""
import dataclasses
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402

MIN_MARGIN = 1e-6


def main():
    for key, cfg in sorted(CONFIGS.items()):
        off = cfg.x_seed
        while True:
            c = dataclasses.replace(cfg, x_seed=off)
            inp = generate(c, parts=("x", "router"))
            l = oracle.router_logits(inp["x"], inp["w_router"], inp["b_router"])
            m = float(oracle.topk_margin(l, c.k).min())
            if m >= MIN_MARGIN:
                break
            off += 1
        print(f"{key}: x_seed={off} min_margin={m:.3e}", flush=True)


if __name__ == "__main__":
    main()
