"""MI355X-native forward pass of a Mixture-of-Experts FFN layer.

The compute lives in libmoe_mi355x.so (HIP, gfx950); this package is its
thin Python binding.  See include/moe.h for the C ABI.
"""
from .api import (MoeBuffers, MoeError, MoeShape, capacity, combine, dispatch, expert_ffn,  # noqa: F401
                  forward, route, workspace_bytes)
