"""MI355X (gfx950) Mixture-of-Experts layer forward pass.

The compute path is the HIP library ``libmoe.so`` (C ABI: include/moe.h);
this package is its Python binding plus the seeded synthetic workloads.
"""
from ._lib import (MoeError, MoeLayer, Forward, balance, bias_update, capacity,  # noqa: F401
                   combine, dispatch,
                   forward, grouped_ffn, last_error, layer_from_inputs, lib, route,
                   route_expert_choice, timing_enable, timing_read)

__all__ = ["MoeError", "MoeLayer", "Forward", "balance", "bias_update", "capacity", "combine",
           "dispatch",
           "forward", "grouped_ffn", "last_error", "layer_from_inputs", "lib", "route",
           "route_expert_choice", "timing_enable", "timing_read"]
