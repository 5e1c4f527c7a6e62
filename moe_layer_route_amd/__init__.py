"""MI355X-native gpt-oss MoE block forward.

The compute runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/moe_layer_route.h``); this package is the thin Python binding
(argument marshalling only) plus the seeded input generator.

``moe_route``, ``moe_forward`` and the stage calls are loaded lazily from the
native library, so ``import moe_layer_route_amd.datagen`` works without it.
"""
from __future__ import annotations

__all__ = ["moe_route", "moe_forward", "moe_forward_ex", "moe_permute", "moe_gate_up",
           "moe_down", "moe_combine", "workspace_bytes", "expert_path", "library", "MoEError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
