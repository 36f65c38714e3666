"""Seeded synthetic inputs for paged decode attention.

Shared by the CPU oracle's tests and the GPU library's tests and benchmark.
It holds no attention, scatter or block-copy arithmetic: only lengths, block
placement and N(0, 1) values.
"""
from .configs import CONFIGS, DTYPE_BYTES, DecodeConfig, kv_bytes
from .layout import Layout, draw_lengths, make_layout, shared_prefix_groups
from .values import POISON_BITS, HostStep, device_values, host_values, to_storage
from .beam import BEAM_CONFIGS, BeamConfig, beam_parents, prompt_values, step_values

__all__ = [
    "CONFIGS", "DTYPE_BYTES", "DecodeConfig", "kv_bytes", "Layout", "draw_lengths",
    "make_layout", "shared_prefix_groups", "POISON_BITS", "HostStep", "device_values", "host_values", "to_storage",
    "BEAM_CONFIGS", "BeamConfig", "beam_parents", "prompt_values", "step_values",
]
