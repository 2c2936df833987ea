"""Seeded synthetic inputs for the paged-KV decode step.

This package is shared by the oracle side (tests, the CPU baseline) and the
GPU side (tests, bench).  It holds only input generation: shapes, seeded
random draws and block-table layouts.  None of the decode step's arithmetic
(slot mapping, store, attention, sampling) lives here.
"""
from .configs import CONFIGS, DecodeConfig, config_by_name
from .generate import (
    HostInputs,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    host_inputs,
    stream_seed,
)

__all__ = [
    "CONFIGS",
    "DecodeConfig",
    "config_by_name",
    "HostInputs",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "host_inputs",
    "stream_seed",
]
