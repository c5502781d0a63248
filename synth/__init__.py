"""Seeded synthetic inputs for the selective scan and the decode step.

This package only draws random numbers and lays them out; it holds none of the
scan's arithmetic (no softplus, no exponentials of the decay, no recurrence).
Both the GPU path's tests/benchmark and the CPU oracle's tests consume it.
"""
from .gen import (  # noqa: F401
    ScanInputs,
    DecodeInputs,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_scan_inputs,
    make_config_inputs,
    make_scan_initial_state,
    make_scan_cotangents,
    SSDInputs,
    make_ssd_inputs,
    make_conv_params,
    make_decode_state,
    make_decode_step,
    make_decode_params,
)
from .configs import CONFIGS, ScanConfig, DecodeConfig, SSDConfig  # noqa: F401
