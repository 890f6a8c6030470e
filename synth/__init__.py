"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package only draws random numbers and arranges them into the shapes of the workloads.
It holds none of the scan's arithmetic, and neither the oracle nor the HIP library imports it.
"""
from .vmscan_inputs import (  # noqa: F401
    CONFIGS,
    round_bf16,
    make_vim_inputs,
    make_vim_v2_inputs,
    make_ss2d_inputs,
    make_conv1d_inputs,
    make_conv2d_inputs,
    dt_bias,
)
