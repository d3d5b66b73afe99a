"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This package only draws random numbers and lays them out; it holds none of the
bit-plane method's arithmetic (no quantizer, no depth rule, no scores).  Both
the host generator here (numpy) and the device generator in ``synth/csrc``
implement the same published counter-based generators, so any element of any
workload can be regenerated on the host bit-for-bit without reading it back
from the device.
"""
from .philox import (  # noqa: F401
    splitmix64,
    philox4x32_10,
    unit_key,
    irwin_hall8_int,
    normal_values,
    STREAM_K,
    STREAM_V,
    STREAM_Q,
    STREAM_SIGMA,
    STREAM_ROT,
    NORMAL_MULT,
)
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
