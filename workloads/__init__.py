"""Seeded synthetic inputs for the paged KV-cache decode path.

This package is the only code shared by the fp64 oracle side and the HIP side of
the tests and the benchmark.  It draws lengths, block tables, query vectors and
K/V rows, and rounds them to fp16/bf16 bit patterns.  It contains none of the
method's arithmetic: no slot/address computation, no attention, no softmax.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    Workload,
    make_workload,
    f32_to_bf16_bits,
    f32_to_f16_bits,
    bits_to_f64,
    NAN_BITS,
)
