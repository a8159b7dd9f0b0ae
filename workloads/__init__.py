"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side
tests and bench.

This package draws random numbers and lays them out; it holds none of the
attention, slot-mapping or merge arithmetic, so neither side of a parity check
can inherit a mistake from the other through it.
"""
from .synth import (  # noqa: F401
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_config,
    make_small_case,
    CONFIG_NAMES,
)
