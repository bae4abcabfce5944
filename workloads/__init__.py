"""Seeded synthetic workloads for the HSMLA forward pass.

This package only describes shapes and draws random inputs.  It holds none
of the method's arithmetic, so both the HIP library's tests/benchmark and the
CPU oracle's tests may use it without sharing any computation.
"""

from .synth import (  # noqa: F401
    Workload,
    WORKLOADS,
    keep_blocks_for,
    make_inputs,
    scaled,
)
