"""Seeded synthetic workloads for the KDA RecoverSSM verify/commit path.

This package only draws random numbers and lays tensors out in memory the way
a serving KV cache does (one page per state slot holding the conv state, the
recurrent state and the verify records).  It contains none of the method's
arithmetic, so both the CPU oracle and the HIP path may consume it.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    LayerTensors,
    Workload,
    make_workload,
    to_f64,
)
