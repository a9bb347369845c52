"""Seeded synthetic inputs for the head-routed hybrid attention prefill.

This package draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, no router, no attention).  Both the HIP path
(through the tests and the bench) and the CPU oracle consume what it makes.
"""
from .gen import (  # noqa: F401
    Case,
    bf16_bits,
    bf16_bits_to_f32,
    build_case,
    custom_case,
    draw_router_weights,
    normal,
)
from .configs import WORKLOADS, Workload, get  # noqa: F401
