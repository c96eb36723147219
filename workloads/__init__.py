"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and lays out shapes; it holds none of the
attention method's arithmetic (no masks, no source resolution, no
quantisation, no softmax).  Both the CPU oracle and the HIP path take their
inputs from here, and nothing else is shared between them.
"""

from .gen import (
    PAGE_SIZE, bf16_from_f32, bf16_to_f32, normal_bf16, rms_normalise_bf16,
    PagePool, make_page_pool,
)
from .configs import (
    LayerSpec, Workload, tiny_workload, e2b_decode_workload, e2b_extend_workload,
    moe26b_decode_workload, int8_long_workload, e2b_layer_types, e4b_layer_types,
    WORKLOADS,
)

from .device import DeviceDraws

__all__ = [
    "DeviceDraws",
    "PAGE_SIZE", "bf16_from_f32", "bf16_to_f32", "normal_bf16", "rms_normalise_bf16",
    "PagePool", "make_page_pool",
    "LayerSpec", "Workload", "tiny_workload", "e2b_decode_workload", "e2b_extend_workload",
    "moe26b_decode_workload", "int8_long_workload", "e2b_layer_types", "e4b_layer_types",
    "WORKLOADS",
]
