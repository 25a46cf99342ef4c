"""MI355X-native MoE layer forward pass: HIP kernels for gfx950 behind a small C ABI.

The compute lives in libmoe.so (built from csrc/ by ``python -m
mixture_experts_layer_group_amd.build``); ``binding`` marshals torch tensors into it.
"""
from .configs import WORKLOADS, SMALL, ALL, BENCH_WORKLOAD  # noqa: F401
