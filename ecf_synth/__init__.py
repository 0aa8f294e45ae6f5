"""Seeded synthetic inputs for the expert-cached MoE layer.

This package generates inputs only: activations, router weights or router
logits, and expert weights (bf16, fp32 or MXFP4-encoded).  It holds none of
the layer's arithmetic (no routing, no expert FFN, no combine), so both the
oracle tests and the GPU path may draw their inputs from it.

The generator is counter based (splitmix64 over a per-tensor key), so any
expert of any layer can be regenerated on its own, on the CPU or on the GPU.
Transcendental functions (log, cos) may differ in the last bit between the
CPU and GPU libraries, so a test generates its inputs once, on one device,
and hands the same bytes to both sides.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    T_X, T_WR, T_WG, T_WU, T_WD, T_LOGITS, T_PERM,
    key_of,
    uniform,
    normal,
    to_bf16,
    quantize_mxfp4,
    expert_weights,
    router_weights,
    activations,
    router_logits,
    zipf_gumbel_logits,
    popularity_rank,
    phase_of,
)
