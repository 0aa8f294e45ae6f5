"""The oracle: a plain, slow CPU definition of the expert-cached MoE layer.

TEST INFRASTRUCTURE ONLY.  tests/, the smoke check and the benchmark's
CPU-baseline leg are its only users; the product path never imports it, and
it imports nothing from the product.  See oracle/ref.py for the API.
"""
from .ref import (  # noqa: F401
    ORC_F32, ORC_BF16, ORC_MXFP4,
    lib,
    e2m1, e8m0,
    logits, route, permute, moe_tokens, moe_layer, expert_ffn, mxfp4_as_bf16,
    qstar, qstar_closed_form,
    LRURef,
)
