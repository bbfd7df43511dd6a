"""Seeded synthetic inputs for one LatentMoE layer with MXFP4 expert weights.

This module is shared by the tests, the smoke check and the benchmark. It
draws inputs and encodes the expert weights into the MXFP4 storage format the
layer consumes; it computes none of the layer itself (no routing, no decode,
no GEMM, no combine).
"""

from .gen import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    LayerInputs,
    make_inputs,
    make_router,
    make_tokens,
    make_expert_weights,
    make_lora,
    quantize_mxfp4,
    LORA_NAMES,
)
