"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle calls.

This module only draws random numbers and builds shapes; it holds none of the
method's arithmetic (no quantisation, no forward pass, no sampling rule).
Every draw is seeded, so both the GPU path and the CPU oracle can be fed the
very same values.
"""
from .generators import (  # noqa: F401
    normal_tensor,
    uniform_codes,
    token_ids,
    model_weights,
    kv_history,
    logits_pair,
)
from .configs import CONFIGS, ModelShape, shape_by_name  # noqa: F401
