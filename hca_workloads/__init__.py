"""Seeded synthetic workloads for the HCA layer forward.

This package only draws inputs: shapes, seeds and value distributions.  It
holds none of the method's arithmetic (no pooling, no attention, no softmax),
so both the HIP path and the CPU oracle can be fed from it without sharing
code.  The shapes follow the model the pages describe (release blog and model
card: 64 attention heads, 512-dimensional HCA heads, one cached entry per 128
tokens, contexts of 128K tokens in pre-training and up to 1M at inference);
the pages publish no dataset for this layer, so every tensor is random.
"""
from .configs import CONFIGS, HcaConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    chunk_inputs,
    cu_from_lengths,
    decode_inputs,
    dsa_inputs,
    draw_lengths,
    backward_inputs,
    prefill_inputs,
    ring_from_raw,
)
