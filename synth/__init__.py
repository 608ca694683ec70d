"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module holds random-number generation and workload shapes only: none of
the decoder layer's arithmetic lives here. Both sides of every parity check
consume the exact bytes produced by these functions.
"""
from .rng import splitmix64, stream_seed, normal, normal_bf16, bf16_round, bf16_bits, bits_to_f32
from .workloads import (LayerShape, WORKLOADS, Stream, image_text_row, text_tokens, IMAGE_TOKEN_ID,
                        VISION_START_ID, VISION_END_ID, make_layer_weights, make_layer_input,
                        TensorId)

__all__ = [
    "splitmix64", "stream_seed", "normal", "normal_bf16", "bf16_round", "bf16_bits", "bits_to_f32",
    "LayerShape", "WORKLOADS", "Stream", "image_text_row", "text_tokens", "IMAGE_TOKEN_ID", "VISION_START_ID",
    "VISION_END_ID", "make_layer_weights", "make_layer_input", "TensorId",
]
