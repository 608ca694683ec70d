"""Layer schedule of the decoder stack, used by callers that drive the layer calls.

The mlxcel Compass issue ("Text decoder forward", and its "Validation" list with the
4-layer case of three sliding layers and one full layer) interleaves the two layer kinds
3:1: every fourth layer, counting from zero at index 3, is a full-attention layer with
no positional encoding; the others are sliding-window layers with MRoPE. The same
section adds the vision tower's deepstack features at the image rows after the first
three layers only. Host logic only: it chooses which C-ABI call and descriptor each
layer gets and does none of the layer's arithmetic.
"""
from __future__ import annotations

SLIDING = "sliding"
FULL = "full"
DEEPSTACK_LAYERS = 3


def layer_kind(i: int) -> str:
    """Kind of layer i (0-based): full attention when i is 3 mod 4, sliding otherwise."""
    if i < 0:
        raise ValueError(f"layer index {i} < 0")
    return FULL if i % 4 == 3 else SLIDING


def takes_deepstack(i: int) -> bool:
    """Whether the deepstack rows are added after layer i (layers 0, 1 and 2)."""
    return 0 <= i < DEEPSTACK_LAYERS
