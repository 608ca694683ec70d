"""The package's layer schedule (host logic that picks each layer's call) against the
page's 28-layer pattern fixture and the oracle's own rule, independently. CPU only."""
import json
import os

import pytest

import cohere2_block_mrope_amd.stack as S
from oracle import compass_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_schedule_matches_page_pattern():
    with open(os.path.join(GOLDEN, "layer_pattern_28.json")) as f:
        g = json.load(f)
    full = [i for i in range(g["n_layers"]) if S.layer_kind(i) == S.FULL]
    assert full == g["full_attention_layers"]
    assert all(S.layer_kind(i) == S.SLIDING for i in range(g["n_layers"]) if i not in full)


def test_schedule_agrees_with_oracle_and_deepstack_layers():
    assert [S.layer_kind(i) for i in range(64)] == [O.layer_kind(i) for i in range(64)]
    assert [i for i in range(28) if S.takes_deepstack(i)] == [0, 1, 2]
    with pytest.raises(ValueError):
        S.layer_kind(-1)
