"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant replaces one oracle function with a plausible wrong variant (a
dropped term, a flipped sign, an off-by-one index, a transposed operand), then
runs the pins that should catch it. CPU only; the oracle module is restored
after every case by monkeypatch.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import compass_oracle as O
import tests.test_oracle_pins as P


def _edited(name, *edits):
    """The oracle function `name` recompiled from its own source with each (old, new) text edit
    applied once: a one-token mistake planted in the real code, not a rewrite. It runs with a
    copy of the oracle's globals, so it calls the unmutated helpers."""
    src = textwrap.dedent(inspect.getsource(getattr(O, name)))
    for old, new in edits:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    g = dict(O.__dict__)
    exec(compile(src, f"<mutant of {name}>", "exec"), g)
    return g[name]


def _rotate_half_wrong_sign(x):
    half = x.shape[-1] // 2
    return np.concatenate([x[..., half:], -x[..., :half]], axis=-1)


def _rotate_half_pairwise(x):
    y = np.empty_like(x)
    y[..., 0::2] = -x[..., 1::2]
    y[..., 1::2] = x[..., 0::2]
    return y


def _axis_map_shifted(section, half):
    s_t, s_h, s_w = section
    ax = np.zeros(half, dtype=np.int64)
    for j in range(half):
        if j % 3 == 0 and j < 3 * s_h:
            ax[j] = 1
        elif j % 3 == 1 and j < 3 * s_w:
            ax[j] = 2
    return ax


def _axis_map_contiguous(section, half):
    s_t, s_h, s_w = section
    return np.array([0] * s_t + [1] * s_h + [2] * s_w, dtype=np.int64)


def _inv_freq_wrong_exponent(theta, hd):
    j = np.arange(hd // 2, dtype=np.float64)
    return float(theta) ** (-j / hd)


def _layer_norm_rms(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x ** 2).mean(-1, keepdims=True) + eps) * w


def _layer_norm_no_weight(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True) + eps)


_orig_attention = O.attention


def _attention_window_off_by_one(q, k, v, kind, window, q_index=None, k_index=None):
    return _orig_attention(q, k, v, kind, window + 1 if kind == "sliding" else window, q_index, k_index)


def _attention_gqa_modulo(q, k, v, kind, window, q_index=None, k_index=None):
    Hq, Hkv = q.shape[0], k.shape[0]
    g = Hq // Hkv
    kk = np.stack([k[h % Hkv] for h in range(Hq)])
    vv = np.stack([v[h % Hkv] for h in range(Hq)])
    if g == 1:
        kk, vv = kk[::-1].copy(), vv[::-1].copy()
    return _orig_attention(q, kk, vv, kind, window, q_index, k_index)


def _attention_no_scale(q, k, v, kind, window, q_index=None, k_index=None):
    return _orig_attention(q * np.sqrt(q.shape[-1]), k, v, kind, window, q_index, k_index)


def _attention_not_causal(q, k, v, kind, window, q_index=None, k_index=None):
    Nk = k.shape[1]
    far = np.full(q.shape[1], 10 ** 9) if q_index is None else np.full(len(q_index), 10 ** 9)
    if kind == "sliding":
        return _orig_attention(q, k, v, kind, window, q_index, k_index)
    return _orig_attention(q, k, v, kind, window, far, k_index)


def _silu_sigmoid_only(x):
    return 1.0 / (1.0 + np.exp(-x))


_orig_chunk = O.layer_prefill_chunk


def _chunk_ignores_cache(shape, w, x, pos, k_cache, v_cache, start):
    return _orig_chunk(shape, w, x, pos, k_cache, v_cache, np.zeros_like(start))


def _decode_positions_without_delta(lens, rope_delta):
    p = np.asarray(lens, dtype=np.int64)
    return np.stack([p, p, p])


def _chunk_start_off_by_one(shape, w, x, pos, k_cache, v_cache, start):
    return _orig_chunk(shape, w, x, pos, k_cache, v_cache, np.maximum(np.asarray(start) - 1, 0))


_orig_varlen = O.layer_prefill_varlen


def _varlen_sequences_see_each_other(shape, w, x, pos, cu_seqlens, k_cache=None, v_cache=None, start=None):
    """The packed batch treated as one long row."""
    if k_cache is not None:
        return _orig_varlen(shape, w, x, pos, cu_seqlens, k_cache, v_cache, start)
    T = np.asarray(x).shape[0]
    return _orig_varlen(shape, w, x, pos, [0, T], None, None, None)[0], None, None


def _varlen_start_ignored(shape, w, x, pos, cu_seqlens, k_cache=None, v_cache=None, start=None):
    return _orig_varlen(shape, w, x, pos, cu_seqlens, k_cache, v_cache,
                        None if start is None else np.zeros(len(start), dtype=np.int64))


_orig_embed = O.embed
_orig_greedy = O.greedy_token


def _embed_ignores_image_rows(tokens, embed_table, image_rows=None, image_feats=None):
    return _orig_embed(tokens, embed_table)


def _greedy_last_maximum(h_last, norm_w, eps, embed_table, logit_scale):
    lg = O.logits(h_last, norm_w, eps, embed_table, logit_scale)
    return lg.shape[1] - 1 - np.argmax(lg[:, ::-1], axis=1)


_orig_unpack_q4 = O.unpack_q4
_orig_dequantize_q4 = O.dequantize_q4


def _unpack_q4_high_first(packed):
    c = _orig_unpack_q4(packed)
    out = c.copy()
    out[:, 0::2], out[:, 1::2] = c[:, 1::2], c[:, 0::2]
    return out


def _dequantize_q4_group_32(packed, scales, biases):
    codes = _orig_unpack_q4(packed).astype(float)
    s = np.repeat(np.asarray(scales, float), 32, axis=1)[:, :codes.shape[1]]
    b = np.repeat(np.asarray(biases, float), 32, axis=1)[:, :codes.shape[1]]
    return s * codes + b


def _dequantize_q4_no_bias(packed, scales, biases):
    return _orig_dequantize_q4(packed, scales, np.zeros_like(np.asarray(biases, float)))


_orig_section_layout = O.mrope_section_layout


def _sections_t_first(section, half):
    axis, fidx = _orig_section_layout(section, half)
    n_t = int(section[0])
    return np.roll(axis, n_t), np.roll(fidx, n_t)


def _sections_unpermuted(section, half):
    axis, _ = _orig_section_layout(section, half)
    return axis, np.arange(half)


MUTANTS = {
    "rotate_half sign": ("rotate_half", _rotate_half_wrong_sign),
    "pairwise rope": ("rotate_half", _rotate_half_pairwise),
    "axis map shifted": ("mrope_axis_map", _axis_map_shifted),
    "axis map contiguous": ("mrope_axis_map", _axis_map_contiguous),
    "inv_freq exponent": ("inv_freq", _inv_freq_wrong_exponent),
    "rmsnorm instead of layernorm": ("layer_norm", _layer_norm_rms),
    "layernorm weight dropped": ("layer_norm", _layer_norm_no_weight),
    "window off by one": ("attention", _attention_window_off_by_one),
    "gqa head map": ("attention", _attention_gqa_modulo),
    "attention scale dropped": ("attention", _attention_no_scale),
    "full layer not causal": ("attention", _attention_not_causal),
    "silu term dropped": ("silu", _silu_sigmoid_only),
    "chunk ignores the cache": ("layer_prefill_chunk", _chunk_ignores_cache),
    "chunk start off by one": ("layer_prefill_chunk", _chunk_start_off_by_one),
    "decode positions ignore rope_delta": ("decode_positions", _decode_positions_without_delta),
    "embed ignores image rows": ("embed", _embed_ignores_image_rows),
    "greedy ties to the last id": ("greedy_token", _greedy_last_maximum),
    "q4 nibbles high first": ("unpack_q4", _unpack_q4_high_first),
    "q4 groups of 32": ("dequantize_q4", _dequantize_q4_group_32),
    "q4 bias dropped": ("dequantize_q4", _dequantize_q4_no_bias),
    "sections ordered T, H, W": ("mrope_section_layout", _sections_t_first),
    "sections without the frequency permutation": ("mrope_section_layout", _sections_unpermuted),
    "image advances positions by t only": ("mrope_positions", _edited(
        "mrope_positions", ("st += max(t, gh, gw)", "st += t"))),
    "rope_delta without the + 1": ("mrope_positions", _edited(
        "mrope_positions", ("delta[b] = st - L", "delta[b] = st - 1 - L"))),
    "image h and w axes swapped": ("mrope_positions", _edited(
        "mrope_positions", ("pos[1, b, l + r] = st + (r // gw) % gh", "pos[1, b, l + r] = st + r % gw"),
        ("pos[2, b, l + r] = st + r % gw", "pos[2, b, l + r] = st + (r // gw) % gh"))),
    "full layers at i % 4 == 0": ("layer_kind", _edited("layer_kind", ("i % 4 == 3", "i % 4 == 0"))),
    "logit scale dropped": ("logits", _edited("logits", ("* float(logit_scale)", "* 1.0"))),
    "deepstack rows shifted by one": ("layer_prefill", _edited(
        "layer_prefill", ("flat[np.asarray(ds_rows)] +=", "flat[np.asarray(ds_rows) + 1] +="))),
    "row sampler key span starts one late": ("layer_prefill_rows", _edited(
        "layer_prefill_rows", ("int(rows.min()) - shape.window + 1", "int(rows.min()) - shape.window + 2"))),
    "row sampler keys not offset by the span start": ("layer_prefill_rows", _edited(
        "layer_prefill_rows", ("k_index=span)", "k_index=span - lo)"))),
    "varlen sequences see each other": ("layer_prefill_varlen", _varlen_sequences_see_each_other),
    "varlen cache start ignored": ("layer_prefill_varlen", _varlen_start_ignored),
    "deepstack after every layer": ("stack_prefill", _edited(
        "stack_prefill", ("i < 3 and i < len(ds)", "i < len(ds)"))),
}

PINS = [
    P.test_split_rope_layout_page_example,
    P.test_axis_sets_page_example,
    lambda: P.test_mrope_equals_1d_rope_when_axes_agree(64, (12, 10, 10)),
    P.test_single_axis_probe_rotates_only_that_axis,
    P.test_layer_norm_vs_torch_and_invariants,
    lambda: P.test_attention_vs_sdpa_and_brute_force("sliding", 3, 9),
    lambda: P.test_attention_vs_sdpa_and_brute_force("full", 0, 9),
    lambda: P.test_parallel_block_vs_library_routines("sliding", 3, 5),
    lambda: P.test_parallel_block_vs_library_routines("full", 0, 5),
    P.test_logits_vs_library_and_scale,
    lambda: P.test_chunked_prefill_equals_one_prefill("sliding", 3),
    lambda: P.test_chunked_prefill_equals_one_prefill("full", 0),
    P.test_greedy_generation_equals_full_recompute,
    P.test_embed_front_end,
    P.test_greedy_token_is_first_maximum,
    P.test_q4_format_from_page_and_nibble_example,
    P.test_q4_dequantize_brute_force_and_closed_forms,
    P.test_q4_round_trip_within_half_step,
    P.test_q4_decode_is_dense_decode_of_dequantized_weights,
    P.test_sections_layout_carries_the_page_axis_sets,
    P.test_sections_rope_is_a_pair_permutation_of_the_interleave,
    P.test_sections_with_equal_axes_is_1d_rope_on_permuted_frequencies,
    P.test_sections_layer_equals_interleaved_layer_with_permuted_qk_rows,
    P.test_positions_image_448_page_example,
    P.test_positions_c1_layout_hand_derived,
    P.test_positions_video_like_and_multi_image,
    P.test_layer_pattern_page_example,
    P.test_deepstack_adds_at_rows_only,
    P.test_stack_deepstack_first_three_layers_only,
    P.test_prefill_decode_consistency,
    lambda: P.test_layer_prefill_rows_equals_whole_prefill("sliding", 3, 1, 0, [0, 1, 5, 9, 16]),
    lambda: P.test_layer_prefill_rows_equals_whole_prefill("sliding", 3, 2, 1, [16, 2, 9, 6]),
    lambda: P.test_layer_prefill_rows_equals_whole_prefill("sliding", 3, 1, 0, [3, 4, 11, 12]),
    P.test_varlen_equal_lengths_equals_batched_prefill,
    lambda: P.test_varlen_each_sequence_is_its_own_prefill("sliding", 3),
    P.test_varlen_continues_each_sequence_cache,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    assert _some_pin_fails(), f"no pin caught the planted mistake: {name}"


def test_pins_pass_on_unmutated_oracle():
    assert not _some_pin_fails()
