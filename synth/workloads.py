"""Workload shapes and seeded tensors for the decoder-layer parity cases and the bench.

Widths follow the Compass text decoder described on the mlxcel Compass issue
("Text decoder forward": hidden 2048, head_dim 128, MRoPE section [24, 20, 20],
base 50000). Value distributions: linear and embedding weights ~ N(0, 0.02);
LayerNorm weights 1 + N(0, 0.02); hidden states, KV caches and deepstack rows
~ N(0, 1). Token ids are uniform over ordinary ids; image-pad runs are laid out
as the position-id rule expects (t * (h/2) * (w/2) pads per image).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

from .rng import normal, bf16_round, stream_seed, splitmix64

IMAGE_TOKEN_ID = 255031
VISION_START_ID = 255028
VISION_END_ID = 255029


class TensorId:
    LN_W = 1
    WQ = 2
    WK = 3
    WV = 4
    WO = 5
    WG = 6
    WU = 7
    WD = 8
    X = 9
    K_CACHE = 10
    V_CACHE = 11
    DS = 12  # + deepstack index (0..2)
    FINAL_LN = 20
    EMBED = 21
    TOKENS = 22
    PERM = 23


@dataclasses.dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    kind: str  # "sliding" | "full"
    window: int
    mrope_section: tuple
    dtype: str  # "f32" | "bf16"
    rope_theta: float = 50000.0
    ln_eps: float = 1e-5
    rope_layout: str = "interleaved"  # "interleaved" | "sections"

    def with_kind(self, kind: str) -> "LayerShape":
        return dataclasses.replace(self, kind=kind)


def _compass(kind: str, window: int) -> LayerShape:
    return LayerShape(hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, intermediate=8192,
                      kind=kind, window=window, mrope_section=(24, 20, 20), dtype="bf16")


class Stream:
    """Seed-stream ids (the `workload` argument of stream_seed) of the named workloads."""
    TINY_SLIDING_F32 = 0
    SLIDING_PREFILL = 1
    FULL_PREFILL = 2
    DECODE_STACK = 3
    STACK_LOGITS = 4


# The workloads, by name: the small fp32 parity case; the sliding-layer prefill the headline
# throughput is quoted on; the full-attention prefill; batched decode over a 4-layer stack;
# the 4-layer stack prefill with deepstack and logits. `stream` seeds each one's inputs.
WORKLOADS: Dict[str, dict] = {
    "tiny_sliding_f32": dict(stream=Stream.TINY_SLIDING_F32, name="tiny sliding layer fp32 (D=256, 4/1 heads, hd=64, I=1024, W=32, L=128)",
            shape=LayerShape(hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64, intermediate=1024,
                             kind="sliding", window=32, mrope_section=(12, 10, 10), dtype="f32"),
            B=1, L=128, layers=1),
    "sliding_prefill": dict(stream=Stream.SLIDING_PREFILL, name="sliding-layer prefill bf16 (D=2048, 16/4 heads, hd=128, I=8192, W=1024, L=4096 = 64 text + 1024 image + 3008 text)",
            shape=_compass("sliding", 1024), B=1, L=4096, layers=1),
    "full_prefill": dict(stream=Stream.FULL_PREFILL, name="full-attention prefill bf16 (D=2048, 16/4 heads, NoPE, causal, B=2, L=8192)",
            shape=_compass("full", 0), B=2, L=8192, layers=1),
    "decode_stack": dict(stream=Stream.DECODE_STACK, name="batched decode bf16, 4-layer 3:1 stack, B=64, KV cache 8192, W=4096",
            shape=_compass("sliding", 4096), B=64, L=1, layers=4, cache_len=8192),
    "stack_logits": dict(stream=Stream.STACK_LOGITS, name="4-layer 3:1 stack prefill bf16, L=4096 mixed image+text, deepstack x3, tied 256000-vocab logits x 0.0625",
            shape=_compass("sliding", 1024), B=1, L=4096, layers=4, vocab=256000, logit_scale=0.0625),
}


def _uniform_ints(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        idx = np.arange(n, dtype=np.uint64)
        z = np.uint64(seed) + (idx + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return (lo + (z % np.uint64(hi - lo))).astype(np.int32)


def text_tokens(seed: int, n: int) -> np.ndarray:
    """Ordinary token ids (never the image-pad id)."""
    return _uniform_ints(seed, n, 1, 255000)


def image_text_row(seed: int, L: int = 4096, n_text_before: int = 64, grid=(1, 64, 64), merge: int = 2):
    """One row: text, one image-pad span for `grid` (patch units), then text up to L.

    Returns (tokens [1, L] int32, grid_thw [1, 3] int32, img_offset [2] int32).
    """
    t, h, w = grid
    n_img = t * (h // merge) * (w // merge)
    n_after = L - n_text_before - n_img
    assert n_after >= 0
    tok = text_tokens(seed, L).copy()
    tok[n_text_before - 1] = VISION_START_ID
    tok[n_text_before:n_text_before + n_img] = IMAGE_TOKEN_ID
    if n_after > 0:
        tok[n_text_before + n_img] = VISION_END_ID
    return (tok.reshape(1, L), np.array([grid], dtype=np.int32), np.array([0, 1], dtype=np.int32))


def permutation(seed: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of arange(n) driven by SplitMix64 outputs."""
    r = _uniform_ints(seed, n, 0, 1 << 62).astype(np.int64)
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int(r[i] % (i + 1))
        p[i], p[j] = p[j], p[i]
    return p


def _store(shape: LayerShape, v: np.ndarray) -> np.ndarray:
    return bf16_round(v) if shape.dtype == "bf16" else v.astype(np.float32)


def make_layer_weights(shape: LayerShape, workload: int, layer: int) -> Dict[str, np.ndarray]:
    """nn.Linear-layout weights [out, in] as fp32 arrays (bf16-exact values for bf16 shapes)."""
    D, Hq, Hkv, hd, I = shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.intermediate
    specs = [("ln_w", TensorId.LN_W, (D,)), ("wq", TensorId.WQ, (Hq * hd, D)), ("wk", TensorId.WK, (Hkv * hd, D)),
             ("wv", TensorId.WV, (Hkv * hd, D)), ("wo", TensorId.WO, (D, Hq * hd)), ("w_gate", TensorId.WG, (I, D)),
             ("w_up", TensorId.WU, (I, D)), ("w_down", TensorId.WD, (D, I))]
    out = {}
    for name, tid, shp in specs:
        n = int(np.prod(shp))
        seed = stream_seed(workload, layer, tid)
        if name == "ln_w":
            v = normal(seed, n, std=0.02, mean=1.0)
        else:
            v = normal(seed, n, std=0.02)
        out[name] = _store(shape, v).reshape(shp)
    return out


Q4_STREAM = 100  # tensor-id offset of the scale (+100) and bias (+200) streams of 4-bit weights


def make_layer_weights_q4(shape: LayerShape, workload: int, layer: int) -> Dict[str, object]:
    """4-bit affine weights in their stored form: ln_w as make_layer_weights, and per matrix
    [out, in] a tuple (codes uint8 [out, in / 2] of uniform random bytes, scales [out, in / 64],
    biases [out, in / 64]), scales |N(0.0067, 0.0012)| and biases -7.5 * scale + N(0, 0.002),
    both bf16-exact, so that the weights they stand for spread like the dense N(0, 0.02) ones."""
    D, Hq, Hkv, hd, I = shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.intermediate
    specs = [("wq", TensorId.WQ, (Hq * hd, D)), ("wk", TensorId.WK, (Hkv * hd, D)),
             ("wv", TensorId.WV, (Hkv * hd, D)), ("wo", TensorId.WO, (D, Hq * hd)), ("w_gate", TensorId.WG, (I, D)),
             ("w_up", TensorId.WU, (I, D)), ("w_down", TensorId.WD, (D, I))]
    out = {"ln_w": bf16_round(normal(stream_seed(workload, layer, TensorId.LN_W), D, std=0.02, mean=1.0))}
    for name, tid, (rows, cols) in specs:
        assert cols % 64 == 0
        codes = _uniform_ints(stream_seed(workload, layer, tid), rows * cols // 2, 0, 256).astype(np.uint8)
        ng = rows * (cols // 64)
        scale = bf16_round(np.abs(normal(stream_seed(workload, layer, tid + Q4_STREAM), ng, std=0.0012,
                                         mean=0.0067)))
        bias = bf16_round(-7.5 * scale + normal(stream_seed(workload, layer, tid + 2 * Q4_STREAM), ng, std=0.002))
        out[name] = (codes.reshape(rows, cols // 2), scale.reshape(rows, cols // 64),
                     bias.reshape(rows, cols // 64))
    return out


def make_layer_input(shape: LayerShape, workload: int, rows: int, tensor_id: int = TensorId.X,
                     layer: int = 0, std: float = 1.0) -> np.ndarray:
    """[rows, D] N(0, std^2) hidden states (bf16-exact for bf16 shapes)."""
    v = normal(stream_seed(workload, layer, tensor_id), rows * shape.hidden, std=std)
    return _store(shape, v).reshape(rows, shape.hidden)


def make_tensor(shape: LayerShape, workload: int, layer: int, tensor_id: int, dims, std=1.0, mean=0.0):
    n = int(np.prod(dims))
    v = normal(stream_seed(workload, layer, tensor_id), n, std=std, mean=mean)
    return _store(shape, v).reshape(dims)
