"""Shared plumbing for the GPU parity tests: seeded inputs as torch tensors, calls
through the C ABI (ctypes binding), and the error metrics the gates use."""
from __future__ import annotations

import numpy as np
import torch

from synth import bf16_round
from synth.workloads import LayerShape

DEV = "cuda"


def B():
    from cohere2_block_mrope_amd import binding
    return binding


def tdtype(shape: LayerShape):
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def cdtype(shape: LayerShape) -> int:
    return 1 if shape.dtype == "bf16" else 0


def desc(shape: LayerShape, ln_fuse: int = 0):
    b = B()
    return b.make_desc(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.intermediate,
                       b.COMPASS_SLIDING if shape.kind == "sliding" else b.COMPASS_FULL,
                       shape.window if shape.kind == "sliding" else 0, shape.mrope_section, shape.rope_theta,
                       shape.ln_eps, cdtype(shape),
                       b.COMPASS_ROPE_SECTIONS if shape.rope_layout == "sections" else b.COMPASS_ROPE_INTERLEAVED,
                       ln_fuse)


def to_dev(a: np.ndarray, dtype) -> torch.Tensor:
    """Exact transfer: bf16 inputs are already bf16-representable fp32 values."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def weights_to_dev(shape: LayerShape, w: dict) -> dict:
    return {k: to_dev(v, tdtype(shape)) for k, v in w.items()}


def ints_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def workspace(nbytes: int) -> torch.Tensor:
    # 256-byte aligned (the caching allocator aligns to at least 512 bytes).
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)


def run_prefill(shape: LayerShape, wdev: dict, x: torch.Tensor, pos, kv=None, ds_rows=None, ds=None,
                out=None, stream=None):
    b = B()
    d = desc(shape)
    Bn, L = x.shape[0], x.shape[1]
    ws = workspace(b.compass_workspace_size(d, Bn, L, 0, 0))
    out = torch.empty_like(x) if out is None else out
    kvs = None if kv is None else b.make_kv(kv[0], kv[1])
    b.compass_layer_prefill(d, b.make_weights(wdev), x, pos, kvs, ds_rows, ds, out, ws, stream)
    return out


def run_prefill_chunk(shape: LayerShape, wdev: dict, x: torch.Tensor, pos, kc, vc, lens, ds_rows=None, ds=None,
                      out=None, stream=None):
    b = B()
    d = desc(shape)
    Bn, L = x.shape[0], x.shape[1]
    ws = workspace(b.compass_workspace_size(d, Bn, L, 0, 0))
    out = torch.empty_like(x) if out is None else out
    b.compass_layer_prefill_chunk(d, b.make_weights(wdev), x, pos, b.make_kv(kc, vc, lens), ds_rows, ds, out, ws,
                                  stream)
    return out


def run_decode(shape: LayerShape, wdev: dict, x: torch.Tensor, pos, kc, vc, lens, out=None, stream=None):
    b = B()
    d = desc(shape)
    Bn = x.shape[0]
    ws = workspace(b.compass_workspace_size(d, Bn, 1, kc.shape[2], 1))
    out = torch.empty_like(x) if out is None else out
    b.compass_layer_decode(d, b.make_weights(wdev), x, pos, b.make_kv(kc, vc, lens), out, ws, stream)
    return out


def q4_to_dev(wq4: dict) -> dict:
    """4-bit weights (codes uint8, bf16-exact scales / biases) as device tensors."""
    out = {"ln_w": to_dev(wq4["ln_w"], torch.bfloat16)}
    for k, v in wq4.items():
        if k != "ln_w":
            q, sc, bi = v
            out[k] = (torch.from_numpy(np.ascontiguousarray(q)).to(DEV), to_dev(sc, torch.bfloat16),
                      to_dev(bi, torch.bfloat16))
    return out


def run_decode_q4(shape: LayerShape, wq4dev: dict, x: torch.Tensor, pos, kc, vc, lens, out=None, stream=None):
    b = B()
    d = desc(shape)
    Bn = x.shape[0]
    ws = workspace(b.compass_workspace_size(d, Bn, 1, kc.shape[2], 1))
    out = torch.empty_like(x) if out is None else out
    b.compass_layer_decode_q4(d, b.make_weights_q4(wq4dev), x, pos, b.make_kv(kc, vc, lens), out, ws, stream)
    return out


def run_logits(h: torch.Tensor, norm_w, eps: float, embed, scale: float, dtype: int, logits=None):
    b = B()
    R, D = h.shape
    ws = workspace(b.compass_logits_workspace_size(R, D, dtype))
    logits = torch.empty(R, embed.shape[0], dtype=torch.float32, device=DEV) if logits is None else logits
    b.compass_logits(h, norm_w, eps, embed, scale, logits, ws, dtype)
    return logits


def np64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the compared set."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def tol(shape: LayerShape) -> float:
    """Gates: 2e-2 for bf16 storage, 1e-4 for fp32."""
    return 2e-2 if shape.dtype == "bf16" else 1e-4


def small_shape(dtype="bf16", kind="sliding", hd=128, Hq=4, Hkv=1, D=256, I=512, window=48, section=None):
    if section is None:
        section = (24, 20, 20) if hd == 128 else (12, 10, 10)
    return LayerShape(hidden=D, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=hd, intermediate=I, kind=kind,
                      window=window, mrope_section=section, dtype=dtype)


def rand_np(seed: int, shape_tuple, std=1.0, mean=0.0, bf16=True) -> np.ndarray:
    from synth import normal
    v = normal(seed, int(np.prod(shape_tuple)), std=std, mean=mean).reshape(shape_tuple)
    return bf16_round(v) if bf16 else v


# Attention probe: a layer with Wo = 64 I and w_down = 0 (needs Hq * hd == D) returns
# out = x + 64 o, which exposes the attention output o alone through the layer call.
PROBE_SCALE = 64.0


def probe_weights(shape: LayerShape, w: dict) -> dict:
    """The attention-probe layer's weights: w with Wo = 64 I and w_down = 0."""
    D = shape.hidden
    assert shape.n_q_heads * shape.head_dim == D, "the probe needs Hq * hd == hidden"
    p = dict(w)
    p["wo"] = (PROBE_SCALE * np.eye(D)).astype(np.float32)
    p["w_down"] = np.zeros_like(w["w_down"])
    return p


def check_attn_rows(shape: LayerShape, out_probe, x, o_ref, what: str = "") -> float:
    """Row-wise gate on the attention output: (out - x) of the probe layer against 64 o of
    the oracle, each row on its own scale, allowing the storage rounding of out."""
    g = np64(out_probe).reshape(-1, shape.hidden) if isinstance(out_probe, torch.Tensor) \
        else np.asarray(out_probe, np.float64).reshape(-1, shape.hidden)
    xr = np.asarray(x, np.float64).reshape(-1, shape.hidden)
    d_ref = PROBE_SCALE * np.asarray(o_ref, np.float64).reshape(-1, shape.hidden)
    ulp = 2.0 ** -8 if shape.dtype == "bf16" else 2.0 ** -23
    excess = np.abs((g - xr) - d_ref) - ulp * np.abs(xr + d_ref)
    per_row = np.max(excess, axis=1) / np.max(np.abs(d_ref), axis=1)
    worst = int(np.argmax(per_row))
    assert per_row[worst] <= tol(shape), f"{what}: attention row {worst} rel err {per_row[worst]:.3e}"
    return float(per_row[worst])
