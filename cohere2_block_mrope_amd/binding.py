"""ctypes binding of libcompass (include/compass.h): argument marshalling only.

Every function has the name of the C entry point it calls. Tensors are torch
tensors on the GPU; only their data pointers and the current HIP stream are
passed down. Errors from the library raise CompassError with the library's
message. There is no fallback: if libcompass.so is missing, importing this
module raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcompass.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")

_lib = ctypes.CDLL(LIB_PATH)

COMPASS_OK = 0
COMPASS_E_INVALID = -1
COMPASS_E_UNSUPPORTED = -2
COMPASS_E_ALIGN = -3
COMPASS_E_WORKSPACE = -4
COMPASS_E_DEVICE = -5
COMPASS_F32 = 0
COMPASS_BF16 = 1
COMPASS_SLIDING = 0
COMPASS_FULL = 1
COMPASS_ROPE_INTERLEAVED = 0
COMPASS_ROPE_SECTIONS = 1
POS_OK, POS_SPAN_MISMATCH, POS_EXTRA_PADS, POS_UNUSED_IMAGES, POS_BAD_GRID, POS_TOO_MANY_IMAGES = range(6)


class CompassError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"compass error {code}: {msg}")
        self.code = code


class compass_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("window", ctypes.c_int32), ("mrope_section", ctypes.c_int32 * 3), ("rope_theta", ctypes.c_float),
                ("ln_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("rope_layout", ctypes.c_int32),
                ("ln_fuse", ctypes.c_int32)]


class compass_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]


class compass_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("lens", ctypes.c_void_p)]


class compass_q4_matrix(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class compass_layer_weights_q4(ctypes.Structure):
    _fields_ = [("ln_w", ctypes.c_void_p)] + [(n, compass_q4_matrix) for n in
                                              ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_sig = {
    "compass_mrope_positions": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P]),
    "compass_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(compass_layer_desc), _I, _I, _I, _I]),
    "compass_layer_prefill": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc), ctypes.POINTER(compass_layer_weights),
                                             _I, _I, _P, _P, ctypes.POINTER(compass_kv), _P, _P, _I, _P, _P,
                                             ctypes.c_size_t, _P]),
    "compass_layer_prefill_chunk": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc),
                                                   ctypes.POINTER(compass_layer_weights), _I, _I, _P, _P,
                                                   ctypes.POINTER(compass_kv), _P, _P, _I, _P, _P,
                                                   ctypes.c_size_t, _P]),
    "compass_varlen_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(compass_layer_desc), _I, _I]),
    "compass_layer_prefill_varlen": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc),
                                                    ctypes.POINTER(compass_layer_weights), _I, _I, _P, _P, _P,
                                                    ctypes.POINTER(compass_kv), _P, _P, _I, _P, _P, _P,
                                                    ctypes.c_size_t, _P]),
    "compass_layer_decode": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc), ctypes.POINTER(compass_layer_weights),
                                            _I, _P, _P, ctypes.POINTER(compass_kv), _P, _P, ctypes.c_size_t, _P]),
    "compass_layer_decode_chained": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc),
                                                    ctypes.POINTER(compass_layer_weights), _I, _P, _P, _P,
                                                    ctypes.POINTER(compass_kv), _P, _P, ctypes.c_float, _P, _P,
                                                    ctypes.c_size_t, _P]),
    "compass_layer_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc),
                                                    ctypes.POINTER(compass_layer_weights), _I, _P, _P,
                                                    ctypes.POINTER(compass_kv), _P, _P]),
    "compass_layer_decode_q4": (ctypes.c_int, [ctypes.POINTER(compass_layer_desc),
                                               ctypes.POINTER(compass_layer_weights_q4), _I, _P, _P,
                                               ctypes.POINTER(compass_kv), _P, _P, ctypes.c_size_t, _P]),
    "compass_logits_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "compass_logits": (ctypes.c_int, [_I, _I, _I, _I, _P, _P, ctypes.c_float, _P, ctypes.c_float, _P, _P,
                                      ctypes.c_size_t, _P]),
    "compass_embed": (ctypes.c_int, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P]),
    "compass_decode_positions": (ctypes.c_int, [_I, _P, _P, _I, _P, _P]),
    "compass_logits_argmax_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "compass_logits_argmax": (ctypes.c_int, [_I, _I, _I, _I, _P, ctypes.c_int64, _P, ctypes.c_float, _P,
                                             ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "compass_last_error": (ctypes.c_char_p, []),
    "compass_version": (ctypes.c_char_p, []),
    "compass_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "compass_profile_reset": (ctypes.c_int, []),
    "compass_profile_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                            ctypes.POINTER(ctypes.c_double)]),
    "compass_profile_kernel_name": (ctypes.c_char_p, [_I]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


def _check(rc: int) -> None:
    if rc != COMPASS_OK:
        raise CompassError(rc, _lib.compass_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_desc(hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int, intermediate: int, kind: int,
              window: int, mrope_section, rope_theta: float, ln_eps: float, dtype: int,
              rope_layout: int = COMPASS_ROPE_INTERLEAVED, ln_fuse: int = 0) -> compass_layer_desc:
    d = compass_layer_desc()
    d.rope_layout = rope_layout
    d.ln_fuse = ln_fuse
    d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.intermediate = hidden, n_q_heads, n_kv_heads, head_dim, intermediate
    d.kind, d.window = kind, window
    d.mrope_section[:] = list(mrope_section)
    d.rope_theta, d.ln_eps, d.dtype = rope_theta, ln_eps, dtype
    return d


def make_weights(w: dict) -> compass_layer_weights:
    s = compass_layer_weights()
    for name, _ in compass_layer_weights._fields_:
        setattr(s, name, _ptr(w[name]))
    return s


def make_weights_q4(w: dict) -> compass_layer_weights_q4:
    """w: ln_w tensor, and for each matrix name a (codes, scales, biases) tuple of tensors."""
    s = compass_layer_weights_q4()
    s.ln_w = _ptr(w["ln_w"])
    for name, _ in compass_layer_weights_q4._fields_[1:]:
        q, sc, bi = w[name]
        setattr(s, name, compass_q4_matrix(_ptr(q), _ptr(sc), _ptr(bi)))
    return s


def make_kv(k, v, lens=None) -> compass_kv:
    s = compass_kv()
    s.k, s.v = _ptr(k), _ptr(v)
    s.capacity = k.shape[2]
    s.lens = _ptr(lens)
    return s


def compass_last_error() -> str:
    return _lib.compass_last_error().decode()


def compass_version() -> str:
    return _lib.compass_version().decode()


def compass_mrope_positions(token_ids, image_token_id: int, grid_thw, img_offset, spatial_merge: int,
                            pos, rope_delta, status, stream=None) -> None:
    B, L = token_ids.shape
    _check(_lib.compass_mrope_positions(_ptr(token_ids), B, L, image_token_id, _ptr(grid_thw), _ptr(img_offset),
                                        spatial_merge, _ptr(pos), _ptr(rope_delta), _ptr(status), _stream(stream)))


def compass_workspace_size(desc: compass_layer_desc, B: int, L: int, capacity: int = 0, decode: int = 0) -> int:
    return int(_lib.compass_workspace_size(ctypes.byref(desc), B, L, capacity, decode))


def compass_layer_prefill(desc, weights: compass_layer_weights, x, pos, kv: Optional[compass_kv], ds_rows, ds,
                          out, workspace, stream=None) -> None:
    B, L = x.shape[0], x.shape[1]
    n_ds = 0 if ds_rows is None else int(ds_rows.numel())
    _check(_lib.compass_layer_prefill(ctypes.byref(desc), ctypes.byref(weights), B, L, _ptr(x), _ptr(pos),
                                      None if kv is None else ctypes.byref(kv), _ptr(ds_rows), _ptr(ds), n_ds,
                                      _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


def compass_layer_prefill_chunk(desc, weights: compass_layer_weights, x, pos, kv: compass_kv, ds_rows, ds,
                                out, workspace, stream=None) -> None:
    B, L = x.shape[0], x.shape[1]
    n_ds = 0 if ds_rows is None else int(ds_rows.numel())
    _check(_lib.compass_layer_prefill_chunk(ctypes.byref(desc), ctypes.byref(weights), B, L, _ptr(x), _ptr(pos),
                                            ctypes.byref(kv), _ptr(ds_rows), _ptr(ds), n_ds, _ptr(out),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))


def compass_varlen_workspace_size(desc, n_seq: int, T: int) -> int:
    return int(_lib.compass_varlen_workspace_size(ctypes.byref(desc), n_seq, T))


def compass_layer_prefill_varlen(desc, weights: compass_layer_weights, cu_seqlens, x, pos, kv: Optional[compass_kv],
                                 ds_rows, ds, out, status, workspace, stream=None) -> None:
    """x [T, D] packed rows; cu_seqlens int32 [n_seq + 1] on the device."""
    T = x.shape[0]
    n_seq = cu_seqlens.shape[0] - 1
    n_ds = 0 if ds_rows is None else int(ds_rows.numel())
    _check(_lib.compass_layer_prefill_varlen(ctypes.byref(desc), ctypes.byref(weights), n_seq, T, _ptr(cu_seqlens),
                                             _ptr(x), _ptr(pos), None if kv is None else ctypes.byref(kv),
                                             _ptr(ds_rows), _ptr(ds), n_ds, _ptr(out), _ptr(status), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))


def compass_layer_decode(desc, weights: compass_layer_weights, x, pos, kv: compass_kv, out, workspace,
                         stream=None) -> None:
    B = x.shape[0]
    _check(_lib.compass_layer_decode(ctypes.byref(desc), ctypes.byref(weights), B, _ptr(x), _ptr(pos),
                                     ctypes.byref(kv), _ptr(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def compass_layer_decode_chained(desc, weights: compass_layer_weights, x, x_norm, pos, kv: compass_kv, out,
                                 next_ln_w, next_ln_eps: float, out_norm, workspace, stream=None) -> None:
    B = x.shape[0]
    _check(_lib.compass_layer_decode_chained(ctypes.byref(desc), ctypes.byref(weights), B, _ptr(x), _ptr(x_norm),
                                             _ptr(pos), ctypes.byref(kv), _ptr(out), _ptr(next_ln_w),
                                             float(next_ln_eps), _ptr(out_norm), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream)))


COMPASS_NOALLOC_SCRATCH_BYTES = 64 << 20


def compass_layer_decode_noalloc(desc, weights: compass_layer_weights, x, pos, kv: compass_kv, out,
                                 stream=None) -> None:
    B = x.shape[0]
    _check(_lib.compass_layer_decode_noalloc(ctypes.byref(desc), ctypes.byref(weights), B, _ptr(x), _ptr(pos),
                                             ctypes.byref(kv), _ptr(out), _stream(stream)))


def compass_layer_decode_q4(desc, weights: compass_layer_weights_q4, x, pos, kv: compass_kv, out, workspace,
                            stream=None) -> None:
    B = x.shape[0]
    _check(_lib.compass_layer_decode_q4(ctypes.byref(desc), ctypes.byref(weights), B, _ptr(x), _ptr(pos),
                                        ctypes.byref(kv), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def compass_logits_workspace_size(R: int, D: int, dtype: int) -> int:
    return int(_lib.compass_logits_workspace_size(R, D, dtype))


def compass_logits(h, norm_w, ln_eps: float, embed, logit_scale: float, logits, workspace, dtype: int,
                   stream=None) -> None:
    R, D = h.shape
    V = embed.shape[0]
    _check(_lib.compass_logits(R, D, V, dtype, _ptr(h), _ptr(norm_w), ln_eps, _ptr(embed), logit_scale,
                               _ptr(logits), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)))


def compass_embed(tokens, embed, img_rows, img_feats, h, status, dtype: int, stream=None) -> None:
    """tokens [R] int32, embed [V, D], img_rows [n_img] int32 or None, img_feats [n_img, D], h out [R, D]."""
    R = int(tokens.numel())
    V, D = embed.shape
    n_img = 0 if img_rows is None else int(img_rows.numel())
    _check(_lib.compass_embed(R, D, V, dtype, _ptr(tokens), _ptr(embed), _ptr(img_rows), _ptr(img_feats), n_img,
                              _ptr(h), _ptr(status), _stream(stream)))


def compass_decode_positions(lens, rope_delta, advance: int, pos, stream=None) -> None:
    """lens [B] int32 (updated in place), rope_delta [B] int32 or None, pos out [3, B] int32."""
    B = int(lens.numel())
    _check(_lib.compass_decode_positions(B, _ptr(lens), _ptr(rope_delta), advance, _ptr(pos), _stream(stream)))


def compass_logits_argmax_workspace_size(R: int, D: int, V: int, dtype: int) -> int:
    return int(_lib.compass_logits_argmax_workspace_size(R, D, V, dtype))


def compass_logits_argmax(h, norm_w, ln_eps: float, embed, logit_scale: float, token, max_logit, workspace,
                          dtype: int, stream=None) -> None:
    """h [R, D] with unit column stride (rows may be strided, e.g. x[:, -1] of [B, L, D])."""
    R, D = h.shape
    if R > 1 and h.stride(1) != 1:
        raise ValueError("h must have unit column stride")
    V = embed.shape[0]
    _check(_lib.compass_logits_argmax(R, D, V, dtype, _ptr(h), h.stride(0) if R > 1 else D, _ptr(norm_w), ln_eps,
                                      _ptr(embed), logit_scale, _ptr(token), _ptr(max_logit), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))


def compass_profile_enable(on: bool) -> None:
    _check(_lib.compass_profile_enable(1 if on else 0))


def compass_profile_reset() -> None:
    _check(_lib.compass_profile_reset())


def compass_profile_read(kernel: Optional[str] = None):
    """(launch count, summed milliseconds) of the recorded launches named `kernel` (all if None)."""
    c = ctypes.c_int64()
    t = ctypes.c_double()
    _check(_lib.compass_profile_read(None if kernel is None else kernel.encode(), ctypes.byref(c), ctypes.byref(t)))
    return int(c.value), float(t.value)


def compass_profile_kernel_names():
    names, i = [], 0
    while True:
        n = _lib.compass_profile_kernel_name(i)
        if n is None:
            return names
        names.append(n.decode())
        i += 1
