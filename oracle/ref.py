"""ctypes loader of the plain fp32 C++ reference (oracle/compass_ref.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the tests use it as a second,
independent oracle next to the fp64 numpy one. build() compiles it with g++.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "compass_ref.cpp")
LIB = os.path.join(HERE, "libcompass_ref.so")


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["g++", "-O2", "-std=c++17", "-fopenmp", "-shared", "-fPIC", "-o", tmp, SRC], check=True)
    os.replace(tmp, LIB)
    return LIB


class cref_shape(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("hd", ctypes.c_int32),
                ("I", ctypes.c_int32), ("sliding", ctypes.c_int32), ("window", ctypes.c_int32),
                ("section", ctypes.c_int32 * 3), ("theta", ctypes.c_float), ("eps", ctypes.c_float),
                ("layout", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
    return _lib


def num_threads() -> int:
    """Threads the reference's parallel loops use."""
    return int(lib().cref_num_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shape(shape) -> cref_shape:
    s = cref_shape()
    s.D, s.Hq, s.Hkv, s.hd, s.I = shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.intermediate
    s.sliding = 1 if shape.kind == "sliding" else 0
    s.window = shape.window
    s.section[:] = list(shape.mrope_section)
    s.theta, s.eps = shape.rope_theta, shape.ln_eps
    s.layout = 1 if getattr(shape, "rope_layout", "interleaved") == "sections" else 0
    return s


WEIGHTS = ("ln_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def mrope_positions(tokens, image_token_id, grid, img_offset, merge):
    """Returns (code, pos [3, B, L], delta [B])."""
    tok = _i32(tokens)
    B, L = tok.shape
    pos = np.zeros((3, B, L), np.int32)
    delta = np.zeros(B, np.int32)
    code = lib().cref_mrope_positions(_p(tok), B, L, int(image_token_id), _p(_i32(grid)), _p(_i32(img_offset)),
                                      int(merge), _p(pos), _p(delta))
    return code, pos, delta


def layer_forward(shape, w, x, pos, k_cache=None, v_cache=None, start=None, ds_rows=None, ds=None):
    """x [B, L, D] -> (out [B, L, D], k_new, v_new [B, Hkv, L, hd]) in fp32."""
    x = _f32(x)
    B, L, D = x.shape
    ws = [_f32(w[n]) for n in WEIGHTS]
    warr = (ctypes.c_void_p * 8)(*[a.ctypes.data for a in ws])
    posa = _i32(pos if pos is not None else np.zeros((3, B, L)))
    kc = None if k_cache is None else _f32(k_cache)
    vc = None if v_cache is None else _f32(v_cache)
    cap = 0 if kc is None else kc.shape[2]
    st = None if start is None else _i32(start)
    dr = None if ds_rows is None else _i32(ds_rows)
    dsa = None if ds is None else _f32(ds)
    out = np.zeros_like(x)
    kn = np.zeros((B, shape.n_kv_heads, L, shape.head_dim), np.float32)
    vn = np.zeros_like(kn)
    s = _shape(shape)
    lib().cref_layer_forward(ctypes.byref(s), warr, B, L, _p(x), _p(posa), _p(kc), _p(vc), cap, _p(st), _p(dr),
                             _p(dsa), 0 if dr is None else len(dr), _p(out), _p(kn), _p(vn))
    return out, kn, vn


def logits(h, norm_w, eps, embed, scale):
    h, E = _f32(h), _f32(embed)
    R, D = h.shape
    V = E.shape[0]
    out = np.zeros((R, V), np.float32)
    lib().cref_logits(R, D, V, _p(h), _p(_f32(norm_w)), ctypes.c_float(eps), _p(E), ctypes.c_float(scale), _p(out))
    return out
