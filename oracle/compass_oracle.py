"""Plain fp64 CPU oracle for the Compass/Cohere2 parallel decoder layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the bench's CPU-baseline leg
use it. It shares no code with the HIP library.

Every function is the plain definition written out in float64 (integers for
position ids), following the mlxcel issue "feat(vlm): add Cohere Compass /
North-Micro-Vision (cohere_compass) VLM" (page 1), section "Text decoder
forward" and its "Interleaved MRoPE" and "Position ids" paragraphs, plus the
"Validation" list of the same page. Library primitives used as steps: numpy
matmul, exp, sqrt, cos, sin. No tiling, fusion or reordering beyond what the
definitions state; rows of a softmax are independent by definition and may be
processed in any grouping.

Readings taken where the page is silent (each one is listed with its reason in
the design notes of the repository):
  * LayerNorm: mean-centred, biased variance, weight only, eps passed in.
  * MRoPE axis rule for sections other than [24, 20, 20]: axis h when
    j % 3 == 1 and j < 3*s_h, axis w when j % 3 == 2 and j < 3*s_w, else t.
  * Sliding window of W keys including the query: key j visible to query i
    iff i - W < j <= i.
  * GQA: query head h reads key/value head h // (Hq / Hkv).
  * Deepstack rows are added after the layer's residual sum.
  * Decode: the new token's key/value sit at cache index n = lens[b]; it sees
    keys n - W < j <= n (sliding) or j <= n (full).
  * Chunked prefill: new token i of row b sits at cache index start[b] + i, with
    the same visibility rule as decode.
  * The corrected rotary layout ("sections", page 1's correction under "Acceptance
    criteria"): contiguous H, W, T sections, each carrying the frequency indices the
    interleave gives its axis, in increasing order. PARITY UNPINNED against the real
    rotary class, whose permutation the page does not print; pinned only to the axis
    sets the page prints and to the structure of this reading.
  * 4-bit weights (the quantization block of page 1's config section: group size
    64, 4 bits, affine): a weight is scale * code + bias with one (scale, bias)
    per 64 consecutive input columns; byte j of a packed row holds column 2j in
    its low nibble and column 2j + 1 in its high nibble.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64

# Status codes of the position-id construction (shared meaning with the C ABI,
# defined independently there).
POS_OK = 0
POS_SPAN_MISMATCH = 1      # an image's pad span runs past L or hits a non-pad token
POS_EXTRA_PADS = 2         # pad tokens left over with no image to consume them
POS_UNUSED_IMAGES = 3      # images left over after the row's last pad span
POS_BAD_GRID = 4           # grid entry non-positive or h/w not divisible by the merge size


class PositionError(ValueError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


# ----------------------------------------------------------------------------------------
# Position ids. Page 1, "Position ids (get_rope_index)". A running counter st gives every
# ordinary token the triple (st, st, st) and then moves on by one. An image spans one pad per
# cell of its merged grid (frames x rows/merge x cols/merge); each pad gets st plus its own
# (frame, row, col) index, and afterwards st moves past the largest of the three extents.
# The row's offset for later tokens is the final counter minus the row length.
# ----------------------------------------------------------------------------------------
def mrope_positions(tokens: np.ndarray, image_token_id: int, grid_thw: np.ndarray,
                    img_offset: np.ndarray, spatial_merge: int) -> Tuple[np.ndarray, np.ndarray]:
    """tokens [B, L] int; grid_thw [n_img, 3] (patch units); img_offset [B+1].

    Returns pos [3, B, L] int64 and rope_delta [B] int64. Raises PositionError.
    """
    tokens = np.asarray(tokens)
    B, L = tokens.shape
    pos = np.zeros((3, B, L), dtype=np.int64)
    delta = np.zeros(B, dtype=np.int64)
    m = int(spatial_merge)
    for b in range(B):
        st = 0                      # first position of the next text token
        k = int(img_offset[b])      # next image of this row
        k_end = int(img_offset[b + 1])
        l = 0
        while l < L:
            if int(tokens[b, l]) != image_token_id:
                pos[:, b, l] = st
                st += 1
                l += 1
                continue
            if k >= k_end:
                raise PositionError(POS_EXTRA_PADS, f"row {b}: pad token at {l} but no image left")
            t, h, w = (int(v) for v in grid_thw[k])
            if t < 1 or h < 1 or w < 1 or h % m or w % m:
                raise PositionError(POS_BAD_GRID, f"image {k}: bad grid {(t, h, w)} for merge {m}")
            gh, gw = h // m, w // m
            n = t * gh * gw
            if l + n > L or np.any(tokens[b, l:l + n] != image_token_id):
                raise PositionError(POS_SPAN_MISMATCH, f"row {b}: image {k} needs {n} pads at {l}")
            for r in range(n):
                pos[0, b, l + r] = st + r // (gh * gw)
                pos[1, b, l + r] = st + (r // gw) % gh
                pos[2, b, l + r] = st + r % gw
            st += max(t, gh, gw)
            k += 1
            l += n
        if k != k_end:
            raise PositionError(POS_UNUSED_IMAGES, f"row {b}: {k_end - k} image(s) not consumed")
        delta[b] = st - L           # == max position + 1 - L
    return pos, delta


def decode_positions(lens: np.ndarray, rope_delta: np.ndarray) -> np.ndarray:
    """Page 1, "Position ids": each new token sits at offset + rope_delta on all three axes."""
    p = np.asarray(lens, dtype=np.int64) + np.asarray(rope_delta, dtype=np.int64)
    return np.stack([p, p, p])


# ----------------------------------------------------------------------------------------
# LayerNorm. Page 1, "Text decoder forward": weight only, no bias, computed in float.
# ----------------------------------------------------------------------------------------
def layer_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(w, dtype=F64)


# ----------------------------------------------------------------------------------------
# Interleaved MRoPE. Page 1, "Interleaved MRoPE (sliding layers)": inv_freq[j] =
# base^(-2j/hd); axis t by default, h when j % 3 == 1 and j < 3*s_h, w when j % 3 == 2 and
# j < 3*s_w; cos/sin of concat(freqs, freqs); q*cos + rotate_half(q)*sin with
# rotate_half(x) = concat(-x2, x1).
# ----------------------------------------------------------------------------------------
def mrope_axis_map(section: Sequence[int], half: int) -> np.ndarray:
    s_t, s_h, s_w = (int(s) for s in section)
    if s_t + s_h + s_w != half:
        raise ValueError(f"mrope section {tuple(section)} does not sum to {half}")
    ax = np.zeros(half, dtype=np.int64)
    for j in range(half):
        if j % 3 == 1 and j < 3 * s_h:
            ax[j] = 1
        elif j % 3 == 2 and j < 3 * s_w:
            ax[j] = 2
    counts = (int((ax == 0).sum()), int((ax == 1).sum()), int((ax == 2).sum()))
    if counts != (s_t, s_h, s_w):
        raise ValueError(f"section {tuple(section)} is not realisable by the interleave (got {counts})")
    return ax


def inv_freq(theta: float, head_dim: int) -> np.ndarray:
    j = np.arange(head_dim // 2, dtype=F64)
    return float(theta) ** (-2.0 * j / head_dim)


def mrope_section_layout(section: Sequence[int], half: int) -> Tuple[np.ndarray, np.ndarray]:
    """The corrected Compass layout (page 1, the correction under "Acceptance criteria": the
    real rotary class pre-permutes inv_freq and gives the axes contiguous [H, W, T] sections).
    The permutation is not printed. Reading (parity unpinned against the real class): each
    axis keeps the frequency indices the interleave gives it, in increasing order, and the
    sections are laid out H, then W, then T. Returns (axis[f], freq_index[f]) for f < half."""
    ax = mrope_axis_map(section, half)
    order = (1, 2, 0)
    fidx = np.concatenate([np.flatnonzero(ax == a) for a in order])
    axis = np.concatenate([np.full(int((ax == a).sum()), a, dtype=np.int64) for a in order])
    return axis, fidx


def mrope_angles(pos3: np.ndarray, section: Sequence[int], theta: float, head_dim: int,
                 layout: str = "interleaved") -> np.ndarray:
    """pos3 [3, N] -> angles [N, hd/2]: freqs[n, j] = pos[axis(j), n] * inv_freq[j]
    (layout "interleaved"); with layout "sections", column f carries frequency index
    freq_index[f] on axis axis[f] of mrope_section_layout."""
    half = head_dim // 2
    pos3 = np.asarray(pos3, dtype=F64)
    f = inv_freq(theta, head_dim)
    if layout == "sections":
        axis, fidx = mrope_section_layout(section, half)
        return pos3[axis, :].T * f[fidx][None, :]
    if layout != "interleaved":
        raise ValueError(f"unknown rope layout {layout!r}")
    ax = mrope_axis_map(section, half)
    return pos3[ax, :].T * f[None, :]


def _angles(shape, pos3: np.ndarray) -> np.ndarray:
    return mrope_angles(pos3, shape.mrope_section, shape.rope_theta, shape.head_dim,
                        getattr(shape, "rope_layout", "interleaved"))


def rotate_half(x: np.ndarray) -> np.ndarray:
    half = x.shape[-1] // 2
    return np.concatenate([-x[..., half:], x[..., :half]], axis=-1)


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """x [..., N, hd], angles [N, hd/2]: x*cos + rotate_half(x)*sin over concat(freqs, freqs)."""
    full = np.concatenate([angles, angles], axis=-1)
    return np.asarray(x, dtype=F64) * np.cos(full) + rotate_half(np.asarray(x, dtype=F64)) * np.sin(full)


# ----------------------------------------------------------------------------------------
# Attention. Page 1, "Text decoder forward": sdpa(q, k, v, scale = hd^-1/2) with a causal
# mask, restricted to the last W keys on sliding layers; plain causal on full layers.
# ----------------------------------------------------------------------------------------
def visible(i: int, j: np.ndarray, kind: str, window: int) -> np.ndarray:
    ok = j <= i
    if kind == "sliding":
        ok &= j > i - window
    return ok


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, kind: str, window: int,
              q_index: Optional[np.ndarray] = None, k_index: Optional[np.ndarray] = None) -> np.ndarray:
    """q [Hq, Nq, hd]; k, v [Hkv, Nk, hd]. Returns o [Nq, Hq*hd].

    q_index / k_index give the sequence index of each query / key (default arange).
    """
    Hq, Nq, hd = q.shape
    Hkv, Nk, _ = k.shape
    g = Hq // Hkv
    qi = np.arange(Nq) if q_index is None else np.asarray(q_index)
    kj = np.arange(Nk) if k_index is None else np.asarray(k_index)
    mask = kj[None, :] <= qi[:, None]
    if kind == "sliding":
        mask &= kj[None, :] > qi[:, None] - window
    out = np.empty((Nq, Hq * hd), dtype=F64)
    scale = 1.0 / np.sqrt(hd)
    for h in range(Hq):
        kh = np.asarray(k[h // g], dtype=F64)
        vh = np.asarray(v[h // g], dtype=F64)
        s = (np.asarray(q[h], dtype=F64) @ kh.T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h * hd:(h + 1) * hd] = p @ vh
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------------------
# The parallel block. Page 1, "Text decoder forward": a = LN(h); h = h + Attn(a) + SwiGLU(a);
# deepstack rows are added after layers 0..2. Weights are nn.Linear [out, in], no biases.
# ----------------------------------------------------------------------------------------
def projections(a: np.ndarray, w: Dict[str, np.ndarray]):
    a = np.asarray(a, dtype=F64)
    f = lambda name: np.asarray(w[name], dtype=F64)
    return a @ f("wq").T, a @ f("wk").T, a @ f("wv").T, a @ f("w_gate").T, a @ f("w_up").T


def _heads(x: np.ndarray, n_heads: int, hd: int) -> np.ndarray:
    """[N, H*hd] -> [H, N, hd]"""
    return x.reshape(x.shape[0], n_heads, hd).transpose(1, 0, 2)


def layer_prefill(shape, w: Dict[str, np.ndarray], x: np.ndarray, pos: Optional[np.ndarray] = None,
                  ds_rows: Optional[np.ndarray] = None, ds: Optional[np.ndarray] = None,
                  return_stages: bool = False):
    """x [B, L, D]; pos [3, B, L] (sliding layers). Returns out [B, L, D] (and stages)."""
    x = np.asarray(x, dtype=F64)
    B, L, D = x.shape
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    out = np.empty_like(x)
    stages = {"q": [], "k": [], "v": [], "act": [], "attn": []}
    for b in range(B):
        a = layer_norm(x[b], w["ln_w"], shape.ln_eps)
        q, k, v, g, u = projections(a, w)
        qh, kh, vh = _heads(q, Hq, hd), _heads(k, Hkv, hd), _heads(v, Hkv, hd)
        if shape.kind == "sliding":
            ang = _angles(shape, pos[:, b, :])
            qh, kh = apply_rope(qh, ang), apply_rope(kh, ang)
        o = attention(qh, kh, vh, shape.kind, shape.window)
        act = silu(g) * u
        attn_out = o @ np.asarray(w["wo"], dtype=F64).T
        mlp_out = act @ np.asarray(w["w_down"], dtype=F64).T
        out[b] = x[b] + attn_out + mlp_out
        if return_stages:
            stages["q"].append(qh); stages["k"].append(kh); stages["v"].append(vh)
            stages["act"].append(act); stages["attn"].append(o)
    if ds_rows is not None and ds is not None and len(ds_rows):
        flat = out.reshape(B * L, D)
        flat[np.asarray(ds_rows)] += np.asarray(ds, dtype=F64)
    if return_stages:
        return out, {k2: np.stack(v2) for k2, v2 in stages.items()}
    return out


def layer_prefill_rows(shape, w: Dict[str, np.ndarray], x: np.ndarray, pos: Optional[np.ndarray],
                       b: int, rows: Sequence[int]) -> np.ndarray:
    """Outputs of selected rows of batch row b, computed one by one from the definition.

    Only the keys each selected query can see are projected: the span from the earliest
    key visible to the smallest selected row up to the largest selected row. Returns
    [len(rows), D] in the order of `rows` (no deepstack term).
    """
    x = np.asarray(x, dtype=F64)
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    lo = 0 if shape.kind == "full" else max(0, int(rows.min()) - shape.window + 1)
    hi = int(rows.max()) + 1
    span = np.arange(lo, hi)
    a_span = layer_norm(x[b, lo:hi], w["ln_w"], shape.ln_eps)
    k = a_span @ np.asarray(w["wk"], dtype=F64).T
    v = a_span @ np.asarray(w["wv"], dtype=F64).T
    kh, vh = _heads(k, Hkv, hd), _heads(v, Hkv, hd)
    a_rows = layer_norm(x[b, rows], w["ln_w"], shape.ln_eps)
    q = a_rows @ np.asarray(w["wq"], dtype=F64).T
    qh = _heads(q, Hq, hd)
    if shape.kind == "sliding":
        kh = apply_rope(kh, _angles(shape, pos[:, b, lo:hi]))
        qh = apply_rope(qh, _angles(shape, pos[:, b, rows]))
    o = attention(qh, kh, vh, shape.kind, shape.window, q_index=rows, k_index=span)
    g = a_rows @ np.asarray(w["w_gate"], dtype=F64).T
    u = a_rows @ np.asarray(w["w_up"], dtype=F64).T
    act = silu(g) * u
    return (x[b, rows] + o @ np.asarray(w["wo"], dtype=F64).T
            + act @ np.asarray(w["w_down"], dtype=F64).T)


# ----------------------------------------------------------------------------------------
# Decode. Page 1, "Text decoder forward" and its correction under "Acceptance criteria"
# (dense cache with the window applied as a mask): one new token per row, keys/values
# appended at index lens[b] after rotation, position lens[b] + rope_delta[b].
# ----------------------------------------------------------------------------------------
def layer_decode(shape, w: Dict[str, np.ndarray], x: np.ndarray, pos: np.ndarray,
                 k_cache: np.ndarray, v_cache: np.ndarray, lens: np.ndarray,
                 rows: Optional[Sequence[int]] = None):
    """x [B, D]; pos [3, B]; caches [B, Hkv, cap, hd] (read only here).

    Returns (out [nb, D], k_new [nb, Hkv, hd], v_new [nb, Hkv, hd]) for the batch rows
    `rows` (default all).
    """
    x = np.asarray(x, dtype=F64)
    B, D = x.shape
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    rows = list(range(B)) if rows is None else list(rows)
    outs, ks, vs = [], [], []
    for b in rows:
        n = int(lens[b])
        a = layer_norm(x[b:b + 1], w["ln_w"], shape.ln_eps)
        q, k, v, g, u = projections(a, w)
        qh, kh, vh = _heads(q, Hq, hd), _heads(k, Hkv, hd), _heads(v, Hkv, hd)
        if shape.kind == "sliding":
            ang = _angles(shape, pos[:, b:b + 1])
            qh, kh = apply_rope(qh, ang), apply_rope(kh, ang)
        lo = 0 if shape.kind == "full" else max(0, n - shape.window + 1)
        kc = np.asarray(k_cache[b, :, lo:n, :], dtype=F64)
        vc = np.asarray(v_cache[b, :, lo:n, :], dtype=F64)
        kk = np.concatenate([kc, kh], axis=1)
        vv = np.concatenate([vc, vh], axis=1)
        o = attention(qh, kk, vv, shape.kind, shape.window, q_index=np.array([n]),
                      k_index=np.arange(lo, n + 1))
        act = silu(g) * u
        out = x[b] + (o @ np.asarray(w["wo"], dtype=F64).T)[0] + (act @ np.asarray(w["w_down"], dtype=F64).T)[0]
        outs.append(out); ks.append(kh[:, 0, :]); vs.append(vh[:, 0, :])
    return np.stack(outs), np.stack(ks), np.stack(vs)


# ----------------------------------------------------------------------------------------
# 4-bit affine weights. Page 1, config section: the 4-bit checkpoint carries a quantization
# block {group_size 64, bits 4, mode affine}. Affine mode: a weight is its group's scale
# times its 4-bit code plus its group's bias; groups are 64 consecutive input columns of
# one output row. The nibble order inside a byte is not printed (reading: low nibble first).
# ----------------------------------------------------------------------------------------
Q4_GROUP = 64


def unpack_q4(packed: np.ndarray) -> np.ndarray:
    """packed uint8 [rows, cols / 2] -> codes [rows, cols] in 0..15."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int64)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    return codes


def dequantize_q4(packed: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """w[r, c] = scales[r, c // 64] * code[r, c] + biases[r, c // 64], in fp64."""
    codes = unpack_q4(packed).astype(F64)
    s = np.repeat(np.asarray(scales, dtype=F64), Q4_GROUP, axis=1)
    b = np.repeat(np.asarray(biases, dtype=F64), Q4_GROUP, axis=1)
    return s * codes + b


Q4_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def dequantize_layer_q4(wq4: Dict[str, object]) -> Dict[str, np.ndarray]:
    """wq4: ln_w plus, for each matrix, a (packed, scales, biases) triple."""
    w = {"ln_w": np.asarray(wq4["ln_w"], dtype=F64)}
    for name in Q4_MATRICES:
        w[name] = dequantize_q4(*wq4[name])
    return w


def layer_decode_q4(shape, wq4: Dict[str, object], x: np.ndarray, pos: np.ndarray, k_cache: np.ndarray,
                    v_cache: np.ndarray, lens: np.ndarray, rows: Optional[Sequence[int]] = None):
    """The decode step with 4-bit weights: the layer of the dequantized weights."""
    return layer_decode(shape, dequantize_layer_q4(wq4), x, pos, k_cache, v_cache, lens, rows)


# ----------------------------------------------------------------------------------------
# Chunked prefill. Page 5 ("feat(mm): serve image input on the Qwen families", "How it fits
# together") serves prompts through chunked prefill over a prefix cache, with image spans
# crossing chunk boundaries; page 1 keeps a dense cache with the window as a mask
# ("Acceptance criteria" correction). A chunk of L new tokens in row b continues a cache
# that already holds start[b] tokens: new token i sits at cache index n = start[b] + i,
# its key/value (rotated on sliding layers) are appended there, and it sees keys j <= n
# (and j > n - W on sliding layers) over cache and chunk together. With L = 1 this is
# the decode step; with start = 0 it is the plain prefill.
# ----------------------------------------------------------------------------------------
def layer_prefill_chunk(shape, w: Dict[str, np.ndarray], x: np.ndarray, pos: Optional[np.ndarray],
                        k_cache: np.ndarray, v_cache: np.ndarray, start: np.ndarray):
    """x [B, L, D]; pos [3, B, L] (sliding layers; the new tokens' positions); caches
    [B, Hkv, cap, hd] holding at least start[b] tokens (read only here).

    Returns (out [B, L, D], k_new [B, Hkv, L, hd], v_new [B, Hkv, L, hd]).
    """
    x = np.asarray(x, dtype=F64)
    B, L, D = x.shape
    Hq, Hkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    out = np.empty_like(x)
    k_new = np.empty((B, Hkv, L, hd), dtype=F64)
    v_new = np.empty_like(k_new)
    for b in range(B):
        s0 = int(start[b])
        a = layer_norm(x[b], w["ln_w"], shape.ln_eps)
        q, k, v, g, u = projections(a, w)
        qh, kh, vh = _heads(q, Hq, hd), _heads(k, Hkv, hd), _heads(v, Hkv, hd)
        if shape.kind == "sliding":
            ang = _angles(shape, pos[:, b, :])
            qh, kh = apply_rope(qh, ang), apply_rope(kh, ang)
        kk = np.concatenate([np.asarray(k_cache[b, :, :s0, :], dtype=F64), kh], axis=1)
        vv = np.concatenate([np.asarray(v_cache[b, :, :s0, :], dtype=F64), vh], axis=1)
        o = attention(qh, kk, vv, shape.kind, shape.window, q_index=s0 + np.arange(L),
                      k_index=np.arange(s0 + L))
        act = silu(g) * u
        out[b] = x[b] + o @ np.asarray(w["wo"], dtype=F64).T + act @ np.asarray(w["w_down"], dtype=F64).T
        k_new[b], v_new[b] = kh, vh
    return out, k_new, v_new


# ----------------------------------------------------------------------------------------
# Varlen prefill. Page 5 ("How it fits together") plans prefill per request, each with its own
# MRoPE positions and its own prefix cache; page 1 ("Validation") requires prefill to stay
# causal within a sequence. Packed rows [cu[s], cu[s+1]) are sequence s, a chunk continuing
# that sequence's dense cache at start[s] (0 when no cache is kept); sequences never see one
# another's keys. A sequence whose chunk does not fit its cache produces nothing.
# ----------------------------------------------------------------------------------------
def layer_prefill_varlen(shape, w: Dict[str, np.ndarray], x: np.ndarray, pos: Optional[np.ndarray],
                         cu_seqlens: Sequence[int], k_cache: Optional[np.ndarray] = None,
                         v_cache: Optional[np.ndarray] = None, start: Optional[Sequence[int]] = None):
    """x [T, D] packed rows; pos [3, T] (sliding layers); cu_seqlens [n_seq + 1] with
    cu[0] = 0 <= cu[1] <= ... <= cu[n_seq] = T; caches [n_seq, Hkv, cap, hd] holding at least
    start[s] tokens of sequence s (read only here), or None with start None.

    Returns (out [T, D], k_new, v_new): k_new / v_new are lists with [Hkv, len_s, hd] per
    sequence. Rows of a sequence whose chunk does not fit its cache come back as NaN."""
    x = np.asarray(x, dtype=F64)
    T, D = x.shape
    cu = [int(c) for c in cu_seqlens]
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError(f"cu_seqlens {cu} do not partition {T} rows")
    Hkv, hd = shape.n_kv_heads, shape.head_dim
    out = np.full((T, D), np.nan)
    k_new, v_new = [], []
    for sq in range(len(cu) - 1):
        lo, hi = cu[sq], cu[sq + 1]
        n = hi - lo
        s0 = 0 if start is None else int(start[sq])
        if k_cache is None:
            kc = np.zeros((1, Hkv, 0, hd))
            vc = np.zeros((1, Hkv, 0, hd))
        else:
            if s0 < 0 or s0 + n > k_cache.shape[2]:
                k_new.append(None); v_new.append(None)
                continue
            kc, vc = k_cache[sq:sq + 1], v_cache[sq:sq + 1]
        if n == 0:
            k_new.append(np.zeros((Hkv, 0, hd))); v_new.append(np.zeros((Hkv, 0, hd)))
            continue
        p = None if pos is None else np.asarray(pos)[:, None, lo:hi]
        o, kn, vn = layer_prefill_chunk(shape, w, x[None, lo:hi], p, kc, vc, np.array([s0]))
        out[lo:hi] = o[0]
        k_new.append(kn[0]); v_new.append(vn[0])
    return out, k_new, v_new


# ----------------------------------------------------------------------------------------
# Logits. Page 1, "Text decoder forward": h = LayerNorm(h); logits = embed.as_linear(h) *
# logit_scale. Page 2 ("Cohere2 Command R"): the scale is an in-place fp32 multiply.
# ----------------------------------------------------------------------------------------
def logits(h: np.ndarray, norm_w: np.ndarray, eps: float, embed: np.ndarray, logit_scale: float,
           rows: Optional[Sequence[int]] = None, cols: Optional[Sequence[int]] = None) -> np.ndarray:
    h = np.asarray(h, dtype=F64)
    if rows is not None:
        h = h[np.asarray(rows)]
    e = np.asarray(embed if cols is None else embed[np.asarray(cols)], dtype=F64)
    return (layer_norm(h, norm_w, eps) @ e.T) * float(logit_scale)


# ----------------------------------------------------------------------------------------
# The stack. Page 1, "Text decoder forward" and "Validation": full attention at layers
# i % 4 == 3, sliding elsewhere; deepstack added after layers 0, 1, 2 only.
# ----------------------------------------------------------------------------------------
def layer_kind(i: int) -> str:
    return "full" if i % 4 == 3 else "sliding"


def stack_prefill(shape, layer_weights: Sequence[Dict[str, np.ndarray]], x: np.ndarray,
                  pos: np.ndarray, ds_rows: Optional[np.ndarray] = None,
                  ds: Optional[Sequence[np.ndarray]] = None) -> np.ndarray:
    h = np.asarray(x, dtype=F64)
    for i, w in enumerate(layer_weights):
        sh = shape.with_kind(layer_kind(i))
        use_ds = ds is not None and i < 3 and i < len(ds)
        h = layer_prefill(sh, w, h, pos, ds_rows if use_ds else None, ds[i] if use_ds else None)
    return h


# ----------------------------------------------------------------------------------------
# Token-id front end and greedy generation. Page 1, "Text decoder forward": h =
# embed_tokens(tokens), and the vision tower's final merger produces "the image embeddings
# that replace the image-pad tokens"; page 5 ("How it fits together") writes those
# gathered rows into the batch with one index_copy. Generation continues a row after its
# prompt with position lens + rope_delta on every axis (page 1, "Position ids") and takes
# the next token as the argmax of the tied-embedding logits (smallest id on ties).
# ----------------------------------------------------------------------------------------
def embed(tokens: np.ndarray, embed_table: np.ndarray, image_rows: Optional[np.ndarray] = None,
          image_feats: Optional[np.ndarray] = None) -> np.ndarray:
    """tokens [N] int -> h [N, D] = E[tokens]; then h[image_rows[r]] = image_feats[r]."""
    h = np.asarray(embed_table, dtype=F64)[np.asarray(tokens)].copy()
    if image_rows is not None and len(image_rows):
        h[np.asarray(image_rows)] = np.asarray(image_feats, dtype=F64)
    return h


def greedy_token(h_last: np.ndarray, norm_w: np.ndarray, eps: float, embed_table: np.ndarray,
                 logit_scale: float) -> np.ndarray:
    """h_last [R, D] -> argmax of the logits per row (first index on ties)."""
    return np.argmax(logits(h_last, norm_w, eps, embed_table, logit_scale), axis=1)


def greedy_generate(shape, layer_weights: Sequence[Dict[str, np.ndarray]], embed_table: np.ndarray,
                    norm_w: np.ndarray, logit_scale: float, tokens: np.ndarray, grid_thw: np.ndarray,
                    img_offset: np.ndarray, image_feats: Optional[np.ndarray], ds: Optional[Sequence[np.ndarray]],
                    image_token_id: int, spatial_merge: int, n_new: int, return_hidden: bool = False):
    """Prompt tokens [B, L] (image pads expanded), image_feats [n_pad_rows, D] for the pad
    tokens in row-major order, ds[i] [n_pad_rows, D] deepstack inputs of layers 0..2.
    Returns the n_new greedily generated tokens [B, n_new] (and, with return_hidden, the
    final hidden row each token was chosen from, [B, n_new, D])."""
    tokens = np.asarray(tokens)
    B, L = tokens.shape
    pos, rope_delta = mrope_positions(tokens, image_token_id, grid_thw, img_offset, spatial_merge)
    pad_rows = np.flatnonzero(tokens.reshape(-1) == image_token_id)
    h = embed(tokens.reshape(-1), embed_table, pad_rows, image_feats).reshape(B, L, -1)
    caches = []
    for i, w in enumerate(layer_weights):
        sh = shape.with_kind(layer_kind(i))
        use_ds = ds is not None and i < 3 and len(pad_rows) > 0
        h, st = layer_prefill(sh, w, h, pos, pad_rows if use_ds else None, ds[i] if use_ds else None,
                              return_stages=True)
        caches.append((st["k"], st["v"]))
    out = np.empty((B, n_new), dtype=np.int64)
    hid = np.empty((B, n_new, h.shape[-1]), dtype=F64)
    hid[:, 0] = h[:, -1]
    tok = greedy_token(h[:, -1], norm_w, shape.ln_eps, embed_table, logit_scale)
    for step in range(n_new):
        out[:, step] = tok
        if step == n_new - 1:
            break
        lens = np.full(B, L + step)
        p3 = decode_positions(lens, rope_delta)
        x = embed(tok, embed_table)
        for i, w in enumerate(layer_weights):
            sh = shape.with_kind(layer_kind(i))
            kc, vc = caches[i]
            kpad = np.concatenate([kc, np.zeros_like(kc[:, :, :1])], axis=2)
            vpad = np.concatenate([vc, np.zeros_like(vc[:, :, :1])], axis=2)
            x, knew, vnew = layer_decode(sh, w, x, p3, kpad, vpad, lens)
            kpad[:, :, -1], vpad[:, :, -1] = knew, vnew
            caches[i] = (kpad, vpad)
        hid[:, step + 1] = x
        tok = greedy_token(x, norm_w, shape.ln_eps, embed_table, logit_scale)
    return (out, hid) if return_hidden else out
