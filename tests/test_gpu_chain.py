"""Chained decode (compass_layer_decode_chained): each layer's residual kernel also writes
the next layer's LayerNorm of its output, and the next layer reads it instead of running
its own LayerNorm kernel.

Gates: every layer's output and new K/V rows equal those of a chain of
compass_layer_decode calls bit for bit (the handed-over rows are what the LayerNorm
kernel computes); each layer's output is within 2e-2 of the fp64 oracle given that
layer's input; the handed-over rows match an fp64 LayerNorm of the layer's bf16 output to
the bf16 rounding; rows whose cache length is out of range keep their output.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import stream_seed
from synth import workloads as W
from synth.workloads import WORKLOADS
import synth.rng_torch as RT
from tests import helpers as H
from tests.test_gpu_small import check_layer_out, layer_case

pytestmark = pytest.mark.gpu


def run_chained(shape, wdev, x, x_norm, pos, kc, vc, lens, next_w, next_eps, out_norm):
    b = H.B()
    d = H.desc(shape)
    ws = H.workspace(b.compass_workspace_size(d, x.shape[0], 1, kc.shape[2], 1))
    out = torch.empty_like(x)
    b.compass_layer_decode_chained(d, b.make_weights(wdev), x, x_norm, pos, b.make_kv(kc, vc, lens), out,
                                   next_w, next_eps, out_norm, ws)
    return out


def check_norm(norm, out, ln_w, eps, rows):
    """The handed-over rows against an fp64 LayerNorm of the bf16 output rows: equal up to
    the bf16 rounding of the result (and the fp32 statistics)."""
    o = H.np64(out)[rows]
    ref = O.layer_norm(o, np.asarray(ln_w, np.float64), eps)
    got = H.np64(norm)[rows]
    err = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)
    assert float(err.max()) <= 1e-5 * float(np.abs(ref).max()), float(err.max())


def chain_case(shapes, ws_np, x, pos_np, caches, lens_np):
    """Runs the layers both ways on identical copies of the caches; returns per layer the
    (input, unchained out, chained out, handed-over LayerNorm or None) and the caches."""
    td = torch.bfloat16
    Bn = x.shape[0]
    lens, pos = H.ints_to_dev(lens_np), H.ints_to_dev(pos_np)
    plain = [(kc.clone(), vc.clone()) for kc, vc in caches]
    chain = [(kc.clone(), vc.clone()) for kc, vc in caches]
    norm = torch.empty((Bn, shapes[0].hidden), dtype=td, device="cuda")
    wdevs = [H.weights_to_dev(sh, w) for sh, w in zip(shapes, ws_np)]
    xa = xb = H.to_dev(x, td) if isinstance(x, np.ndarray) else x
    outs = []
    for i, sh in enumerate(shapes):
        last = i == len(shapes) - 1
        oa = H.run_decode(sh, wdevs[i], xa, pos, plain[i][0], plain[i][1], lens)
        ob = run_chained(sh, wdevs[i], xb, None if i == 0 else norm, pos, chain[i][0], chain[i][1], lens,
                         None if last else wdevs[i + 1]["ln_w"], 0.0 if last else shapes[i + 1].ln_eps,
                         None if last else norm)
        torch.cuda.synchronize()
        outs.append((xb, oa, ob, None if last else norm.clone()))
        xa, xb = oa, ob
    return outs, plain, chain


def small_stack():
    base = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 40)
    return [base.with_kind(O.layer_kind(i)) for i in range(4)]


@pytest.mark.parametrize("Bn", [9, 70])
def test_chained_decode_small_stack(Bn):
    """Four layers [S, S, S, F] at small widths with ragged lengths, the last row's length
    outside the cache; B = 70 puts two 64-row tiles in the decode GEMMs (another split-K
    count in the residual)."""
    shapes = small_stack()
    cap = 301
    base = np.array([0, 1, 39, 40, 41, 255, 256, 300], np.int32)
    lens_np = np.concatenate([np.resize(base, Bn - 1), [cap]]).astype(np.int32)  # the last row is skipped
    live = lens_np < cap
    ws_np = [layer_case(sh, 1, 8, seed=40 + i)[0] for i, sh in enumerate(shapes)]
    x = H.rand_np(50, (Bn, shapes[0].hidden), bf16=True)
    pos_np = O.decode_positions(lens_np, np.arange(Bn, dtype=np.int64) - 4)
    caches = [(H.to_dev(H.rand_np(60 + i, (Bn, 1, cap, 128), bf16=True), torch.bfloat16),
               H.to_dev(H.rand_np(70 + i, (Bn, 1, cap, 128), bf16=True), torch.bfloat16)) for i in range(4)]
    cache_in = [(H.np64(k), H.np64(v)) for k, v in caches]
    outs, plain, chain = chain_case(shapes, ws_np, x, pos_np, caches, lens_np)
    rows = [r for r in range(Bn) if live[r]]
    for i, (xin, oa, ob, nm) in enumerate(outs):
        # (the skipped row's output is never written, in either run)
        assert torch.equal(oa[rows], ob[rows]), f"layer {i}: chained output differs from the unchained one"
        assert torch.equal(plain[i][0], chain[i][0]) and torch.equal(plain[i][1], chain[i][1]), f"layer {i}: caches"
        if nm is not None:
            check_norm(nm, ob, ws_np[i + 1]["ln_w"], shapes[i + 1].ln_eps, rows)
        x64 = H.np64(xin)
        ref, knew, vnew = O.layer_decode(shapes[i], ws_np[i], x64, pos_np, cache_in[i][0], cache_in[i][1],
                                         lens_np, rows=rows)
        check_layer_out(shapes[i], ob[rows], x64[rows], ref, f"chained layer {i}")
        kg = H.np64(chain[i][0])
        for j, r in enumerate(rows):
            assert H.rel_err(kg[r, :, lens_np[r]], knew[j]) <= H.tol(shapes[i]), f"layer {i} row {r} new K"
    # The skipped row's output and LayerNorm are never written.
    sh = shapes[0]
    out = torch.full((Bn, sh.hidden), 3.0, dtype=torch.bfloat16, device="cuda")
    norm = torch.full((Bn, sh.hidden), 5.0, dtype=torch.bfloat16, device="cuda")
    b = H.B()
    kc, vc = caches[0][0].clone(), caches[0][1].clone()
    d = H.desc(sh)
    wdev = H.weights_to_dev(sh, ws_np[0])  # the ctypes struct holds raw pointers: keep the tensors alive
    nw = H.to_dev(ws_np[1]["ln_w"], torch.bfloat16)
    lens_d = H.ints_to_dev(lens_np)
    b.compass_layer_decode_chained(d, b.make_weights(wdev), H.to_dev(x, torch.bfloat16), None,
                                   H.ints_to_dev(pos_np), b.make_kv(kc, vc, lens_d), out, nw, shapes[1].ln_eps,
                                   norm, H.workspace(b.compass_workspace_size(d, Bn, 1, cap, 1)))
    torch.cuda.synchronize()
    assert torch.all(out[Bn - 1] == 3.0) and torch.all(norm[Bn - 1] == 5.0)
    assert torch.equal(out[:Bn - 1], outs[0][2][:Bn - 1])
    assert torch.equal(norm[:Bn - 1], outs[0][3][:Bn - 1])


@pytest.mark.slow
def test_chained_decode_compass_widths():
    """The last two layers of the 3:1 stack (sliding, then full) at the Compass widths with
    B = 64 and ragged cache lengths: the launch configuration of the bench's decode step
    (split-K projection tiles, the skinny output GEMM's 8 K-slices)."""
    cfg = WORKLOADS["decode_stack"]
    shapes = [dataclasses.replace(cfg["shape"], kind=O.layer_kind(i)) for i in (2, 3)]
    Bn, cap = 64, 1100
    Hkv, hd = shapes[0].n_kv_heads, shapes[0].head_dim
    rng = np.random.default_rng(64)
    lens_np = rng.integers(0, cap - 1, Bn).astype(np.int32)
    pos_np = O.decode_positions(lens_np, rng.integers(-30, 30, Bn)).astype(np.int32)
    ws_np = [W.make_layer_weights(sh, W.Stream.DECODE_STACK, 20 + i) for i, sh in enumerate(shapes)]
    x = W.make_layer_input(shapes[0], W.Stream.DECODE_STACK, Bn, layer=20)
    caches = []
    for i in range(2):
        kc = RT.normal(stream_seed(W.Stream.DECODE_STACK, 20 + i, W.TensorId.K_CACHE), Bn * Hkv * cap * hd)
        vc = RT.normal(stream_seed(W.Stream.DECODE_STACK, 20 + i, W.TensorId.V_CACHE), Bn * Hkv * cap * hd)
        caches.append((kc.to(torch.bfloat16).view(Bn, Hkv, cap, hd), vc.to(torch.bfloat16).view(Bn, Hkv, cap, hd)))
    cache_in = [(H.np64(k), H.np64(v)) for k, v in caches]
    outs, plain, chain = chain_case(shapes, ws_np, x, pos_np, caches, lens_np)
    rows = [0, 17, 40, 63]
    for i, (xin, oa, ob, nm) in enumerate(outs):
        assert torch.equal(oa, ob), f"layer {i}: chained output differs from the unchained one"
        assert torch.equal(plain[i][0], chain[i][0]) and torch.equal(plain[i][1], chain[i][1]), f"layer {i}: caches"
        if nm is not None:
            check_norm(nm, ob, ws_np[i + 1]["ln_w"], shapes[i + 1].ln_eps, list(range(Bn)))
        x64 = H.np64(xin)
        w64 = {k: np.asarray(v, np.float64) for k, v in ws_np[i].items()}
        ref, _, _ = O.layer_decode(shapes[i], w64, x64, pos_np, cache_in[i][0], cache_in[i][1], lens_np, rows=rows)
        check_layer_out(shapes[i], ob[rows], x64[rows], ref, f"chained Compass layer {i}")


def test_chained_decode_into_the_greedy_head():
    """The last layer hands over the final LayerNorm (next_ln_w = the final norm weight) and
    the greedy head takes those rows with norm_w NULL: the same tokens and maxima, bit for
    bit, as the head normalizing the layer output itself."""
    sh = small_stack()[3]
    Bn, cap, V = 9, 301, 777
    lens_np = np.array([0, 1, 39, 40, 41, 255, 256, 299, 300], np.int32)
    w = layer_case(sh, 1, 8, seed=90)[0]
    wdev = H.weights_to_dev(sh, w)
    x = H.to_dev(H.rand_np(91, (Bn, sh.hidden), bf16=True), torch.bfloat16)
    pos = H.ints_to_dev(O.decode_positions(lens_np, np.zeros(Bn, np.int64)))
    kc = H.to_dev(H.rand_np(92, (Bn, 1, cap, 128), bf16=True), torch.bfloat16)
    vc = H.to_dev(H.rand_np(93, (Bn, 1, cap, 128), bf16=True), torch.bfloat16)
    fnw = H.to_dev(H.rand_np(94, (sh.hidden,), std=0.1, mean=1.0), torch.bfloat16)
    E = H.to_dev(H.rand_np(95, (V, sh.hidden), std=0.5), torch.bfloat16)
    norm = torch.empty_like(x)
    out = run_chained(sh, wdev, x, None, pos, kc, vc, H.ints_to_dev(lens_np), fnw, sh.ln_eps, norm)
    b = H.B()
    ws = H.workspace(b.compass_logits_argmax_workspace_size(Bn, sh.hidden, V, 1))
    res = []
    for h, nw in ((out, fnw), (norm, None)):
        tok = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
        mx = torch.empty((Bn,), dtype=torch.float32, device="cuda")
        b.compass_logits_argmax(h, nw, sh.ln_eps, E, 0.25, tok, mx, ws, 1)
        torch.cuda.synchronize()
        res.append((tok.clone(), mx.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    assert int(res[1][0].min()) >= 0
