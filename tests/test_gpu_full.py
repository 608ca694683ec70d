"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Outputs are compared on sampled rows that the fp64 oracle computes one by one
(oracle.layer_prefill_rows / layer_decode), or on the whole result where the oracle
finishes in seconds. Large random tensors (decode caches, the tied embedding) are
generated on the GPU by synth.rng_torch and copied to the host for the oracle: they
are inputs, not results of the HIP path. Gates: max relative error 2e-2 (bf16), and
the branch sum out - x within 2e-2 of its own scale after allowing for the bf16
rounding of out.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import stream_seed
from synth import workloads as W
from synth.workloads import WORKLOADS, layer_kind
import synth.rng_torch as RT
from tests import helpers as H
from tests.test_gpu_small import check_layer_out

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def gpu_positions(tok, grid, off):
    b = H.B()
    Bn, L = tok.shape
    pos = torch.empty((3, Bn, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    status = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    b.compass_mrope_positions(H.ints_to_dev(tok), W.IMAGE_TOKEN_ID, H.ints_to_dev(grid), H.ints_to_dev(off), 2,
                              pos, delta, status)
    return pos, delta, status


def test_sliding_prefill_full_size():
    """hidden 2048, 16/4 heads, hd 128, I 8192, window 1024, L = 4096 (64 text + 1024 image + 3008 text)."""
    cfg = WORKLOADS["sliding_prefill"]
    sh, L = cfg["shape"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.SLIDING_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.SLIDING_PREFILL, L).reshape(1, L, sh.hidden)
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.SLIDING_PREFILL, 0, W.TensorId.TOKENS))
    ref_pos, ref_delta = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    pos, delta, status = gpu_positions(tok, grid, off)
    out = H.run_prefill(sh, H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), pos)
    torch.cuda.synchronize()
    assert status.item() == 0
    assert np.array_equal(pos.cpu().numpy(), ref_pos) and delta.item() == ref_delta[0]
    rows = [0, 1, 63, 64, 65, 600, 1023, 1024, 1087, 1088, 1089, 2047, 2048, 3000, 4094, 4095]
    ref = O.layer_prefill_rows(sh, w, x, ref_pos, 0, rows)
    got = H.np64(out[0, rows])
    check_layer_out(sh, got_t(got), x[0, rows], ref)


def got_t(a):
    return torch.from_numpy(a)


def test_chunked_prefill_full_size():
    """The same row as 4 chunks of 1024 tokens, each continuing the dense cache (the chunked
    workload bench.py times): sampled rows against the fp64 oracle, the cache against the one
    a single prefill of the row writes (the projection's arithmetic per element does not depend
    on the rows in the launch, so bitwise), and every output row within the bf16 gate of that
    prefill's (the chunks' output GEMM splits K, so not bitwise)."""
    cfg = WORKLOADS["sliding_prefill"]
    sh, L = cfg["shape"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.SLIDING_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.SLIDING_PREFILL, L).reshape(1, L, sh.hidden)
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.SLIDING_PREFILL, 0, W.TensorId.TOKENS))
    ref_pos, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    pos, _, status = gpu_positions(tok, grid, off)
    wd, xd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16)
    n_chunks, Lc = 4, L // 4
    kc = torch.full((1, sh.n_kv_heads, L, sh.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    outs = []
    for i in range(n_chunks):
        lens = H.ints_to_dev(np.array([i * Lc], dtype=np.int32))
        outs.append(H.run_prefill_chunk(sh, wd, xd[:, i * Lc:(i + 1) * Lc].contiguous(),
                                        pos[:, :, i * Lc:(i + 1) * Lc].contiguous(), kc, vc, lens))
    got = torch.cat(outs, dim=1)
    kf, vf = torch.empty_like(kc), torch.empty_like(vc)
    whole = H.run_prefill(sh, wd, xd, pos, kv=(kf, vf))
    torch.cuda.synchronize()
    assert status.item() == 0
    assert torch.equal(kc, kf) and torch.equal(vc, vf)
    rows = [0, 63, 64, 1023, 1024, 1025, 1087, 1088, 2047, 2048, 3071, 3072, 4095]
    ref = O.layer_prefill_rows(sh, w, x, ref_pos, 0, rows)
    check_layer_out(sh, got_t(H.np64(got[0, rows])), x[0, rows], ref)
    assert H.rel_err(H.np64(got), H.np64(whole)) <= H.tol(sh)


def test_full_attention_prefill_full_size_and_relabel_invariance():
    """Full (NoPE) layer, B = 2, L = 8192; also bitwise invariance to permuted position ids."""
    cfg = WORKLOADS["full_prefill"]
    sh, Bn, L = cfg["shape"], cfg["B"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.FULL_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.FULL_PREFILL, Bn * L).reshape(Bn, L, sh.hidden)
    wd, xd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16)
    ar = np.broadcast_to(np.arange(L, dtype=np.int32), (3, Bn, L)).copy()
    perm = np.stack([np.stack([W.permutation(stream_seed(W.Stream.FULL_PREFILL, 3 * b + a, W.TensorId.PERM), L) for b in range(Bn)])
                     for a in range(3)]).astype(np.int32)
    o1 = H.run_prefill(sh, wd, xd, H.ints_to_dev(ar))
    o2 = H.run_prefill(sh, wd, xd, H.ints_to_dev(perm))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for b, rows in enumerate([[0, 1, 127, 128, 5000, 8191], [0, 255, 256, 4096, 8190, 8191]]):
        ref = O.layer_prefill_rows(sh, w, x, None, b, rows)
        check_layer_out(sh, got_t(H.np64(o1[b, rows])), x[b, rows], ref)


def test_batched_decode_stack_full_size():
    """4 layers [S, S, S, F], B = 64, cache 8192, window 4096: one decode step."""
    cfg = WORKLOADS["decode_stack"]
    sh, Bn, n_layers, n = cfg["shape"], cfg["B"], cfg["layers"], cfg["cache_len"]
    cap = n + 8
    Hkv, hd = sh.n_kv_heads, sh.head_dim
    rows = [0, 17, 42, 63]
    x = W.make_layer_input(sh, W.Stream.DECODE_STACK, Bn)
    lens_np = np.full(Bn, n, np.int32)
    pos_np = O.decode_positions(lens_np, np.zeros(Bn, np.int64)).astype(np.int32)
    h = H.to_dev(x, torch.bfloat16)
    lens, pos = H.ints_to_dev(lens_np), H.ints_to_dev(pos_np)
    layers = []
    for i in range(n_layers):
        shi = dataclasses.replace(sh, kind=layer_kind(i))
        w = W.make_layer_weights(shi, W.Stream.DECODE_STACK, i)
        kc = RT.normal(stream_seed(W.Stream.DECODE_STACK, i, W.TensorId.K_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
        vc = RT.normal(stream_seed(W.Stream.DECODE_STACK, i, W.TensorId.V_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
        kc_host = H.np64(kc[rows, :, :n])  # cache contents before the step (inputs)
        vc_host = H.np64(vc[rows, :, :n])
        H.run_decode(shi, H.weights_to_dev(shi, w), h, pos, kc, vc, lens, out=h)
        layers.append((shi, w, kc, vc, kc_host, vc_host))
    torch.cuda.synchronize()
    hx = x[rows].astype(np.float64)
    sub_lens = np.full(len(rows), n)
    sub_pos = pos_np[:, rows]
    for i, (shi, w, kc, vc, kh, vh) in enumerate(layers):
        kpad = np.zeros((len(rows), Hkv, n + 1, hd))
        vpad = np.zeros_like(kpad)
        kpad[:, :, :n], vpad[:, :, :n] = kh, vh
        hx, knew, vnew = O.layer_decode(shi, w, hx, sub_pos, kpad, vpad, sub_lens)
        assert H.rel_err(H.np64(kc[rows, :, n]), knew) <= 2e-2, f"layer {i} new K"
        assert H.rel_err(H.np64(vc[rows, :, n]), vnew) <= 2e-2, f"layer {i} new V"
    e = H.rel_err(H.np64(h[rows]), hx)
    assert e <= 2e-2, e


def test_stack_prefill_deepstack_logits_full_size():
    """4-layer [S, S, S, F] prefill, L = 4096, deepstack after layers 0-2, 256000-vocab logits x 0.0625."""
    cfg = WORKLOADS["stack_logits"]
    sh, L, n_layers, V, scale = cfg["shape"], cfg["L"], cfg["layers"], cfg["vocab"], cfg["logit_scale"]
    D = sh.hidden
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.TOKENS))
    pos_np, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    x = W.make_layer_input(sh, W.Stream.STACK_LOGITS, L).reshape(1, L, D)
    ds = [W.make_tensor(sh, 4, i, W.TensorId.DS + i, (1024, D)) for i in range(3)]
    ds_rows = np.arange(64, 64 + 1024, dtype=np.int32)
    ws = [W.make_layer_weights(dataclasses.replace(sh, kind=layer_kind(i)), W.Stream.STACK_LOGITS, i) for i in range(n_layers)]
    nw = W.make_tensor(sh, 4, 0, W.TensorId.FINAL_LN, (D,), std=0.02, mean=1.0)
    E = RT.normal(stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.EMBED), V * D, std=0.02).to(torch.bfloat16).view(V, D)
    pos = H.ints_to_dev(pos_np)
    h = H.to_dev(x, torch.bfloat16)
    rows_d = H.ints_to_dev(ds_rows)
    for i in range(n_layers):
        shi = dataclasses.replace(sh, kind=layer_kind(i))
        use = i < 3
        H.run_prefill(shi, H.weights_to_dev(shi, ws[i]), h, pos, ds_rows=rows_d if use else None,
                      ds=H.to_dev(ds[i], torch.bfloat16) if use else None, out=h)
    logits = H.run_logits(h.view(L, D), H.to_dev(nw, torch.bfloat16), sh.ln_eps, E, scale, 1)
    torch.cuda.synchronize()
    ref_h = O.stack_prefill(sh, ws, x, pos_np, ds_rows, ds)[0]
    check_layer_out(sh, got_t(H.np64(h[0])), x[0], ref_h, "stack")
    rows = [0, 64, 1087, 1088, 2500, 4095]
    cols = np.concatenate([np.arange(0, 2048), np.arange(V - 1024, V),
                           np.random.default_rng(0).integers(0, V, 4096)])
    Ecols = H.np64(E[torch.from_numpy(cols).cuda()])
    ref_l = O.logits(ref_h[rows], nw, sh.ln_eps, Ecols, scale)
    got_l = H.np64(logits[rows][:, torch.from_numpy(cols).cuda()])
    e = H.rel_err(got_l, ref_l)
    assert e <= 2e-2, e
