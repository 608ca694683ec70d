"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Every output is compared whole against the fp64 oracle on the same seeded inputs:
oracle.layer_prefill for the sliding and full prefill layers and for the chunked row,
oracle.layer_decode for all 64 rows of every decode layer, oracle.stack_prefill and
oracle.logits for the stack. Large random tensors (decode caches, the tied embedding)
are generated on the GPU by synth.rng_torch and copied to the host for the oracle:
they are inputs, not results of the HIP path. Layer kinds on the oracle side come
from oracle.layer_kind, on the GPU side from the package's stack schedule.

Gates: max relative error 2e-2 (bf16) on each output tensor, and the branch sum
out - x within 2e-2 of its own scale after allowing for the bf16 rounding of out.
The attention output is also gated on its own, row by row: an attention-probe layer
with Wo = 64 I and w_down = 0 (possible because Hq * hd = D at these widths) returns
out = x + 64 o, so out - x exposes o alone, and each row is compared on that row's
own scale. That makes a window or chunk-merge error visible on every row, where the
branch sum (dominated by the MLP) would hide it.
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
import cohere2_block_mrope_amd.stack as S
from tests import helpers as H
from tests.test_gpu_small import check_layer_out

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

PROBE_SCALE = H.PROBE_SCALE
probe_weights = H.probe_weights
check_attn_rows = H.check_attn_rows


def f64w(w):
    """Weights as float64 once, so the oracle does not convert them on every call."""
    return {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}


def gpu_positions(tok, grid, off):
    b = H.B()
    Bn, L = tok.shape
    pos = torch.empty((3, Bn, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    status = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    b.compass_mrope_positions(H.ints_to_dev(tok), W.IMAGE_TOKEN_ID, H.ints_to_dev(grid), H.ints_to_dev(off), 2,
                              pos, delta, status)
    return pos, delta, status


@pytest.fixture(scope="module")
def sliding_case():
    """The sliding-layer workload (hidden 2048, 16/4 heads, hd 128, I 8192, window 1024,
    L = 4096 = 64 text + 1024 image + 3008 text) and its whole fp64 oracle result."""
    cfg = WORKLOADS["sliding_prefill"]
    sh, L = cfg["shape"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.SLIDING_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.SLIDING_PREFILL, L).reshape(1, L, sh.hidden)
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.SLIDING_PREFILL, 0, W.TensorId.TOKENS))
    ref_pos, ref_delta = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    ref, st = O.layer_prefill(sh, f64w(w), x, ref_pos, return_stages=True)
    return dict(sh=sh, L=L, w=w, x=x, tok=tok, grid=grid, off=off, ref_pos=ref_pos, ref_delta=ref_delta,
                ref=ref, st=st)


def test_sliding_prefill_full_size(sliding_case):
    """The whole [4096, 2048] output against the oracle (bench's call: no cache), the K/V cache
    written by the same layer with a cache, and every row's attention output on its own scale
    (rows 1024.. are those whose window no longer reaches key 0)."""
    c = sliding_case
    sh, L, w, x = c["sh"], c["L"], c["w"], c["x"]
    pos, delta, status = gpu_positions(c["tok"], c["grid"], c["off"])
    wd, xd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16)
    out = H.run_prefill(sh, wd, xd, pos)
    kc = torch.full((1, sh.n_kv_heads, L, sh.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out_kv = H.run_prefill(sh, wd, xd, pos, kv=(kc, vc))
    probe = H.run_prefill(sh, H.weights_to_dev(sh, probe_weights(sh, w)), xd, pos)
    torch.cuda.synchronize()
    assert status.item() == 0
    assert np.array_equal(pos.cpu().numpy(), c["ref_pos"]) and delta.item() == c["ref_delta"][0]
    e_out, e_br = check_layer_out(sh, out, x, c["ref"], "sliding layer")
    assert torch.equal(out, out_kv)
    assert H.rel_err(H.np64(kc), c["st"]["k"]) <= H.tol(sh)
    assert H.rel_err(H.np64(vc), c["st"]["v"]) <= H.tol(sh)
    e_att = check_attn_rows(sh, probe, x, c["st"]["attn"], "sliding layer")
    print(f"sliding full size: out {e_out:.2e} branch {e_br:.2e} attention rows {e_att:.2e}")


def test_chunked_prefill_full_size(sliding_case):
    """The same row as 4 chunks of 1024 tokens, each continuing the dense cache (the chunked
    workload bench.py times): every output row against the oracle's whole-row prefill (a chunk
    over the first tokens' cache is that prefill, pinned on the CPU), every row's attention
    output through the probe layer, and the cache against the one a single prefill of the row
    writes (the projection's arithmetic per element does not depend on the rows in the
    launch, so bitwise)."""
    c = sliding_case
    sh, L, w, x = c["sh"], c["L"], c["w"], c["x"]
    pos, _, status = gpu_positions(c["tok"], c["grid"], c["off"])
    xd = H.to_dev(x, torch.bfloat16)
    n_chunks, Lc = 4, L // 4

    def chunked(wd):
        kc = torch.full((1, sh.n_kv_heads, L, sh.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        outs = []
        for i in range(n_chunks):
            lens = H.ints_to_dev(np.array([i * Lc], dtype=np.int32))
            outs.append(H.run_prefill_chunk(sh, wd, xd[:, i * Lc:(i + 1) * Lc].contiguous(),
                                            pos[:, :, i * Lc:(i + 1) * Lc].contiguous(), kc, vc, lens))
        return torch.cat(outs, dim=1), kc, vc

    wd = H.weights_to_dev(sh, w)
    got, kc, vc = chunked(wd)
    probe, _, _ = chunked(H.weights_to_dev(sh, probe_weights(sh, w)))
    kf, vf = torch.empty_like(kc), torch.empty_like(vc)
    H.run_prefill(sh, wd, xd, pos, kv=(kf, vf))
    torch.cuda.synchronize()
    assert status.item() == 0
    assert torch.equal(kc, kf) and torch.equal(vc, vf)
    check_layer_out(sh, got, x, c["ref"], "chunked row")
    check_attn_rows(sh, probe, x, c["st"]["attn"], "chunked row")


def test_full_attention_prefill_full_size_and_relabel_invariance():
    """Full (NoPE) layer, B = 2, L = 8192: both rows whole against the oracle, every row's
    attention output through the probe layer, and bitwise invariance to permuted position ids."""
    cfg = WORKLOADS["full_prefill"]
    sh, Bn, L = cfg["shape"], cfg["B"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.FULL_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.FULL_PREFILL, Bn * L).reshape(Bn, L, sh.hidden)
    wd, xd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16)
    ar = np.broadcast_to(np.arange(L, dtype=np.int32), (3, Bn, L)).copy()
    perm = np.stack([np.stack([W.permutation(stream_seed(W.Stream.FULL_PREFILL, 3 * b + a, W.TensorId.PERM), L)
                               for b in range(Bn)]) for a in range(3)]).astype(np.int32)
    o0 = H.run_prefill(sh, wd, xd, None)
    o1 = H.run_prefill(sh, wd, xd, H.ints_to_dev(ar))
    o2 = H.run_prefill(sh, wd, xd, H.ints_to_dev(perm))
    probe = H.run_prefill(sh, H.weights_to_dev(sh, probe_weights(sh, w)), xd, None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o0, o1)
    ref, st = O.layer_prefill(sh, f64w(w), x, None, return_stages=True)
    e_out, e_br = check_layer_out(sh, o0, x, ref, "full layer")
    e_att = check_attn_rows(sh, probe, x, st["attn"], "full layer")
    print(f"full layer full size: out {e_out:.2e} branch {e_br:.2e} attention rows {e_att:.2e}")


def test_batched_decode_stack_full_size():
    """4 layers [S, S, S, F], B = 64, cache 8192, window 4096: one decode step. Each layer's
    64 rows against the oracle run on that layer's own input (the sliding layers merge 16
    chunks of 256 keys plus the new key, the full layer 33), its new K/V rows, and every
    row's attention output through the probe layer on the same cache; then the stack's
    output against the oracle's own 4-layer chain."""
    cfg = WORKLOADS["decode_stack"]
    sh, Bn, n_layers, n = cfg["shape"], cfg["B"], cfg["layers"], cfg["cache_len"]
    cap = n + 8
    Hkv, hd = sh.n_kv_heads, sh.head_dim
    x = W.make_layer_input(sh, W.Stream.DECODE_STACK, Bn)
    lens_np = np.full(Bn, n, np.int32)
    pos_np = O.decode_positions(lens_np, np.zeros(Bn, np.int64)).astype(np.int32)
    h = H.to_dev(x, torch.bfloat16)
    lens, pos = H.ints_to_dev(lens_np), H.ints_to_dev(pos_np)
    hx = x.astype(np.float64)
    worst = []
    for i in range(n_layers):
        shi = dataclasses.replace(sh, kind=S.layer_kind(i))
        sh_ref = dataclasses.replace(sh, kind=O.layer_kind(i))
        w = W.make_layer_weights(shi, W.Stream.DECODE_STACK, i)
        kc = RT.normal(stream_seed(W.Stream.DECODE_STACK, i, W.TensorId.K_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
        vc = RT.normal(stream_seed(W.Stream.DECODE_STACK, i, W.TensorId.V_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
        # Cache contents before the step (inputs); the oracle reads only indices < lens.
        k_in = kc[:, :, :n].float().cpu().numpy()
        v_in = vc[:, :, :n].float().cpu().numpy()
        h_in = h.clone()
        probe = H.run_decode(shi, H.weights_to_dev(shi, probe_weights(sh, w)), h_in, pos, kc, vc, lens)
        H.run_decode(shi, H.weights_to_dev(shi, w), h, pos, kc, vc, lens, out=h)
        torch.cuda.synchronize()
        wf = f64w(w)
        hin = H.np64(h_in)
        own, knew, vnew = O.layer_decode(sh_ref, wf, hin, pos_np, k_in, v_in, lens_np)
        check_layer_out(sh, h, hin, own, f"decode layer {i}")
        assert H.rel_err(H.np64(kc[:, :, n]), knew) <= 2e-2, f"layer {i} new K"
        assert H.rel_err(H.np64(vc[:, :, n]), vnew) <= 2e-2, f"layer {i} new V"
        ref_p, _, _ = O.layer_decode(sh_ref, f64w(probe_weights(sh, w)), hin, pos_np, k_in, v_in, lens_np)
        worst.append(check_attn_rows(sh, probe, hin, (ref_p - hin) / PROBE_SCALE, f"decode layer {i}"))
        hx, _, _ = O.layer_decode(sh_ref, wf, hx, pos_np, k_in, v_in, lens_np)
        del kc, vc, k_in, v_in
    e = H.rel_err(H.np64(h), hx)
    assert e <= 2e-2, e
    print(f"decode stack: out {e:.2e}, attention rows per layer {[f'{v:.2e}' for v in worst]}")


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_compass_widths_odd_batch(kind):
    """One decode layer at the Compass widths with B = 37 rows (the decode GEMMs' 64-row tiles
    hold 27 clamped rows) and ragged cache lengths 0 .. 1500 (window 1024 on the sliding
    layer): every row against the oracle, the attention through the probe layer on its own
    scale, and the new K/V rows."""
    cfg = WORKLOADS["decode_stack"]
    sh = dataclasses.replace(cfg["shape"], kind=kind, window=1024)
    Bn, cap = 37, 1504
    Hkv, hd = sh.n_kv_heads, sh.head_dim
    rng = np.random.default_rng(37)
    lens_np = np.sort(rng.integers(0, cap - 3, Bn)).astype(np.int32)
    lens_np[0], lens_np[-1] = 0, cap - 4
    delta = rng.integers(-50, 50, Bn).astype(np.int64)
    pos_np = O.decode_positions(lens_np, delta).astype(np.int32)
    w = W.make_layer_weights(sh, W.Stream.DECODE_STACK, 5)
    x = W.make_layer_input(sh, W.Stream.DECODE_STACK, Bn, layer=5)
    kc = RT.normal(stream_seed(W.Stream.DECODE_STACK, 5, W.TensorId.K_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
    vc = RT.normal(stream_seed(W.Stream.DECODE_STACK, 5, W.TensorId.V_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
    k_in, v_in = kc.float().cpu().numpy(), vc.float().cpu().numpy()
    lens, pos = H.ints_to_dev(lens_np), H.ints_to_dev(pos_np)
    xd = H.to_dev(x, torch.bfloat16)
    probe = H.run_decode(sh, H.weights_to_dev(sh, probe_weights(sh, w)), xd, pos, kc.clone(), vc.clone(), lens)
    out = H.run_decode(sh, H.weights_to_dev(sh, w), xd, pos, kc, vc, lens)
    torch.cuda.synchronize()
    sh_ref = dataclasses.replace(sh, kind=O.layer_kind(0 if kind == "sliding" else 3))
    xin = H.np64(xd)
    ref, knew, vnew = O.layer_decode(sh_ref, f64w(w), xin, pos_np, k_in, v_in, lens_np)
    check_layer_out(sh, out, xin, ref, f"{kind} decode, B = 37")
    ref_p, _, _ = O.layer_decode(sh_ref, f64w(probe_weights(sh, w)), xin, pos_np, k_in, v_in, lens_np)
    e_att = check_attn_rows(sh, probe, xin, (ref_p - xin) / PROBE_SCALE, f"{kind} decode, B = 37")
    kg, vg = H.np64(kc), H.np64(vc)
    for i, n in enumerate(lens_np):
        assert H.rel_err(kg[i, :, n], knew[i]) <= 2e-2, f"row {i} new K"
        assert H.rel_err(vg[i, :, n], vnew[i]) <= 2e-2, f"row {i} new V"
    print(f"{kind} decode at the Compass widths, B = 37: attention rows {e_att:.2e}")


def test_stack_prefill_deepstack_logits_full_size():
    """4-layer [S, S, S, F] prefill, L = 4096, deepstack after layers 0-2, 256000-vocab logits x 0.0625:
    the whole stack output against oracle.stack_prefill; the logits of six rows over 7168 vocabulary
    columns (the first 2048, the last 1024 and 4096 spread at random) against oracle.logits."""
    cfg = WORKLOADS["stack_logits"]
    sh, L, n_layers, V, scale = cfg["shape"], cfg["L"], cfg["layers"], cfg["vocab"], cfg["logit_scale"]
    D = sh.hidden
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.TOKENS))
    pos_np, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    x = W.make_layer_input(sh, W.Stream.STACK_LOGITS, L).reshape(1, L, D)
    ds = [W.make_tensor(sh, 4, i, W.TensorId.DS + i, (1024, D)) for i in range(3)]
    ds_rows = np.arange(64, 64 + 1024, dtype=np.int32)
    ws = [W.make_layer_weights(dataclasses.replace(sh, kind=S.layer_kind(i)), W.Stream.STACK_LOGITS, i)
          for i in range(n_layers)]
    nw = W.make_tensor(sh, 4, 0, W.TensorId.FINAL_LN, (D,), std=0.02, mean=1.0)
    E = RT.normal(stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.EMBED), V * D, std=0.02).to(torch.bfloat16).view(V, D)
    pos = H.ints_to_dev(pos_np)
    h = H.to_dev(x, torch.bfloat16)
    rows_d = H.ints_to_dev(ds_rows)
    for i in range(n_layers):
        shi = dataclasses.replace(sh, kind=S.layer_kind(i))
        use = S.takes_deepstack(i)
        H.run_prefill(shi, H.weights_to_dev(shi, ws[i]), h, pos, ds_rows=rows_d if use else None,
                      ds=H.to_dev(ds[i], torch.bfloat16) if use else None, out=h)
    logits = H.run_logits(h.view(L, D), H.to_dev(nw, torch.bfloat16), sh.ln_eps, E, scale, 1)
    torch.cuda.synchronize()
    ref_h = O.stack_prefill(sh, [f64w(w) for w in ws], x, pos_np, ds_rows, ds)[0]
    check_layer_out(sh, h[0], x[0], ref_h, "stack")
    rows = [0, 64, 1087, 1088, 2500, 4095]
    cols = np.concatenate([np.arange(0, 2048), np.arange(V - 1024, V),
                           np.random.default_rng(0).integers(0, V, 4096)])
    Ecols = H.np64(E[torch.from_numpy(cols).cuda()])
    ref_l = O.logits(ref_h[rows], nw, sh.ln_eps, Ecols, scale)
    got_l = H.np64(logits[rows][:, torch.from_numpy(cols).cuda()])
    e = H.rel_err(got_l, ref_l)
    assert e <= 2e-2, e
