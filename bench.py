"""Benchmark of the Compass/Cohere2 parallel decoder layer on one MI355X.

Timed step (the headline): the sliding-layer prefill workload — hidden 2048, 16/4
heads, head_dim 128, SwiGLU 8192, window 1024, MRoPE [24, 20, 20], one row of 4096
tokens laid out as 64 text + 1024 image (patch grid 1 x 64 x 64, merge 2) + 3008
text — i.e. compass_mrope_positions followed by compass_layer_prefill on inputs
already resident in HBM. value = tokens per second per layer.

Also reported (one JSON line, key "extra"): the full-attention prefill (B=2, L=8192),
batched decode of a 4-layer 3:1 stack (B=64, cache 8192, window 4096) in us/step,
the 4-layer stack prefill with deepstack plus tied 256000-vocab logits, and the
headline row prefilled as 4 chunks continuing the KV cache.

"roofline" describes the dominant kernel of the headline step (the fused projection
GEMM): algorithmic flops per launch / its mean launch time from HIP events recorded
around every launch while the timed steps are repeated (the throughput itself is timed
without the events). "traffic" is its HBM bytes per launch from committed rocprofv3
counter passes (profiles/gemm_proj_sliding_prefill_traffic.json) while they match the current kernel
sources. "cpu_baseline" is the plain fp32 C++ oracle (OpenMP) timed on this host on one
whole layer of the same workload, with the host's CPU model, nproc and the threads used,
and the fp64 numpy oracle on that layer as a second figure. "extra" also holds the tiny
fp32 layer (hidden 256, L = 128) on the GPU and on the C++ oracle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-extra", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only", default=None, help="run one workload: sliding_prefill|tiny_f32|full_prefill|decode_stack|stack_logits|chunked_prefill|varlen_prefill (for profiling)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run plain 512 MiB copies (reference launches for the HBM byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_stats(b, names):
    out = {}
    for n in names:
        c, ms = b.compass_profile_read(n)
        if c:
            out[n] = {"launches": c, "mean_us": 1e3 * ms / c}
    return out


def timed(fn, steps, warmup, b, torch):
    """Warm up, then time `steps` steps twice on the same inputs: first plain (the step
    time reported as throughput), then with a HIP event pair recorded around every library
    launch (per-kernel mean durations for the roofline; the events cost a few percent of
    the step, so they stay out of the throughput figure)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    b.compass_profile_reset()
    b.compass_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    b.compass_profile_enable(False)
    stats = kernel_stats(b, b.compass_profile_kernel_names())
    return sec, stats


# ------------------------------------------------------------------------ workloads
def setup_sliding_prefill(H, W, torch):
    from synth.workloads import WORKLOADS
    cfg = WORKLOADS["sliding_prefill"]
    sh = cfg["shape"]
    L = cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.SLIDING_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.SLIDING_PREFILL, L).reshape(1, L, sh.hidden)
    tok, grid, off = W.image_text_row(W.stream_seed(W.Stream.SLIDING_PREFILL, 0, W.TensorId.TOKENS))
    return sh, w, x, tok, grid, off


def run_sliding_prefill(args, b, H, W, torch):
    sh, w, x, tok, grid, off = setup_sliding_prefill(H, W, torch)
    L = x.shape[1]
    wd = H.weights_to_dev(sh, w)
    xd = H.to_dev(x, torch.bfloat16)
    tokd, gridd, offd = H.ints_to_dev(tok), H.ints_to_dev(grid), H.ints_to_dev(off)
    pos = torch.empty((3, 1, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((1,), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(xd)
    d = H.desc(sh)
    ws = H.workspace(b.compass_workspace_size(d, 1, L, 0, 0))
    wts = b.make_weights(wd)

    def step():
        b.compass_mrope_positions(tokd, W.IMAGE_TOKEN_ID, gridd, offd, 2, pos, delta, status)
        b.compass_layer_prefill(d, wts, xd, pos, None, None, None, out, ws)

    sec, stats = timed(step, args.steps, args.warmup, b, torch)
    assert int(status.item()) == 0
    return sh, w, x, tok, grid, off, sec, stats


def layer_flops(sh, L):
    D, Hq, Hkv, hd, I = sh.hidden, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.intermediate
    nv = (Hq + 2 * Hkv) * hd + 2 * I
    proj = 2.0 * L * D * nv
    out = 2.0 * L * (Hq * hd + I) * D
    pairs = sum(min(i + 1, sh.window) for i in range(L)) if sh.kind == "sliding" else L * (L + 1) / 2
    attn = 4.0 * pairs * Hq * hd
    return proj, out, attn


def run_full_prefill(args, b, H, W, torch):
    from synth.workloads import WORKLOADS
    cfg = WORKLOADS["full_prefill"]
    sh, Bn, L = cfg["shape"], cfg["B"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.FULL_PREFILL, 0)
    import synth.rng_torch as RT
    x = RT.normal(W.stream_seed(W.Stream.FULL_PREFILL, 0, W.TensorId.X), Bn * L * sh.hidden).to(torch.bfloat16).view(Bn, L, sh.hidden)
    wd = H.weights_to_dev(sh, w)
    d = H.desc(sh)
    ws = H.workspace(b.compass_workspace_size(d, Bn, L, 0, 0))
    out = torch.empty_like(x)
    wts = b.make_weights(wd)
    step = lambda: b.compass_layer_prefill(d, wts, x, None, None, None, None, out, ws)
    sec, stats = timed(step, max(3, args.steps // 4), 2, b, torch)
    proj, outf, attn = [Bn * f for f in layer_flops(sh, L)]
    return {"workload": cfg["name"], "tokens_per_s_per_layer": Bn * L / sec, "ms_per_layer": 1e3 * sec,
            "mfma_frac_layer": (proj + outf + attn) / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()}}


def run_decode_stack(args, b, H, W, torch):
    from synth.workloads import WORKLOADS
    from cohere2_block_mrope_amd.stack import layer_kind
    import dataclasses
    import synth.rng_torch as RT
    cfg = WORKLOADS["decode_stack"]
    sh, Bn, n_layers, n = cfg["shape"], cfg["B"], cfg["layers"], cfg["cache_len"]
    cap = n + 8
    Hkv, hd = sh.n_kv_heads, sh.head_dim
    layers = []
    for i in range(n_layers):
        shi = dataclasses.replace(sh, kind=layer_kind(i))
        wd = H.weights_to_dev(shi, W.make_layer_weights(shi, W.Stream.DECODE_STACK, i))
        kc = RT.normal(W.stream_seed(W.Stream.DECODE_STACK, i, W.TensorId.K_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
        vc = RT.normal(W.stream_seed(W.Stream.DECODE_STACK, i, W.TensorId.V_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
        d = H.desc(shi)
        ws = H.workspace(b.compass_workspace_size(d, Bn, 1, cap, 1))
        layers.append((d, b.make_weights(wd), wd, kc, vc, ws))
    x = RT.normal(W.stream_seed(W.Stream.DECODE_STACK, 0, W.TensorId.X), Bn * sh.hidden).to(torch.bfloat16).view(Bn, sh.hidden)
    lens = torch.full((Bn,), n, dtype=torch.int32, device="cuda")
    pos = torch.full((3, Bn), n, dtype=torch.int32, device="cuda")
    h = torch.empty_like(x)
    # The layers run chained: each layer's residual kernel also writes the next layer's
    # LayerNorm of its output, which the next layer reads instead of running its LayerNorm
    # kernel. The same step as independent compass_layer_decode calls is timed beside it.
    nrm = torch.empty_like(x)

    def decode_layers(final_w=None):
        """The chained layers; with final_w the last layer also hands over the final LayerNorm."""
        last = len(layers) - 1
        for i, (d, wts, _, kc, vc, ws) in enumerate(layers):
            nxt = final_w if i == last else layers[i + 1][2]["ln_w"]
            b.compass_layer_decode_chained(d, wts, h, None if i == 0 else nrm, pos, b.make_kv(kc, vc, lens), h,
                                           nxt, sh.ln_eps, None if nxt is None else nrm, ws)

    def step():
        h.copy_(x)
        decode_layers()

    def step_unchained():
        h.copy_(x)
        for d, wts, _, kc, vc, ws in layers:
            b.compass_layer_decode(d, wts, h, pos, b.make_kv(kc, vc, lens), h, ws)

    sec, stats = timed(step, max(5, args.steps), 3, b, torch)
    sec_u, stats_u = timed(step_unchained, max(5, args.steps), 3, b, torch)

    # A whole greedy decode step: embed the 64 tokens, decode positions, the 4 layers, then
    # the tied 256000-vocab head reduced to the next token ids, which feed the next step.
    # lens is not advanced (advance 0), so every timed step does the same work.
    V = WORKLOADS["stack_logits"]["vocab"]
    E = RT.normal(W.stream_seed(W.Stream.DECODE_STACK, 0, W.TensorId.EMBED), V * sh.hidden, std=0.02).to(torch.bfloat16).view(V, sh.hidden)
    nw = RT.normal(W.stream_seed(W.Stream.DECODE_STACK, 0, W.TensorId.FINAL_LN), sh.hidden, std=0.02, mean=1.0).to(torch.bfloat16)
    tok = torch.arange(Bn, dtype=torch.int32, device="cuda") * 17
    delta = torch.zeros((Bn,), dtype=torch.int32, device="cuda")
    gws = H.workspace(b.compass_logits_argmax_workspace_size(Bn, sh.hidden, V, 1))
    est = torch.zeros((1,), dtype=torch.int32, device="cuda")

    def greedy_step():
        b.compass_embed(tok, E, None, None, h, est, 1)
        b.compass_decode_positions(lens, delta, 0, pos)
        decode_layers(final_w=nw)  # the greedy head takes the final LayerNorm from the last layer
        b.compass_logits_argmax(nrm, None, sh.ln_eps, E, WORKLOADS["stack_logits"]["logit_scale"], tok, None, gws, 1)

    sec_g, stats_g = timed(greedy_step, max(5, args.steps), 3, b, torch)
    assert int(est.item()) == 0

    # The same decode step with 4-bit affine weights (group 64) in the four layers.
    # The ctypes structs hold raw device pointers: q4_dev keeps the tensors alive.
    q4_dev = [H.q4_to_dev(W.make_layer_weights_q4(dataclasses.replace(sh, kind=layer_kind(i)), W.Stream.DECODE_STACK, i))
              for i in range(n_layers)]
    q4 = [b.make_weights_q4(wd) for wd in q4_dev]

    def q4_step():
        h.copy_(x)
        for (d, _, _, kc, vc, ws), wq in zip(layers, q4):
            b.compass_layer_decode_q4(d, wq, h, pos, b.make_kv(kc, vc, lens), h, ws)

    sec_q, stats_q = timed(q4_step, max(5, args.steps), 3, b, torch)
    kv_bytes_slide = Bn * Hkv * sh.window * hd * 2 * 2
    kv_bytes_full = Bn * Hkv * (n + 1) * hd * 2 * 2
    w_bytes = 2 * (sh.hidden * ((sh.n_q_heads + 2 * Hkv) * hd + 2 * sh.intermediate)
                   + (sh.n_q_heads * hd + sh.intermediate) * sh.hidden)
    step_bytes = 3 * kv_bytes_slide + kv_bytes_full + n_layers * w_bytes
    att = stats.get("decode_attn", {})
    att_bytes_mean = (3 * kv_bytes_slide + kv_bytes_full) / 4
    res = {"workload": cfg["name"], "us_per_step": 1e6 * sec, "hbm_frac_step": step_bytes / sec / 1e9 / HBM_PEAK_GBS,
           "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()},
           "unchained": {"us_per_step": 1e6 * sec_u,
                         "what": "the same step as four independent compass_layer_decode calls (each runs its "
                                 "own LayerNorm kernel)",
                         "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats_u.items()}}}
    if att:
        res["decode_attn_hbm_frac"] = att_bytes_mean / (att["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
    # HBM bytes per decode-attention launch from the committed counter passes (null once the
    # kernel's sources have changed since), next to the algorithmic bytes.
    res["decode_attn_traffic"] = {
        "sliding": {"hbm_bytes": traffic_for("decode_attn_sliding_decode_stack", DECODE_SOURCES),
                    "algorithmic_bytes": kv_bytes_slide},
        "full": {"hbm_bytes": traffic_for("decode_attn_full_decode_stack", DECODE_SOURCES),
                 "algorithmic_bytes": kv_bytes_full}}
    q4_bytes_proj = (sh.hidden // 2 + 4 * (sh.hidden // 64)) * ((sh.n_q_heads + 2 * Hkv) * hd + 2 * sh.intermediate)
    K2 = sh.n_q_heads * hd + sh.intermediate
    q4_bytes_out = (K2 // 2 + 4 * (K2 // 64)) * sh.hidden
    res["q4_step"] = {"us_per_step": 1e6 * sec_q,
                      "what": "the same 4-layer decode step with 4-bit affine weights (group 64)",
                      "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats_q.items()}}
    for name, nbytes in (("gemm_proj_decode_q4", q4_bytes_proj), ("gemm_out_decode_q4", q4_bytes_out)):
        st = stats_q.get(name)
        if st:
            res["q4_step"][name + "_weight_hbm_frac"] = nbytes / (st["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
    lg = stats_g.get("gemm_logits_argmax", {})
    res["greedy_step"] = {"us_per_step": 1e6 * sec_g,
                          "what": "embed + decode positions + the 4 chained layers (the last one writing the "
                                  "final LayerNorm) + tied 256000-vocab logits argmax",
                          "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats_g.items()
                                         if k in ("embed", "decode_positions", "logits_layernorm",
                                                  "gemm_logits_argmax", "argmax")}}
    if lg:
        res["greedy_step"]["logits_hbm_frac"] = V * sh.hidden * 2 / (lg["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS
    return res


def run_stack_logits(args, b, H, W, torch):
    from synth.workloads import WORKLOADS
    from cohere2_block_mrope_amd.stack import layer_kind
    import dataclasses
    import synth.rng_torch as RT
    cfg = WORKLOADS["stack_logits"]
    sh, L, n_layers, V, scale = cfg["shape"], cfg["L"], cfg["layers"], cfg["vocab"], cfg["logit_scale"]
    tok, grid, off = W.image_text_row(W.stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.TOKENS))
    pos = torch.empty((3, 1, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((1,), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    b.compass_mrope_positions(H.ints_to_dev(tok), W.IMAGE_TOKEN_ID, H.ints_to_dev(grid), H.ints_to_dev(off), 2,
                              pos, delta, status)
    assert int(status.item()) == 0
    layers = []
    for i in range(n_layers):
        shi = dataclasses.replace(sh, kind=layer_kind(i))
        wd = H.weights_to_dev(shi, W.make_layer_weights(shi, W.Stream.STACK_LOGITS, i))
        layers.append((H.desc(shi), b.make_weights(wd), wd))
    x = RT.normal(W.stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.X), L * sh.hidden).to(torch.bfloat16).view(1, L, sh.hidden)
    ds = [RT.normal(W.stream_seed(W.Stream.STACK_LOGITS, i, W.TensorId.DS + i), 1024 * sh.hidden).to(torch.bfloat16).view(1024, sh.hidden)
          for i in range(3)]
    ds_rows = torch.arange(64, 64 + 1024, dtype=torch.int32, device="cuda")
    E = RT.normal(W.stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.EMBED), V * sh.hidden, std=0.02).to(torch.bfloat16).view(V, sh.hidden)
    nw = RT.normal(W.stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.FINAL_LN), sh.hidden, std=0.02, mean=1.0).to(torch.bfloat16)
    ws = H.workspace(max(b.compass_workspace_size(layers[0][0], 1, L, 0, 0),
                         b.compass_logits_workspace_size(L, sh.hidden, 1)))
    h = torch.empty_like(x)
    logits = torch.empty((L, V), dtype=torch.float32, device="cuda")

    def step():
        h.copy_(x)
        for i, (d, wts, _) in enumerate(layers):
            use = i < 3
            b.compass_layer_prefill(d, wts, h, pos, None, ds_rows if use else None, ds[i] if use else None, h, ws)
        b.compass_logits(h.view(L, sh.hidden), nw, sh.ln_eps, E, scale, logits, ws, 1)

    sec, stats = timed(step, max(3, args.steps // 4), 2, b, torch)
    lg = stats.get("gemm_logits", {})
    res = {"workload": cfg["name"], "ms_per_step": 1e3 * sec,
           "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()}}
    if lg:
        res["logits_mfma_frac"] = 2.0 * L * sh.hidden * V / (lg["mean_us"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    return res


def run_chunked_prefill(args, b, H, W, torch):
    """The headline row prefilled as 4 chunks of 1024 tokens, each continuing the dense cache
    (compass_layer_prefill_chunk; positions from the whole row), against one prefill of the
    row writing the same cache."""
    sh, w, x, tok, grid, off = setup_sliding_prefill(H, W, torch)
    L = x.shape[1]
    n_chunks, Lc = 4, L // 4
    wd = H.weights_to_dev(sh, w)
    xd = H.to_dev(x, torch.bfloat16)
    pos = torch.empty((3, 1, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((1,), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    b.compass_mrope_positions(H.ints_to_dev(tok), W.IMAGE_TOKEN_ID, H.ints_to_dev(grid), H.ints_to_dev(off), 2,
                              pos, delta, status)
    assert int(status.item()) == 0
    cap = L
    kc = torch.empty((1, sh.n_kv_heads, cap, sh.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    d = H.desc(sh)
    wts = b.make_weights(wd)
    ws = H.workspace(b.compass_workspace_size(d, 1, L, 0, 0))
    out = torch.empty_like(xd)
    xs = [xd[:, i * Lc:(i + 1) * Lc].contiguous() for i in range(n_chunks)]
    ps = [pos[:, :, i * Lc:(i + 1) * Lc].contiguous() for i in range(n_chunks)]
    outs = [torch.empty_like(t) for t in xs]
    starts = [torch.full((1,), i * Lc, dtype=torch.int32, device="cuda") for i in range(n_chunks)]
    kvs = [b.make_kv(kc, vc, s_) for s_ in starts]
    kv0 = b.make_kv(kc, vc)

    def chunked():
        for i in range(n_chunks):
            b.compass_layer_prefill_chunk(d, wts, xs[i], ps[i], kvs[i], None, None, outs[i], ws)

    def whole():
        b.compass_layer_prefill(d, wts, xd, pos, kv0, None, None, out, ws)

    sec_c, stats = timed(chunked, args.steps, args.warmup, b, torch)
    sec_w, _ = timed(whole, args.steps, args.warmup, b, torch)
    return {"workload": f"chunked prefill of the sliding-layer headline row: {n_chunks} chunks of {Lc} tokens "
                        f"continuing the dense cache",
            "ms_per_row_chunked": 1e3 * sec_c, "ms_per_row_one_prefill": 1e3 * sec_w,
            "tokens_per_s_chunked": L / sec_c,
            "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()}}


def run_varlen_prefill(args, b, H, W, torch):
    """Varlen prefill of the sliding layer (headline widths, window 1024): 8 sequences of
    1536, 1024, 512, 384, 256, 200, 128 and 56 tokens (4096 in all, text positions per
    sequence) packed into one launch, each written to its own cache."""
    sh, w, _, _, _, _ = setup_sliding_prefill(H, W, torch)
    lens = [1536, 1024, 512, 384, 256, 200, 128, 56]
    T = sum(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    pos = torch.from_numpy(np.concatenate([np.broadcast_to(np.arange(n), (3, n)) for n in lens], axis=1)
                           .astype(np.int32)).cuda()
    import synth.rng_torch as RT
    x = RT.normal(W.stream_seed(W.Stream.SLIDING_PREFILL, 1, W.TensorId.X), T * sh.hidden).to(torch.bfloat16).view(T, sh.hidden)
    wd = H.weights_to_dev(sh, w)
    d = H.desc(sh)
    kc = torch.empty((len(lens), sh.n_kv_heads, max(lens), sh.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kv = b.make_kv(kc, vc)
    ws = H.workspace(b.compass_varlen_workspace_size(d, len(lens), T))
    out = torch.empty_like(x)
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    wts = b.make_weights(wd)
    step = lambda: b.compass_layer_prefill_varlen(d, wts, cu, x, pos, kv, None, None, out, status, ws)
    sec, stats = timed(step, args.steps, args.warmup, b, torch)
    assert int(status.item()) == 0
    return {"workload": f"varlen prefill, sliding layer (headline widths, window 1024): {len(lens)} sequences "
                        f"of {lens} tokens packed into {T} rows, one launch per kernel, caches written",
            "ms_per_step": 1e3 * sec, "tokens_per_s_per_layer": T / sec,
            "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()}}


def cpu_info():
    """The host CPU's model string and the core count nproc reports."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count(), len(os.sched_getaffinity(0))


def cpu_baseline(sh, w, x, tok, grid, off):
    """The oracles (test infrastructure) timed on this host: the only use of oracle/ here.

    The figure is the plain fp32 C++ oracle (OpenMP over rows, queries and heads, as
    many threads as OMP_NUM_THREADS allows) on one whole layer of the headline workload,
    positions included. The fp64 numpy oracle on the same layer is a second figure."""
    import threadpoolctl
    from oracle import compass_oracle as O
    from oracle import ref as R
    from synth.workloads import IMAGE_TOKEN_ID
    model, ncpu, naff = cpu_info()
    L = x.shape[1]
    threads = R.num_threads()
    t0 = time.perf_counter()
    code, pos, _ = R.mrope_positions(tok, IMAGE_TOKEN_ID, grid, off, 2)
    R.layer_forward(sh, w, x, pos)
    sec = time.perf_counter() - t0
    assert code == 0
    info = threadpoolctl.threadpool_info()
    blas = max([i.get("num_threads", 1) for i in info] or [1])
    t1 = time.perf_counter()
    pos64, _ = O.mrope_positions(tok, IMAGE_TOKEN_ID, grid, off, 2)
    O.layer_prefill(sh, w, x, pos64)
    sec64 = time.perf_counter() - t1
    return {"value": L / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one whole sliding-layer prefill of the headline workload ({L} tokens, positions + layer) "
                      f"by the plain fp32 C++ oracle (double accumulation) on {threads} OpenMP threads: {sec:.1f} s",
            "cpu_model": model, "nproc": ncpu, "affinity_cpus": naff,
            "numpy_fp64": {"value": L / sec64, "unit": "tokens/s", "blas_threads": blas,
                           "sample": f"the same layer by the fp64 numpy oracle: {sec64:.1f} s"}}


def run_tiny_f32(args, b, H, W, torch):
    """The fp32 parity workload (hidden 256, 4/1 heads, hd 64, I 1024, window 32, MRoPE [12, 10, 10],
    128 text tokens): positions + one fp32 layer on the GPU, and the C++ oracle on the same layer."""
    from synth.workloads import WORKLOADS
    cfg = WORKLOADS["tiny_sliding_f32"]
    sh, L = cfg["shape"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.TINY_SLIDING_F32, 0)
    x = W.make_layer_input(sh, W.Stream.TINY_SLIDING_F32, L).reshape(1, L, sh.hidden)
    tok = W.text_tokens(W.stream_seed(W.Stream.TINY_SLIDING_F32, 0, W.TensorId.TOKENS), L).reshape(1, L)
    grid, off = np.zeros((1, 3), np.int32), np.zeros(2, np.int32)
    wd, xd = H.weights_to_dev(sh, w), H.to_dev(x, torch.float32)
    tokd, gridd, offd = H.ints_to_dev(tok), H.ints_to_dev(grid), H.ints_to_dev(off)
    pos = torch.empty((3, 1, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((1,), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(xd)
    d = H.desc(sh)
    ws = H.workspace(b.compass_workspace_size(d, 1, L, 0, 0))
    wts = b.make_weights(wd)

    def step():
        b.compass_mrope_positions(tokd, W.IMAGE_TOKEN_ID, gridd, offd, 2, pos, delta, status)
        b.compass_layer_prefill(d, wts, xd, pos, None, None, None, out, ws)

    sec, stats = timed(step, max(20, args.steps), 5, b, torch)
    assert int(status.item()) == 0
    res = {"workload": cfg["name"], "us_per_step": 1e6 * sec, "tokens_per_s_per_layer": L / sec,
           "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()}}
    if not args.no_cpu:
        from oracle import ref as R
        p = np.arange(L)
        t0 = time.perf_counter()
        for _ in range(3):
            R.layer_forward(sh, w, x, np.stack([p, p, p])[:, None, :])
        res["cpu_oracle_us_per_layer"] = 1e6 * (time.perf_counter() - t0) / 3
        res["cpu_oracle_threads"] = R.num_threads()
    return res


GEMM_SOURCES = ["gemm_bf16.hip", "gemm_common.h", "common.h", "launch.h"]
DECODE_SOURCES = ["decode.hip", "common.h", "launch.h"]


def traffic_for(name: str, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<name>_traffic.json), if it was taken on the current sources of the kernel;
    else None."""
    from cohere2_block_mrope_amd.pmc_traffic import source_digest
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_digest(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(torch, nbytes=512 << 20, copies=3):
    """Plain device-to-device copies of a known size: the reference launches for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(copies):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "copies": copies}


def achievable(torch, proj_shape):
    """What the box itself delivers, measured in the same run, beside the published peaks: a
    device-to-device copy of 1 GiB (read + write bytes over time) and the vendor bf16 GEMM
    (torch.matmul, 2-D and contiguous) on 8192^3 and on the projection's own shape (no epilogue).
    Each figure is the median of 10 timed calls after 3 warm-up calls."""
    def med(fn, n=10):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return t[n // 2] * 1e-3
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    copy_s = med(lambda: dst.copy_(src))
    del src, dst
    out = {"copy_read_write_TBps": 2 * nb / copy_s / 1e12}
    # Both operand layouts (B as [K, N], and as [N, K] read through a transposed 2-D view, the
    # layout of this library's weights); the faster one counts.
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    bm = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    t = min(med(lambda: torch.matmul(a, bm)), med(lambda: torch.matmul(a, bm.t())))
    out["vendor_gemm_bf16_8192cube_TFLOPs"] = 2 * n ** 3 / t / 1e12
    del a, bm
    M, K, N = proj_shape
    a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    w_kn = torch.randn(K, N, device="cuda").to(torch.bfloat16)
    w_nk = w_kn.t().contiguous()
    t = min(med(lambda: torch.matmul(a, w_kn)), med(lambda: torch.matmul(a, w_nk.t())))
    out["vendor_gemm_bf16_projection_shape"] = {"M": M, "K": K, "N": N, "us": t * 1e6,
                                                 "TFLOPs": 2 * M * K * N / t / 1e12}
    del a, w_kn, w_nk
    torch.cuda.empty_cache()
    return out


def proj_bytes(sh, L):
    """Algorithmic HBM bytes of one fused-projection launch: the normalized activations and
    the five weight matrices read once, q / k / v / SwiGLU output written once (bf16)."""
    D, Hq, Hkv, hd, I = sh.hidden, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.intermediate
    nv = (Hq + 2 * Hkv) * hd + 2 * I
    return 2.0 * (L * D + nv * D + L * ((Hq + 2 * Hkv) * hd + I))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design "
              f"note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from cohere2_block_mrope_amd import binding as b
    from synth import workloads as W
    from tests import helpers as H
    torch.cuda.set_device(0)

    res_extra = {}
    if args.only in (None, "sliding_prefill"):
        log("sliding_prefill: generating inputs")
        sh, w, x, tok, grid, off, sec, stats = run_sliding_prefill(args, b, H, W, torch)
        L = x.shape[1]
        proj, outf, attn = layer_flops(sh, L)
        gp = stats["gemm_proj"]
        achieved = proj / (gp["mean_us"] * 1e-6) / 1e12
        line = {
            "metric": "prefill tokens/s per layer + decode µs/step; % of MFMA / HBM peak",
            "value": L / sec, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": 1e3 * sec, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic: seeded N(0,0.02) weights, LayerNorm 1+N(0,0.02), N(0,1) hidden states",
            "config": {"workload": "sliding-layer prefill: D=2048, 16/4 heads, hd=128, I=8192, window=1024, "
                                   "MRoPE [24,20,20], B=1, L=4096 (64 text + 1024 image + 3008 text); "
                                   "step = position ids + one layer",
                       "global_batch": 1, "seq_len": L, "parallelism": "single GPU"},
            "layer_mfma_frac": (proj + outf + attn) / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "kernels_us": {k: round(v["mean_us"], 1) for k, v in stats.items()},
            "roofline": {"kernel": "gemm_proj (fused LN-input q/k/v/gate/up projection + MRoPE/SwiGLU epilogue)",
                         "bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": traffic_for("gemm_proj_sliding_prefill", GEMM_SOURCES),
                         "flops_per_launch": proj, "mean_launch_us": gp["mean_us"],
                         "algorithmic_bytes": proj_bytes(sh, L)},
        }
        # (Left out of counter passes: their own copies would mix with the calibration copies.)
        if not args.copy_calibration:
            Nv = (sh.n_q_heads + 2 * sh.n_kv_heads) * sh.head_dim + 2 * sh.intermediate
            ach = achievable(torch, (L, sh.hidden, Nv))
            line["roofline"]["measured_achievable"] = ach
            line["roofline"]["frac_of_vendor_gemm_8192cube"] = achieved / ach["vendor_gemm_bf16_8192cube_TFLOPs"]
        if not args.no_cpu:
            log("sliding_prefill: timing the CPU oracle")
            line["cpu_baseline"] = cpu_baseline(sh, w, x, tok, grid, off)
        else:
            line["cpu_baseline"] = None
    else:
        line = None
    if not args.no_extra:
        for key, fn in (("tiny_f32", run_tiny_f32), ("full_prefill", run_full_prefill),
                        ("decode_stack", run_decode_stack), ("stack_logits", run_stack_logits),
                        ("chunked_prefill", run_chunked_prefill), ("varlen_prefill", run_varlen_prefill)):
            if args.only in (None, key):
                log(f"{key}: running")
                res_extra[key] = fn(args, b, H, W, torch)
                torch.cuda.empty_cache()
    if args.copy_calibration:
        res_extra["copy_calibration"] = copy_calibration(torch)
    if line is None:
        print(json.dumps({"extra": res_extra}))
    else:
        line["extra"] = res_extra
        print(json.dumps(line))


if __name__ == "__main__":
    main()
