"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on the capture stream)
and replayed. The library allocates nothing, never synchronizes and records no memset, so
a whole step can be captured once and replayed.

Each replay is checked against the eager result bitwise (the kernels are deterministic),
with eager work of the program's own between the replays (the output and cache cleared,
an unrelated fp32 matmul) and a synchronization before every check.
"""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import workloads as W
from tests import helpers as H
from tests.test_gpu_small import layer_case, mixed_tokens

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _eager_noise():
    a = torch.randn(256, 256, device="cuda")
    return (a @ a.t()).sum()


def test_prefill_step_graph_replays_match_eager():
    """Position ids + one sliding layer (the headline step's structure) in one graph."""
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 48)
    Bn, L = 2, 200
    b = H.B()
    w, x, _ = layer_case(sh, Bn, L, seed=5)
    tok, grid, off = mixed_tokens(Bn, L, 5)
    wd = H.weights_to_dev(sh, w)
    wts = b.make_weights(wd)
    d = H.desc(sh)
    xd = H.to_dev(x, torch.bfloat16)
    tokd, gridd, offd = H.ints_to_dev(tok), H.ints_to_dev(grid), H.ints_to_dev(off)
    pos = torch.empty((3, Bn, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    status = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    kc = torch.zeros((Bn, sh.n_kv_heads, L, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kv = b.make_kv(kc, vc)
    out = torch.empty_like(xd)
    ws = H.workspace(b.compass_workspace_size(d, Bn, L, 0, 0))

    def step():
        b.compass_mrope_positions(tokd, W.IMAGE_TOKEN_ID, gridd, offd, 2, pos, delta, status)
        b.compass_layer_prefill(d, wts, xd, pos, kv, None, None, out, ws)

    step()  # eager (also sets the kernels' LDS attributes before any capture)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * Bn
    ref_out, ref_k, ref_v, ref_pos = out.clone(), kc.clone(), vc.clone(), pos.clone()
    ref_pos_np, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    np.testing.assert_array_equal(ref_pos.cpu().numpy(), ref_pos_np)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.zero_(); kc.zero_(); vc.zero_(); pos.fill_(-1)
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pos, ref_pos), f"replay {r}: positions"
        assert torch.equal(out, ref_out), f"replay {r}: layer output"
        assert torch.equal(kc, ref_k) and torch.equal(vc, ref_v), f"replay {r}: K/V cache"


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_step_graph_replays_match_eager(kind):
    sh = H.small_shape("bf16", kind, 128, 4, 1, 256, 512, 16)
    Bn, cap = 3, 40
    b = H.B()
    w, _, _ = layer_case(sh, 1, 8, seed=11)
    wd = H.weights_to_dev(sh, w)
    wts = b.make_weights(wd)
    d = H.desc(sh)
    x = H.to_dev(H.rand_np(12, (Bn, sh.hidden), bf16=True), torch.bfloat16)
    lens_np = np.array([0, 17, 39], np.int32)
    pos = H.ints_to_dev(O.decode_positions(lens_np, np.array([0, -3, 5])))
    lens = H.ints_to_dev(lens_np)
    kc = H.to_dev(H.rand_np(13, (Bn, sh.n_kv_heads, cap, 128), bf16=True), torch.bfloat16)
    vc = H.to_dev(H.rand_np(14, (Bn, sh.n_kv_heads, cap, 128), bf16=True), torch.bfloat16)
    kc0, vc0 = kc.clone(), vc.clone()
    kv = b.make_kv(kc, vc, lens)
    out = torch.empty_like(x)
    ws = H.workspace(b.compass_workspace_size(d, Bn, 1, cap, 1))

    def step():
        b.compass_layer_decode(d, wts, x, pos, kv, out, ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_k, ref_v = out.clone(), kc.clone(), vc.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.zero_()
        kc.copy_(kc0); vc.copy_(vc0)  # the appended rows are written again by the replay
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: layer output"
        assert torch.equal(kc, ref_k) and torch.equal(vc, ref_v), f"replay {r}: K/V cache"


def test_chained_decode_graph_replays_match_eager():
    """Two chained decode layers (sliding, then full; the first hands the second its
    LayerNorm) captured as one graph."""
    shapes = [H.small_shape("bf16", k, 128, 4, 1, 256, 512, 16) for k in ("sliding", "full")]
    Bn, cap = 3, 40
    b = H.B()
    wd = [H.weights_to_dev(sh, layer_case(sh, 1, 8, seed=21 + i)[0]) for i, sh in enumerate(shapes)]
    wts = [b.make_weights(w) for w in wd]
    ds = [H.desc(sh) for sh in shapes]
    x = H.to_dev(H.rand_np(22, (Bn, shapes[0].hidden), bf16=True), torch.bfloat16)
    lens_np = np.array([0, 17, 39], np.int32)
    pos = H.ints_to_dev(O.decode_positions(lens_np, np.array([0, -3, 5])))
    lens = H.ints_to_dev(lens_np)
    caches = [(H.to_dev(H.rand_np(23 + 2 * i, (Bn, 1, cap, 128), bf16=True), torch.bfloat16),
               H.to_dev(H.rand_np(24 + 2 * i, (Bn, 1, cap, 128), bf16=True), torch.bfloat16)) for i in range(2)]
    cache0 = [(k.clone(), v.clone()) for k, v in caches]
    kvs = [b.make_kv(k, v, lens) for k, v in caches]
    h1, out, nrm = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    ws = [H.workspace(b.compass_workspace_size(d, Bn, 1, cap, 1)) for d in ds]

    def step():
        b.compass_layer_decode_chained(ds[0], wts[0], x, None, pos, kvs[0], h1, wd[1]["ln_w"], shapes[1].ln_eps,
                                       nrm, ws[0])
        b.compass_layer_decode_chained(ds[1], wts[1], h1, nrm, pos, kvs[1], out, None, 0.0, None, ws[1])

    step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_caches = [(k.clone(), v.clone()) for k, v in caches]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.zero_(); h1.zero_(); nrm.zero_()
        for (k, v), (k0, v0) in zip(caches, cache0):
            k.copy_(k0); v.copy_(v0)  # the appended rows are written again by the replay
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: output"
        for i, ((k, v), (rk, rv)) in enumerate(zip(caches, ref_caches)):
            assert torch.equal(k, rk) and torch.equal(v, rv), f"replay {r}: layer {i} K/V cache"
