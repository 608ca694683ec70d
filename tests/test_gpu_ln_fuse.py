"""The LayerNorm fused into the projection GEMM (descriptor ln_fuse = 1: a statistics pass,
then each A tile normalized in registers as it is staged) against the default path (the
LayerNorm kernel writing normalized rows): both compute (x - mean) * rstd * ln_w in fp32 with
the same statistics and round it once to bf16, so every output and every cache row must be
bitwise equal. Plain prefill (256- and 128-row GEMM tiles), chunked prefill, varlen prefill,
and the headline sliding layer at full size; plus the fused output against the oracle."""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import stream_seed
from synth import workloads as W
from synth.workloads import WORKLOADS
from tests import helpers as H
from tests.test_gpu_small import check_layer_out, layer_case

pytestmark = pytest.mark.gpu


def prefill(sh, wd, x, pos, ln_fuse, kv=None, chunk_lens=None):
    b = H.B()
    d = H.desc(sh, ln_fuse)
    Bn, L = x.shape[0], x.shape[1]
    ws = H.workspace(b.compass_workspace_size(d, Bn, L, 0, 0))
    out = torch.empty_like(x)
    if chunk_lens is not None:
        b.compass_layer_prefill_chunk(d, b.make_weights(wd), x, pos, b.make_kv(kv[0], kv[1], chunk_lens), None, None,
                                      out, ws)
    else:
        b.compass_layer_prefill(d, b.make_weights(wd), x, pos, None if kv is None else b.make_kv(*kv), None, None,
                                out, ws)
    return out


@pytest.mark.parametrize("kind,L", [("sliding", 700), ("full", 300), ("sliding", 2100)])
def test_fused_layernorm_is_bitwise_the_default_path(kind, L):
    sh = H.small_shape("bf16", kind, 128, 4, 1, 512, 512, 100)
    w, x, pos = layer_case(sh, 1, L, seed=17)
    wd, xd, pd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos)
    caches = [tuple(torch.full((1, 1, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(2))
              for _ in range(2)]
    o0 = prefill(sh, wd, xd, pd, 0, kv=caches[0])
    o1 = prefill(sh, wd, xd, pd, 1, kv=caches[1])
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    assert torch.equal(caches[0][0], caches[1][0]) and torch.equal(caches[0][1], caches[1][1])
    check_layer_out(sh, o1, x, O.layer_prefill(sh, w, x, pos), "fused LayerNorm")


def test_fused_layernorm_chunked_and_varlen_bitwise():
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 48)
    Bn, L = 2, 150
    w, x, pos = layer_case(sh, Bn, L, seed=19)
    wd, xd, pd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos)
    lens = H.ints_to_dev(np.array([0, 40], np.int32))
    outs, caches = [], []
    for f in (0, 1):
        kc = torch.zeros((Bn, 1, L + 40, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        outs.append(prefill(sh, wd, xd, pd, f, kv=(kc, vc), chunk_lens=lens))
        caches.append((kc, vc))
    b = H.B()
    cu = H.ints_to_dev(np.array([0, 150, 300], np.int32))
    xp, pp = xd.reshape(Bn * L, -1), pd.reshape(3, Bn * L).contiguous()
    vouts = []
    for f in (0, 1):
        d = H.desc(sh, f)
        ws = H.workspace(b.compass_varlen_workspace_size(d, 2, Bn * L))
        o = torch.empty_like(xp)
        st = torch.zeros((1,), dtype=torch.int32, device="cuda")
        b.compass_layer_prefill_varlen(d, b.make_weights(wd), cu, xp, pp, None, None, None, o, st, ws)
        vouts.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(caches[0][0], caches[1][0]) and torch.equal(caches[0][1], caches[1][1])
    assert torch.equal(vouts[0], vouts[1])


@pytest.mark.slow
def test_fused_layernorm_headline_layer_bitwise():
    """The headline sliding layer (hidden 2048, 16/4 heads, hd 128, I 8192, window 1024, L = 4096)."""
    cfg = WORKLOADS["sliding_prefill"]
    sh, L = cfg["shape"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.SLIDING_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.SLIDING_PREFILL, L).reshape(1, L, sh.hidden)
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.SLIDING_PREFILL, 0, W.TensorId.TOKENS))
    pos, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    wd, xd, pd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos)
    o0 = prefill(sh, wd, xd, pd, 0)
    o1 = prefill(sh, wd, xd, pd, 1)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
