"""compass_layer_decode_noalloc (the decode step on the library's own device scratch,
for callers that cannot allocate) against compass_layer_decode with a caller workspace,
through the C ABI: two calls in a row, the second with a smaller input, each output and
each cache bitwise equal (the same kernels in the same launch shapes), and the second
call's output within the bf16 gate of the fp64 oracle. A step whose workspace exceeds
the scratch is rejected before any launch."""
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


def both(sh, wd, x, pos, kc, vc, lens):
    """The step through both entry points, each on its own copy of the cache."""
    b = H.B()
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    ref = H.run_decode(sh, wd, x, pos, k1, v1, lens)
    out = torch.full_like(x, float("nan"))
    b.compass_layer_decode_noalloc(H.desc(sh), b.make_weights(wd), x, pos, b.make_kv(k2, v2, lens), out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    return out


def test_noalloc_decode_equals_workspace_decode_twice():
    b = H.B()
    # Call 1: the batched-decode widths (hidden 2048, 16/4 heads, hd 128, I 8192) on a
    # full-attention layer, B = 64 over a cache of 8200 keys with ragged lens up to 8192.
    cfg = WORKLOADS["decode_stack"]
    sh = dataclasses.replace(cfg["shape"], kind="full")
    Bn, cap = 64, 8200
    Hkv, hd = sh.n_kv_heads, sh.head_dim
    need = b.compass_workspace_size(H.desc(sh), Bn, 1, cap, 1)
    assert 0 < need <= b.COMPASS_NOALLOC_SCRATCH_BYTES
    w = W.make_layer_weights(sh, W.Stream.DECODE_STACK, 3)
    kc = RT.normal(stream_seed(W.Stream.DECODE_STACK, 3, W.TensorId.K_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
    vc = RT.normal(stream_seed(W.Stream.DECODE_STACK, 3, W.TensorId.V_CACHE), Bn * Hkv * cap * hd).to(torch.bfloat16).view(Bn, Hkv, cap, hd)
    lens_np = np.linspace(0, 8192, Bn).astype(np.int32)
    x = H.to_dev(W.make_layer_input(sh, W.Stream.DECODE_STACK, Bn), torch.bfloat16)
    pos = H.ints_to_dev(O.decode_positions(lens_np, np.zeros(Bn, np.int64)))
    both(sh, H.weights_to_dev(sh, w), x, pos, kc, vc, H.ints_to_dev(lens_np))
    del kc, vc

    # Call 2: a smaller sliding layer (hidden 256, 4/1 heads, hd 128), B = 5, capacity 300,
    # on the same scratch; also against the oracle.
    sh2 = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 40)
    lens2 = np.array([0, 1, 39, 40, 299], np.int32)
    w2, _, _ = layer_case(sh2, 1, 8, seed=5)
    x2 = H.rand_np(6, (5, sh2.hidden))
    k2 = H.rand_np(7, (5, 1, 300, 128))
    v2 = H.rand_np(8, (5, 1, 300, 128))
    pos2 = O.decode_positions(lens2, np.array([0, 2, -7, 0, 11], np.int64))
    out2 = both(sh2, H.weights_to_dev(sh2, w2), H.to_dev(x2, torch.bfloat16), H.ints_to_dev(pos2),
                H.to_dev(k2, torch.bfloat16), H.to_dev(v2, torch.bfloat16), H.ints_to_dev(lens2))
    ref2, _, _ = O.layer_decode(sh2, w2, x2, pos2, k2, v2, lens2)
    check_layer_out(sh2, out2, x2, ref2, "no-allocation decode")


def test_noalloc_decode_rejects_steps_beyond_the_scratch():
    b = H.B()
    sh = dataclasses.replace(WORKLOADS["decode_stack"]["shape"], kind="full")
    Bn, cap = 64, 1 << 16  # a full layer over 65536 keys needs more than the scratch holds
    assert b.compass_workspace_size(H.desc(sh), Bn, 1, cap, 1) > b.COMPASS_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((Bn, sh.hidden), dtype=torch.bfloat16, device="cuda")
    wd = H.weights_to_dev(sh, W.make_layer_weights(sh, W.Stream.DECODE_STACK, 3))
    # Real caches of the stated capacity (4.3 GB each), so every pointer is valid whatever happens.
    kc = torch.zeros((Bn, sh.n_kv_heads, cap, sh.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    lens = H.ints_to_dev(np.zeros(Bn, np.int32))
    out = torch.full_like(x, 7.0)
    with pytest.raises(b.CompassError) as e:
        b.compass_layer_decode_noalloc(H.desc(sh), b.make_weights(wd), x, None, b.make_kv(kc, vc, lens), out)
    assert e.value.code == b.COMPASS_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was launched
