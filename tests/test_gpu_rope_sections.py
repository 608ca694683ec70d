"""GPU parity of the sections rotary layout (COMPASS_ROPE_SECTIONS): prefill (bf16 and fp32,
head_dim 128 and 64, several sections) and decode against the oracle in the same layout.

Parity is pinned to the oracle's reading of the layout only: the real rotary class's
permutation is not printed by the pages (parity unpinned against that class). Gates as
for the interleaved layout: 2e-2 (bf16), 1e-4 (fp32).
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from tests import helpers as H
from tests.test_gpu_small import check_layer_out, layer_case

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, hd, Hq, Hkv, D, I, window, B, L, section
    ("bf16", 128, 4, 1, 256, 512, 48, 2, 200, (24, 20, 20)),
    ("bf16", 64, 8, 2, 256, 512, 100, 1, 333, (14, 8, 10)),
    ("f32", 64, 4, 1, 256, 512, 32, 1, 128, (12, 10, 10)),
    ("f32", 128, 2, 1, 256, 256, 40, 2, 77, (28, 16, 20)),
]


def sections_shape(dt, hd, Hq, Hkv, D, I, win, section):
    sh = H.small_shape(dt, "sliding", hd, Hq, Hkv, D, I, win, section=section)
    return dataclasses.replace(sh, rope_layout="sections")


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-hd{c[1]}-{'-'.join(map(str, c[9]))}" for c in CASES])
def test_sections_prefill_parity(case):
    dt, hd, Hq, Hkv, D, I, win, Bn, L, section = case
    sh = sections_shape(dt, hd, Hq, Hkv, D, I, win, section)
    w, x, pos = layer_case(sh, Bn, L, seed=hd + L)
    ref, st = O.layer_prefill(sh, w, x, pos, return_stages=True)
    td = H.tdtype(sh)
    kc = torch.full((Bn, Hkv, L + 2, hd), float("nan"), dtype=td, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = H.run_prefill(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kv=(kc, vc))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x, ref, "sections prefill")
    assert H.rel_err(H.np64(kc[:, :, :L]), st["k"]) <= H.tol(sh)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sections_decode_parity(dt):
    sh = sections_shape(dt, 128, 4, 1, 256, 512, 60, (24, 20, 20))
    bf = dt == "bf16"
    lens = np.array([0, 5, 59, 60, 300], np.int32)
    Bn, cap = len(lens), 301
    w, _, _ = layer_case(sh, 1, 8, seed=17)
    x = H.rand_np(18, (Bn, sh.hidden), bf16=bf)
    kc = H.rand_np(19, (Bn, 1, cap, 128), bf16=bf)
    vc = H.rand_np(20, (Bn, 1, cap, 128), bf16=bf)
    pos = O.decode_positions(lens, np.array([0, -3, 7, -100, 2]))
    ref, knew, _ = O.layer_decode(sh, w, x, pos, kc, vc, lens)
    td = H.tdtype(sh)
    kd, vd = H.to_dev(kc, td), H.to_dev(vc, td)
    out = H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kd, vd, H.ints_to_dev(lens))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x, ref, "sections decode")
    kg = H.np64(kd)
    for i, n in enumerate(lens):
        assert H.rel_err(kg[i, :, n], knew[i]) <= H.tol(sh)


def test_sections_differs_from_interleaved():
    """The layout flag reaches the kernels: the same inputs give different K in the two layouts."""
    sh = sections_shape("bf16", 128, 4, 1, 256, 512, 48, (24, 20, 20))
    w, x, pos = layer_case(sh, 1, 64, seed=5)
    outs = []
    for s in (sh, dataclasses.replace(sh, rope_layout="interleaved")):
        kc = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        H.run_prefill(s, H.weights_to_dev(s, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos), kv=(kc, vc))
        outs.append(H.np64(kc))
    torch.cuda.synchronize()
    assert H.rel_err(outs[0], outs[1]) > 0.1
