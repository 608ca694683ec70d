"""GPU parity of chunked prefill (compass_layer_prefill_chunk) against the fp64 oracle.

A chunk of L tokens continues a dense cache that already holds lens[b] tokens of row b
(ragged per row). Cache rows past each row's end are filled with NaN, so a read of an
invisible key or a write outside the chunk's slots shows up. Gates as for the plain
prefill: max relative error 2e-2 (bf16) / 1e-4 (fp32), plus the branch-sum check.
"""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from tests import helpers as H
from tests.test_gpu_small import check_layer_out, layer_case

pytestmark = pytest.mark.gpu

CHUNK_CASES = [
    # dtype, kind, hd, Hq, Hkv, D, I, window, starts, Lc
    ("bf16", "sliding", 128, 4, 1, 256, 512, 48, (0, 37, 130), 70),
    ("bf16", "full", 128, 4, 2, 256, 512, 0, (0, 64, 200), 130),
    ("bf16", "sliding", 64, 8, 2, 256, 256, 100, (5, 260), 33),
    ("bf16", "sliding", 128, 4, 1, 256, 512, 300, (0, 200, 90), 520),   # chunks of >= 512 queries
    ("bf16", "full", 64, 4, 2, 256, 256, 0, (70, 0), 600),
    ("f32", "sliding", 64, 4, 1, 256, 512, 32, (0, 17, 90), 40),
    ("f32", "full", 128, 2, 1, 256, 256, 0, (3, 50), 25),
]


def make_cache(sh, starts, cap, seed, td):
    """Random already-cached K/V for indices [0, start); NaN elsewhere."""
    Bn = len(starts)
    r = np.random.default_rng(seed)
    kc = np.full((Bn, sh.n_kv_heads, cap, sh.head_dim), np.nan)
    vc = np.full_like(kc, np.nan)
    for b, s0 in enumerate(starts):
        kc[b, :, :s0] = r.standard_normal((sh.n_kv_heads, s0, sh.head_dim))
        vc[b, :, :s0] = r.standard_normal((sh.n_kv_heads, s0, sh.head_dim))
    if td == torch.bfloat16:
        kc, vc = H.bf16_round(kc), H.bf16_round(vc)
    return kc, vc


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_chunk_parity(case):
    dt, kind, hd, Hq, Hkv, D, I, win, starts, Lc = case
    sh = H.small_shape(dt, kind, hd, Hq, Hkv, D, I, win)
    Bn = len(starts)
    w, x, pos = layer_case(sh, Bn, Lc, seed=hd + Lc)
    td = H.tdtype(sh)
    cap = max(starts) + Lc + 5
    kc_np, vc_np = make_cache(sh, starts, cap, seed=Lc, td=td)
    starts_np = np.asarray(starts, dtype=np.int32)
    ref, kref, vref = O.layer_prefill_chunk(sh, w, x, pos, kc_np, vc_np, starts_np)
    kc, vc = H.to_dev(kc_np, td), H.to_dev(vc_np, td)
    out = H.run_prefill_chunk(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kc, vc,
                              H.ints_to_dev(starts_np))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x, ref)
    kg, vg = H.np64(kc), H.np64(vc)
    for b, s0 in enumerate(starts):
        assert H.rel_err(kg[b, :, s0:s0 + Lc], kref[b]) <= H.tol(sh)
        assert H.rel_err(vg[b, :, s0:s0 + Lc], vref[b]) <= H.tol(sh)
        assert np.array_equal(kg[b, :, :s0], H.np64(H.to_dev(kc_np[b, :, :s0], td)))  # prefix untouched
        assert np.isnan(kg[b, :, s0 + Lc:]).all() and np.isnan(vg[b, :, s0 + Lc:]).all()  # nothing past the chunk


def test_chunk_rows_that_do_not_fit_are_skipped():
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 48)
    Lc, cap = 40, 100
    starts = np.array([10, cap - Lc + 1, -3], dtype=np.int32)  # rows 1 and 2 do not fit
    w, x, pos = layer_case(sh, 3, Lc, seed=7)
    kc_np, vc_np = make_cache(sh, [10, 0, 0], cap, seed=8, td=torch.bfloat16)
    kc, vc = H.to_dev(kc_np, torch.bfloat16), H.to_dev(vc_np, torch.bfloat16)
    out = torch.full((3, Lc, sh.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    ds_rows = H.ints_to_dev(np.array([Lc + 3, 2 * Lc + 1, 5], dtype=np.int32))  # rows in b = 1, 2, 0
    ds = torch.ones((3, sh.hidden), dtype=torch.bfloat16, device="cuda")
    H.run_prefill_chunk(sh, H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos), kc, vc,
                        H.ints_to_dev(starts), ds_rows=ds_rows, ds=ds, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[1:] == 7.0)  # skipped rows (deepstack included) untouched
    assert torch.isnan(kc[1:]).all() and torch.isnan(vc[1:]).all()
    ref, _, _ = O.layer_prefill_chunk(sh, w, x[:1], pos[:, :1], kc_np[:1], vc_np[:1], starts[:1])
    ref[0, 5] += 1.0
    check_layer_out(sh, out[:1], x[:1], ref)


@pytest.mark.parametrize("kind,win", [("sliding", 48), ("full", 0)])
def test_prefill_then_chunk_equals_one_prefill(kind, win):
    """prefill(x[:, :L1]) writing the cache, then a chunk of the remaining rows, reproduces
    one prefill of the whole rows (within the bf16 gate)."""
    sh = H.small_shape("bf16", kind, 128, 4, 1, 256, 512, win)
    Bn, L, L1 = 2, 300, 130
    w, x, pos = layer_case(sh, Bn, L, seed=11)
    wd, td = H.weights_to_dev(sh, w), torch.bfloat16
    xd, posd = H.to_dev(x, td), H.ints_to_dev(pos)
    full = H.run_prefill(sh, wd, xd, posd)
    cap = L + 8
    kc = torch.full((Bn, sh.n_kv_heads, cap, sh.head_dim), float("nan"), dtype=td, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    first = H.run_prefill(sh, wd, xd[:, :L1].contiguous(), posd[:, :, :L1].contiguous(), kv=(kc, vc))
    lens = H.ints_to_dev(np.full(Bn, L1, dtype=np.int32))
    rest = H.run_prefill_chunk(sh, wd, xd[:, L1:].contiguous(), posd[:, :, L1:].contiguous(), kc, vc, lens)
    torch.cuda.synchronize()
    assert torch.equal(first, full[:, :L1])  # causality: the first rows do not see the rest
    got = torch.cat([first, rest], dim=1)
    ref = O.layer_prefill(sh, w, x, pos)
    check_layer_out(sh, got, x, ref)
    assert H.rel_err(H.np64(rest), H.np64(full[:, L1:])) <= H.tol(sh)
