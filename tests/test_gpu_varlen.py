"""Varlen prefill (compass_layer_prefill_varlen) against oracle.layer_prefill_varlen.

Packed sequences of different lengths in one launch: empty and one-token sequences,
lengths on both sides of the attention's 128-query tiles, sliding and full layers, bf16
and fp32, head_dim 64 and 128, GQA groups 1 to 8; with and without caches (per-sequence
starts, a sequence that does not fit its cache, untouched cache rows NaN), deepstack on
packed rows, invalid offsets (nothing written), and the Compass widths at a mixed batch
of 8226 rows with every row's attention output gated through the probe layer.
"""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import workloads as W
from tests import helpers as H
from tests.test_gpu_small import check_layer_out, layer_case

pytestmark = pytest.mark.gpu


def run_varlen(sh, wd, cu, x, pos, kv=None, ds_rows=None, ds=None, out=None):
    b = H.B()
    T = x.shape[0]
    n_seq = len(cu) - 1
    ws = H.workspace(b.compass_varlen_workspace_size(H.desc(sh), n_seq, T))
    out = torch.empty_like(x) if out is None else out
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    kvs = None if kv is None else b.make_kv(*kv)
    b.compass_layer_prefill_varlen(H.desc(sh), b.make_weights(wd), H.ints_to_dev(cu), x,
                                   None if pos is None else H.ints_to_dev(pos), kvs, ds_rows, ds, out, status, ws)
    return out, status


def packed_case(sh, lens, seed):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    w, _, _ = layer_case(sh, 1, 8, seed=seed)
    x = H.rand_np(seed + 1, (T, sh.hidden), bf16=sh.dtype == "bf16")
    pos = np.random.default_rng(seed + 2).integers(0, 3 * max(lens), size=(3, T))
    return w, x, pos, cu


VARLEN_CASES = [
    # dtype, kind, hd, Hq, Hkv, D, I, window, lengths
    ("bf16", "sliding", 128, 4, 1, 256, 512, 48, [5, 1, 0, 129, 128, 127, 300]),
    ("bf16", "full", 128, 4, 2, 256, 512, 0, [257, 1, 64, 0, 0, 130]),
    ("bf16", "sliding", 64, 8, 1, 256, 256, 100, [1, 1, 1, 700, 33]),
    ("bf16", "full", 64, 8, 4, 512, 256, 0, [128, 256, 384]),
    ("bf16", "sliding", 128, 8, 1, 512, 512, 1, [3, 200]),
    ("f32", "sliding", 64, 4, 1, 256, 1024, 32, [5, 1, 0, 129, 77]),
    ("f32", "full", 128, 4, 2, 256, 512, 0, [40, 1, 90]),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "-".join(map(str, c[:8])) + f"-n{len(c[8])}")
def test_varlen_prefill_parity(case):
    dt, kind, hd, Hq, Hkv, D, I, win, lens = case
    sh = H.small_shape(dt, kind, hd, Hq, Hkv, D, I, win)
    w, x, pos, cu = packed_case(sh, lens, seed=hd + Hq + len(lens))
    td = H.tdtype(sh)
    out, status = run_varlen(sh, H.weights_to_dev(sh, w), cu, H.to_dev(x, td), pos)
    torch.cuda.synchronize()
    assert status.item() == 0
    ref, _, _ = O.layer_prefill_varlen(sh, w, x, pos if kind == "sliding" else None, cu)
    check_layer_out(sh, out, x, ref, f"varlen {lens}")


@pytest.mark.parametrize("dt,kind", [("bf16", "sliding"), ("bf16", "full"), ("f32", "sliding")])
def test_varlen_prefill_continues_caches(dt, kind):
    """Each sequence continues its own cache at lens[s]; one sequence does not fit its cache
    and is skipped (status bit 1, no K/V written, its out rows untouched); cache rows outside
    each chunk stay NaN; deepstack rows land on packed rows of live sequences only."""
    sh = H.small_shape(dt, kind, 128, 4, 1, 256, 512, 40)
    lens = [70, 1, 130, 9, 50]
    starts = np.array([0, 300, 120, 340, 5], np.int32)
    cap = 345  # sequence 3 (340 + 9) does not fit
    w, x, pos, cu = packed_case(sh, lens, seed=61)
    td = H.tdtype(sh)
    bf = dt == "bf16"
    n_seq = len(lens)
    kc0 = H.rand_np(62, (n_seq, 1, cap, 128), bf16=bf)
    vc0 = H.rand_np(63, (n_seq, 1, cap, 128), bf16=bf)
    for s_ in range(n_seq):  # rows at and past each chunk start are unknown: NaN
        kc0[s_, :, starts[s_]:] = np.nan
        vc0[s_, :, starts[s_]:] = np.nan
    kd, vd = H.to_dev(kc0, td), H.to_dev(vc0, td)
    ds_rows = np.array([0, 71, 80, 205, 209, 255], np.int32)  # 205 lies in the skipped sequence
    ds = H.rand_np(64, (len(ds_rows), sh.hidden), bf16=bf)
    out = torch.full_like(H.to_dev(x, td), 7.0)
    xd = H.to_dev(x, td)
    got, status = run_varlen(sh, H.weights_to_dev(sh, w), cu, xd, pos, kv=(kd, vd, H.ints_to_dev(starts)),
                             ds_rows=H.ints_to_dev(ds_rows), ds=H.to_dev(ds, td), out=out)
    torch.cuda.synchronize()
    assert status.item() == 2
    ref, kn, vn = O.layer_prefill_varlen(sh, w, x, pos if kind == "sliding" else None, cu,
                                         np.nan_to_num(kc0), np.nan_to_num(vc0), starts)
    flat = ref.copy()
    live_rows = np.ones(len(x), bool)
    live_rows[cu[3]:cu[4]] = False
    for r, d_ in zip(ds_rows, ds):
        if live_rows[r]:
            flat[r] += d_
    g = H.np64(got)
    assert np.all(g[~live_rows] == 7.0)
    check_layer_out(sh, g[live_rows], x[live_rows], flat[live_rows], "varlen with caches")
    kg, vg = H.np64(kd), H.np64(vd)
    for s_, (n, s0) in enumerate(zip(lens, starts)):
        if s_ == 3:
            assert np.all(np.isnan(kg[s_, :, s0:])) and np.all(np.isnan(vg[s_, :, s0:]))
            continue
        assert H.rel_err(kg[s_, :, s0:s0 + n], kn[s_]) <= H.tol(sh)
        assert H.rel_err(vg[s_, :, s0:s0 + n], vn[s_]) <= H.tol(sh)
        assert np.all(np.isnan(kg[s_, :, s0 + n:]))
        assert np.array_equal(kg[s_, :, :s0], kc0[s_, :, :s0])


@pytest.mark.parametrize("cu", [[1, 5, 9], [0, 6, 3, 9], [0, 4, 8]], ids=["first", "decreasing", "short"])
def test_varlen_invalid_offsets_write_nothing(cu):
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 40)
    w, x, pos, _ = packed_case(sh, [4, 5], seed=71)
    out = torch.full_like(H.to_dev(x, torch.bfloat16), 7.0)
    kc = torch.full((len(cu) - 1, 1, 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    _, status = run_varlen(sh, H.weights_to_dev(sh, w), np.array(cu, np.int32), H.to_dev(x, torch.bfloat16), pos,
                           kv=(kc, vc, None), out=out)
    torch.cuda.synchronize()
    assert status.item() == 1
    assert torch.all(out == 7.0) and torch.isnan(kc).all() and torch.isnan(vc).all()


@pytest.mark.slow
@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_varlen_prefill_compass_widths(kind):
    """Hidden 2048, 16/4 heads, hd 128, I 8192 (window 1024 on the sliding layer): five
    sequences of 4096 (the image-row layout with its positions), 1000, 1, 3000 and 129 tokens
    packed into 8226 rows, written to caches; whole output and K/V against the oracle, and
    every row's attention output through the probe layer (Wo = 64 I, w_down = 0)."""
    from synth import stream_seed
    from synth.workloads import WORKLOADS
    sh = W.WORKLOADS["sliding_prefill"]["shape"]
    import dataclasses
    sh = dataclasses.replace(sh, kind=kind, window=1024 if kind == "sliding" else 0)
    lens = [4096, 1000, 1, 3000, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    w = W.make_layer_weights(sh, W.Stream.SLIDING_PREFILL, 0)
    x = W.make_layer_input(sh, W.Stream.SLIDING_PREFILL, T)
    tok, grid, off = W.image_text_row(stream_seed(W.Stream.SLIDING_PREFILL, 0, W.TensorId.TOKENS))
    p0, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    pos = np.concatenate([p0[:, 0]] + [np.broadcast_to(np.arange(n), (3, n)) for n in lens[1:]], axis=1)
    cap = max(lens)
    kc = torch.full((len(lens), sh.n_kv_heads, cap, sh.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    xd = H.to_dev(x, torch.bfloat16)
    out, status = run_varlen(sh, H.weights_to_dev(sh, w), cu, xd, pos, kv=(kc, vc, None))
    probe, _ = run_varlen(sh, H.weights_to_dev(sh, H.probe_weights(sh, w)), cu, xd, pos)
    torch.cuda.synchronize()
    assert status.item() == 0
    wf = {k: np.asarray(v, np.float64) for k, v in w.items()}
    ref, kn, vn = O.layer_prefill_varlen(sh, wf, x, pos if kind == "sliding" else None, cu)
    check_layer_out(sh, out, x, ref, f"varlen {kind} Compass widths")
    kg = H.np64(kc)
    for s_, n in enumerate(lens):
        assert H.rel_err(kg[s_, :, :n], kn[s_]) <= 2e-2
    # Attention output alone: the oracle's probe layer is x + 64 o.
    ref_p, _, _ = O.layer_prefill_varlen(sh, {k: np.asarray(v, np.float64) for k, v in H.probe_weights(sh, w).items()},
                                         x, pos if kind == "sliding" else None, cu)
    e = H.check_attn_rows(sh, probe, x, (ref_p - x) / H.PROBE_SCALE, f"varlen {kind}")
    print(f"varlen {kind} Compass widths: attention rows {e:.2e}")
