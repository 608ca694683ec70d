"""GPU parity at small sizes: every entry point of the C ABI against the fp64 oracle.

Sizes span several tiles and a ragged tail; inputs are seeded (synth). Gates:
positions bit-exact; layer outputs, K/V cache rows and logits within 2e-2 (bf16)
or 1e-4 (fp32) as max|gpu - oracle| / max|oracle|. Layer outputs are also gated on
the branch sum out - x, allowing for the bf16 rounding of out itself.
"""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu


def mixed_tokens(B, L, seed):
    """Rows with text, images of a few grids (including back-to-back images) and text."""
    toks, grids, offs = [], [], [0]
    layouts = [[(3, (1, 4, 6)), (2, (2, 4, 4)), (0, (1, 2, 2))], [(7, (1, 8, 12))], [], [(0, (1, 6, 2))]]
    for b in range(B):
        row = list(W.text_tokens(seed + b, L))
        p = 0
        for gap, g in layouts[b % len(layouts)]:
            p += gap
            n = g[0] * (g[1] // 2) * (g[2] // 2)
            if p + n > L:
                break
            row[p:p + n] = [W.IMAGE_TOKEN_ID] * n
            grids.append(g)
            p += n
        toks.append(row)
        offs.append(len(grids))
    return (np.array(toks, np.int32), np.array(grids, np.int32).reshape(-1, 3), np.array(offs, np.int32))


# ------------------------------------------------------------------------------ positions
def gpu_positions(tok, grid, off, merge=2):
    b = H.B()
    Bn, L = tok.shape
    pos = torch.full((3, Bn, L), -7, dtype=torch.int32, device="cuda")
    delta = torch.full((Bn,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((Bn,), -7, dtype=torch.int32, device="cuda")
    g = H.ints_to_dev(grid if len(grid) else np.zeros((1, 3), np.int32))
    b.compass_mrope_positions(H.ints_to_dev(tok), W.IMAGE_TOKEN_ID, g, H.ints_to_dev(off), merge, pos, delta, status)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), delta.cpu().numpy(), status.cpu().numpy()


@pytest.mark.parametrize("B,L", [(1, 1), (2, 37), (4, 300), (3, 2500)])
def test_positions_bit_exact(B, L):
    tok, grid, off = mixed_tokens(B, L, seed=L)
    pos, delta, status = gpu_positions(tok, grid, off)
    ref_pos, ref_delta = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    assert np.all(status == 0)
    assert np.array_equal(pos, ref_pos)
    assert np.array_equal(delta, ref_delta)


def test_positions_c1_layout_bit_exact():
    tok, grid, off = W.image_text_row(seed=5)
    pos, delta, status = gpu_positions(tok, grid, off)
    ref_pos, ref_delta = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    assert status.tolist() == [0]
    assert np.array_equal(pos, ref_pos) and np.array_equal(delta, ref_delta)
    assert delta[0] == -992


@pytest.mark.parametrize("case", ["short_span", "extra_pads", "unused_image", "bad_grid", "span_past_end",
                                  "grid_product_past_int64"])
def test_positions_error_codes(case):
    n = 4
    I = W.IMAGE_TOKEN_ID
    rows = {
        "short_span": ([[1] + [I] * (n - 1) + [2, 3]], [[1, 4, 4]]),
        "extra_pads": ([[1] + [I] * (n + 1) + [2]], [[1, 4, 4]]),
        "unused_image": ([[1] + [I] * n + [2]], [[1, 4, 4], [1, 2, 2]]),
        "bad_grid": ([[1] + [I] * n + [2]], [[1, 3, 4]]),
        "span_past_end": ([[1, 2] + [I] * (n - 1)], [[1, 4, 4]]),
        # merged grid 2^21 x 2^21 x 2^22: the pad count 2^64 wraps a 64-bit product to 0
        "grid_product_past_int64": ([[1] + [I] * n + [2]], [[1 << 21, 1 << 22, 1 << 23]]),
    }
    tok, grid = rows[case]
    tok = np.array(tok, np.int32)
    grid = np.array(grid, np.int32)
    # Row 1 is a clean text row: its status must stay 0 and its positions exact.
    tok2 = np.concatenate([tok, np.arange(10, 10 + tok.shape[1], dtype=np.int32)[None]], 0)
    off = np.array([0, len(grid), len(grid)], np.int32)
    _, _, status = gpu_positions(tok2, grid, off)
    with pytest.raises(O.PositionError) as e:
        O.mrope_positions(tok, I, grid, np.array([0, len(grid)]), 2)
    assert status.tolist() == [e.value.code, 0]


# ------------------------------------------------------------------------------ prefill
def layer_case(shape, Bn, L, seed, wstd=0.06):
    w = {}
    r = np.random.default_rng(seed)
    base = W.make_layer_weights(shape, 100 + seed % 50, seed)
    for k, v in base.items():  # rescale the N(0, 0.02) weights so both branches are sizeable
        w[k] = v if k == "ln_w" else (H.bf16_round(v * (wstd / 0.02)) if shape.dtype == "bf16" else v * (wstd / 0.02))
    x = H.rand_np(seed + 1, (Bn, L, shape.hidden), bf16=shape.dtype == "bf16")
    tok, grid, off = mixed_tokens(Bn, L, seed)
    pos, _ = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    return w, x, pos


def check_layer_out(shape, out_gpu, x, ref, what=""):
    g = H.np64(out_gpu)
    e_out = H.rel_err(g, ref)
    assert e_out <= H.tol(shape), f"{what} out rel err {e_out:.3e}"
    d_ref = ref - x
    d_gpu = g - x
    rounding = (2.0 ** -8 if shape.dtype == "bf16" else 2.0 ** -23) * np.abs(ref)
    excess = np.abs(d_gpu - d_ref) - rounding
    e_delta = float(np.max(excess) / np.max(np.abs(d_ref)))
    assert e_delta <= H.tol(shape), f"{what} branch-sum rel err {e_delta:.3e}"
    return e_out, e_delta


PREFILL_CASES = [
    # dtype, kind, hd, Hq, Hkv, D, I, window, B, L
    ("f32", "sliding", 64, 4, 1, 256, 1024, 32, 1, 128),     # the fp32 parity workload's shape
    ("f32", "full", 128, 4, 2, 256, 512, 0, 2, 77),
    ("bf16", "sliding", 128, 4, 1, 256, 512, 48, 2, 200),
    ("bf16", "full", 128, 4, 1, 256, 512, 0, 2, 200),
    ("bf16", "sliding", 64, 8, 2, 256, 512, 100, 1, 333),
    ("bf16", "full", 64, 8, 4, 512, 256, 0, 1, 130),
    ("bf16", "sliding", 128, 8, 1, 512, 1024, 1, 1, 70),    # window of one key
    ("bf16", "sliding", 128, 2, 2, 256, 256, 5000, 1, 257),  # window >= L
    ("bf16", "sliding", 128, 4, 2, 256, 256, 300, 1, 700),   # window spans several key tiles
    ("bf16", "full", 128, 2, 1, 256, 256, 0, 1, 600),        # several 256-query blocks, ragged tail
    ("bf16", "sliding", 64, 4, 2, 256, 256, 200, 2, 530),    # head_dim 64 with 64-query waves
    ("bf16", "full", 64, 8, 1, 256, 256, 0, 1, 1100),
    ("bf16", "sliding", 128, 4, 1, 256, 256, 64, 1, 777),    # window shorter than a wave's 64 queries
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_parity(case):
    dt, kind, hd, Hq, Hkv, D, I, win, Bn, L = case
    sh = H.small_shape(dt, kind, hd, Hq, Hkv, D, I, win)
    w, x, pos = layer_case(sh, Bn, L, seed=hd + Hq + L)
    ref, st = O.layer_prefill(sh, w, x, pos, return_stages=True)
    td = H.tdtype(sh)
    wd = H.weights_to_dev(sh, w)
    xd = H.to_dev(x, td)
    posd = H.ints_to_dev(pos)
    cap = L + 3
    kc = torch.full((Bn, Hkv, cap, hd), float("nan"), dtype=td, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = H.run_prefill(sh, wd, xd, posd, kv=(kc, vc))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x, ref)
    assert H.rel_err(H.np64(kc[:, :, :L]), st["k"]) <= H.tol(sh)
    assert H.rel_err(H.np64(vc[:, :, :L]), st["v"]) <= H.tol(sh)
    assert torch.isnan(kc[:, :, L:]).all()  # rows past L untouched


def test_prefill_in_place_and_deepstack():
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 40)
    Bn, L = 2, 150
    w, x, pos = layer_case(sh, Bn, L, seed=7)
    rows = np.array([3, 4, 5, 160, 299], np.int32)
    ds = H.rand_np(99, (len(rows), sh.hidden))
    ref = O.layer_prefill(sh, w, x, pos, rows, ds)
    xd = H.to_dev(x, torch.bfloat16)
    H.run_prefill(sh, H.weights_to_dev(sh, w), xd, H.ints_to_dev(pos), ds_rows=H.ints_to_dev(rows),
                  ds=H.to_dev(ds, torch.bfloat16), out=xd)
    torch.cuda.synchronize()
    check_layer_out(sh, xd, x, ref)


def test_full_layer_position_relabel_bitwise():
    sh = H.small_shape("bf16", "full", 128, 4, 1, 256, 512, 0)
    Bn, L = 2, 190
    w, x, pos = layer_case(sh, Bn, L, seed=11)
    perm = np.stack([np.stack([np.random.default_rng(3 * b + a).permutation(pos[a, b]) for b in range(Bn)])
                     for a in range(3)])
    wd, xd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16)
    o1 = H.run_prefill(sh, wd, xd, H.ints_to_dev(pos))
    o2 = H.run_prefill(sh, wd, xd, H.ints_to_dev(perm))
    o3 = H.run_prefill(sh, wd, xd, None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_window_at_least_L_equals_full_causal_without_rope_difference():
    """W >= L: the sliding layer equals the same layer with a plain causal mask (same rope)."""
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 300)
    Bn, L = 1, 300
    w, x, pos = layer_case(sh, Bn, L, seed=12)
    wd, xd, pd = H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos)
    o1 = H.run_prefill(sh, wd, xd, pd)
    import dataclasses
    o2 = H.run_prefill(dataclasses.replace(sh, window=10 ** 6), wd, xd, pd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ------------------------------------------------------------------------------ decode
DECODE_CASES = [
    ("bf16", "sliding", 128, 4, 1, 256, 512, 40),
    ("bf16", "sliding", 128, 8, 1, 512, 512, 300),   # 8 query heads per kv head
    ("bf16", "full", 64, 8, 1, 256, 512, 0),
    ("bf16", "full", 128, 4, 1, 256, 512, 0),
    ("bf16", "sliding", 64, 8, 2, 256, 512, 300),
    ("f32", "sliding", 64, 4, 1, 256, 1024, 32),
    ("f32", "full", 128, 4, 2, 256, 512, 0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_parity(case):
    dt, kind, hd, Hq, Hkv, D, I, win = case
    sh = H.small_shape(dt, kind, hd, Hq, Hkv, D, I, win)
    bf = dt == "bf16"
    lens = np.array([0, 1, 37, 255, 256, 257, 600, 1000], np.int32)
    Bn, cap = len(lens), 1003
    w, _, _ = layer_case(sh, 1, 8, seed=hd + Hq)
    x = H.rand_np(5, (Bn, D), bf16=bf)
    kc = H.rand_np(6, (Bn, Hkv, cap, hd), bf16=bf)
    vc = H.rand_np(7, (Bn, Hkv, cap, hd), bf16=bf)
    delta = np.array([0, -3, 5, -992, 0, 17, -200, 1], np.int64)
    pos = O.decode_positions(lens, delta)
    ref, knew, vnew = O.layer_decode(sh, w, x, pos, kc, vc, lens)
    td = H.tdtype(sh)
    kd, vd = H.to_dev(kc, td), H.to_dev(vc, td)
    out = H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kd, vd,
                       H.ints_to_dev(lens))
    torch.cuda.synchronize()
    e = H.rel_err(H.np64(out), ref)
    assert e <= H.tol(sh), e
    kg, vg = H.np64(kd), H.np64(vd)
    for i, n in enumerate(lens):
        assert H.rel_err(kg[i, :, n], knew[i]) <= H.tol(sh)
        assert H.rel_err(vg[i, :, n], vnew[i]) <= H.tol(sh)
    # Every other cache row is untouched.
    mask = np.ones((Bn, cap), bool)
    mask[np.arange(Bn), lens] = False
    assert np.array_equal(kg.transpose(0, 2, 1, 3)[mask], kc.transpose(0, 2, 1, 3)[mask])


@pytest.mark.parametrize("case", [c for c in DECODE_CASES if c[0] == "bf16"], ids=lambda c: "-".join(map(str, c)))
def test_decode_reads_only_the_new_row_and_visible_keys(case):
    """Every cache row from lens[b] on starts as NaN: row lens[b] is the new token's K/V,
    written in the same step before the attention reads it, and rows past it are never
    visible. A read of the new row before it is written, or any read past it that is not
    masked before the PV product, turns the output NaN."""
    dt, kind, hd, Hq, Hkv, D, I, win = case
    sh = H.small_shape(dt, kind, hd, Hq, Hkv, D, I, win)
    lens = np.array([0, 1, 63, 64, 255, 256, 257, 511, 700], np.int32)
    Bn, cap = len(lens), 770
    w, _, _ = layer_case(sh, 1, 8, seed=hd + Hq + 1)
    x = H.rand_np(15, (Bn, D), bf16=True)
    kc = H.rand_np(16, (Bn, Hkv, cap, hd), bf16=True)
    vc = H.rand_np(17, (Bn, Hkv, cap, hd), bf16=True)
    pos = O.decode_positions(lens, np.zeros(Bn, np.int64))
    ref, knew, vnew = O.layer_decode(sh, w, x, pos, kc, vc, lens)
    kn, vn = kc.copy(), vc.copy()
    for i, n in enumerate(lens):
        kn[i, :, n:] = np.nan
        vn[i, :, n:] = np.nan
    kd, vd = H.to_dev(kn, torch.bfloat16), H.to_dev(vn, torch.bfloat16)
    out = H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos), kd, vd,
                       H.ints_to_dev(lens))
    torch.cuda.synchronize()
    o = H.np64(out)
    assert np.isfinite(o).all()
    assert H.rel_err(o, ref) <= H.tol(sh)
    kg, vg = H.np64(kd), H.np64(vd)
    for i, n in enumerate(lens):
        assert H.rel_err(kg[i, :, n], knew[i]) <= H.tol(sh)
        assert H.rel_err(vg[i, :, n], vnew[i]) <= H.tol(sh)
        assert np.isnan(kg[i, :, n + 1:]).all() and np.isnan(vg[i, :, n + 1:]).all()


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_more_rows_than_one_tile(kind):
    """B = 70 bf16 rows: two 64-row tiles in the decode GEMMs (the projection's split-K tiles and
    the output GEMM's general path, which takes over above 64 rows), ragged lens."""
    sh = H.small_shape("bf16", kind, 128, 4, 1, 256, 512, 40 if kind == "sliding" else 0)
    Bn, cap = 70, 300
    rng = np.random.default_rng(70)
    lens = rng.integers(0, cap - 1, Bn).astype(np.int32)
    w, _, _ = layer_case(sh, 1, 8, seed=70)
    x = H.rand_np(71, (Bn, sh.hidden), bf16=True)
    kc = H.rand_np(72, (Bn, 1, cap, 128), bf16=True)
    vc = H.rand_np(73, (Bn, 1, cap, 128), bf16=True)
    pos = O.decode_positions(lens, rng.integers(-20, 20, Bn))
    ref, knew, vnew = O.layer_decode(sh, w, x, pos, kc, vc, lens)
    kd, vd = H.to_dev(kc, torch.bfloat16), H.to_dev(vc, torch.bfloat16)
    out = H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos), kd, vd,
                       H.ints_to_dev(lens))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x.astype(np.float64), ref, f"{kind} decode, B = 70")
    kg, vg = H.np64(kd), H.np64(vd)
    for i, n in enumerate(lens):
        assert H.rel_err(kg[i, :, n], knew[i]) <= H.tol(sh)
        assert H.rel_err(vg[i, :, n], vnew[i]) <= H.tol(sh)


def test_decode_skips_rows_with_lens_out_of_range():
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 256, 512, 40)
    lens = np.array([5, 64, 63], np.int32)  # capacity 64: row 1 is out of range
    Bn, cap = 3, 64
    w, _, _ = layer_case(sh, 1, 8, seed=3)
    x = H.rand_np(5, (Bn, sh.hidden))
    kc = H.rand_np(6, (Bn, 1, cap, 128))
    vc = H.rand_np(7, (Bn, 1, cap, 128))
    pos = O.decode_positions(lens, np.zeros(Bn, np.int64))
    out = torch.full((Bn, sh.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    kd, vd = H.to_dev(kc, torch.bfloat16), H.to_dev(vc, torch.bfloat16)
    H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos), kd, vd,
                 H.ints_to_dev(lens), out=out)
    torch.cuda.synchronize()
    assert torch.all(out[1] == 7.0)
    assert np.array_equal(H.np64(kd[1]), kc[1])
    ref, _, _ = O.layer_decode(sh, w, x, pos, kc, vc, lens, rows=[0, 2])
    assert H.rel_err(H.np64(out[[0, 2]]), ref) <= 2e-2


def test_prefill_then_decode_matches_longer_prefill():
    """Row L-1 of prefill(L) equals decode of token L-1 over the cache prefill(L-1) wrote."""
    for kind in ("sliding", "full"):
        sh = H.small_shape("bf16", kind, 128, 4, 1, 256, 512, 50)
        Bn, L = 2, 130
        w, x, pos = layer_case(sh, Bn, L, seed=21)
        wd = H.weights_to_dev(sh, w)
        cap = L + 5
        kc = torch.zeros((Bn, 1, cap, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        xd = H.to_dev(x, torch.bfloat16)
        full = H.run_prefill(sh, wd, xd, H.ints_to_dev(pos))
        H.run_prefill(sh, wd, xd[:, :L - 1].contiguous(), H.ints_to_dev(pos[:, :, :L - 1]), kv=(kc, vc))
        lens = torch.full((Bn,), L - 1, dtype=torch.int32, device="cuda")
        dec = H.run_decode(sh, wd, xd[:, L - 1].contiguous(), H.ints_to_dev(pos[:, :, L - 1]), kc, vc, lens)
        torch.cuda.synchronize()
        assert H.rel_err(H.np64(dec), H.np64(full[:, L - 1])) <= 2e-2


@pytest.mark.parametrize("kind,win", [("full", 0), ("sliding", 4096), ("sliding", 1000)])
def test_decode_long_cache_attention_probe(kind, win):
    """Caches past 4096 keys: the full layer merges up to 20 chunks of 256 keys (more than one
    group of 16 in the chunk merge) and the window-4096 layer up to 17. Each row's attention
    output is gated on its own scale through the probe layer (Wo = 64 I, w_down = 0), which a
    window or merge error cannot hide behind the MLP branch; the plain layer output too."""
    sh = H.small_shape("bf16", kind, 128, 4, 1, 512, 512, win)
    lens = np.array([0, 17, 255, 1000, 4095, 4096, 4097, 4500, 4999], np.int32)
    Bn, cap = len(lens), 5000
    w, _, _ = layer_case(sh, 1, 8, seed=91)
    x = H.rand_np(92, (Bn, sh.hidden))
    kc = H.rand_np(93, (Bn, 1, cap, 128))
    vc = H.rand_np(94, (Bn, 1, cap, 128))
    pos = O.decode_positions(lens, np.array([0, 3, -5, 0, 7, 0, -992, 0, 1], np.int64))
    wp = H.probe_weights(sh, w)
    kd, vd = H.to_dev(kc, torch.bfloat16), H.to_dev(vc, torch.bfloat16)
    args = (H.to_dev(x, torch.bfloat16), H.ints_to_dev(pos), kd, vd, H.ints_to_dev(lens))
    out = H.run_decode(sh, H.weights_to_dev(sh, w), *args)
    probe = H.run_decode(sh, H.weights_to_dev(sh, wp), *args)
    torch.cuda.synchronize()
    ref, _, _ = O.layer_decode(sh, w, x, pos, kc, vc, lens)
    ref_p, _, _ = O.layer_decode(sh, wp, x, pos, kc, vc, lens)
    check_layer_out(sh, out, x, ref, f"decode {kind} W={win}")
    H.check_attn_rows(sh, probe, x, (ref_p - x) / H.PROBE_SCALE, f"decode {kind} W={win}")


@pytest.mark.parametrize("offset", [8100, 32700])
def test_prefill_then_decode_at_large_positions(offset):
    """Row L-1 of prefill(L) against decode of token L-1 over prefill(L-1)'s cache with the
    positions moved up by `offset`, where the rotation angles are largest. The prefill
    epilogue evaluates each angle in turns with the hardware sine and cosine, the decode
    epilogue in radians with the accurate sincosf; both stay within the gate of each other and
    of the oracle, and so do the rotated keys of the last token."""
    sh = H.small_shape("bf16", "sliding", 128, 4, 1, 512, 512, 50)
    Bn, L = 2, 130
    w, x, pos = layer_case(sh, Bn, L, seed=23)
    pos = pos + offset
    wd = H.weights_to_dev(sh, w)
    cap = L + 5
    kc = torch.zeros((Bn, 1, cap, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kf = torch.zeros_like(kc)
    xd = H.to_dev(x, torch.bfloat16)
    full = H.run_prefill(sh, wd, xd, H.ints_to_dev(pos), kv=(kf, torch.zeros_like(kc)))
    H.run_prefill(sh, wd, xd[:, :L - 1].contiguous(), H.ints_to_dev(pos[:, :, :L - 1]), kv=(kc, vc))
    lens = torch.full((Bn,), L - 1, dtype=torch.int32, device="cuda")
    dec = H.run_decode(sh, wd, xd[:, L - 1].contiguous(), H.ints_to_dev(pos[:, :, L - 1]), kc, vc, lens)
    torch.cuda.synchronize()
    ref, st = O.layer_prefill(sh, w, x, pos, return_stages=True)
    assert H.rel_err(H.np64(dec), H.np64(full[:, L - 1])) <= 2e-2
    check_layer_out(sh, dec, x[:, L - 1], ref[:, L - 1], f"decode at offset {offset}")
    check_layer_out(sh, full, x, ref, f"prefill at offset {offset}")
    assert H.rel_err(H.np64(kc[:, :, L - 1]), st["k"][:, :, L - 1]) <= 2e-2  # decode's rotation
    assert H.rel_err(H.np64(kf[:, :, L - 1]), st["k"][:, :, L - 1]) <= 2e-2  # prefill's rotation


# ------------------------------------------------------------------------------ logits
@pytest.mark.parametrize("dt,R,D,V", [("bf16", 37, 256, 1000), ("bf16", 300, 512, 2048), ("f32", 20, 256, 517)])
def test_logits_parity_and_scale(dt, R, D, V):
    bf = dt == "bf16"
    h = H.rand_np(31, (R, D), bf16=bf)
    nw = H.rand_np(32, (D,), std=0.02, mean=1.0, bf16=bf)
    E = H.rand_np(33, (V, D), std=0.02, bf16=bf)
    td = torch.bfloat16 if bf else torch.float32
    hd_, nd, Ed = H.to_dev(h, td), H.to_dev(nw, td), H.to_dev(E, td)
    c = 1 if bf else 0
    lg = H.run_logits(hd_, nd, 1e-5, Ed, 0.0625, c)
    l1 = H.run_logits(hd_, nd, 1e-5, Ed, 1.0, c)
    torch.cuda.synchronize()
    ref = O.logits(h, nw, 1e-5, E, 0.0625)
    assert H.rel_err(H.np64(lg), ref) <= (2e-2 if bf else 1e-4)
    assert torch.equal(lg, l1 * 0.0625)


def test_tiny_fp32_workload_against_both_oracles():
    """The fp32 parity workload exactly (hidden 256, 4/1 heads, hd 64, I 1024, MRoPE [12,10,10],
    window 32, 128 text tokens with t = h = w = index, N(0, 0.02) weights): the GPU layer against
    the fp64 numpy oracle and against the plain fp32 C++ reference, 1e-4 each."""
    from oracle import ref as R
    cfg = W.WORKLOADS["tiny_sliding_f32"]
    sh, L = cfg["shape"], cfg["L"]
    w = W.make_layer_weights(sh, W.Stream.TINY_SLIDING_F32, 0)
    x = W.make_layer_input(sh, W.Stream.TINY_SLIDING_F32, L).reshape(1, L, sh.hidden)
    p = np.arange(L)
    pos = np.stack([p, p, p])[:, None, :]
    out = H.run_prefill(sh, H.weights_to_dev(sh, w), H.to_dev(x, torch.float32), H.ints_to_dev(pos))
    torch.cuda.synchronize()
    got = H.np64(out)
    ref64 = O.layer_prefill(sh, w, x, pos)
    ref32, _, _ = R.layer_forward(sh, w, x, pos)
    assert H.rel_err(got, ref64) <= 1e-4
    assert H.rel_err(got, ref32) <= 1e-4
    check_layer_out(sh, out, x, ref64, "fp32 workload")
