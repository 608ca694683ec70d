"""Degenerate and maximum-size cases through the C ABI, against the oracles.

* one-token prefill (B = 1 and B = 3, sliding and full, bf16 and fp32) and two-token rows;
* decode over an empty cache (the new token attends only to itself) and a single row;
* decode with a window of one or two keys, one row writing the cache's last slot;
* the one-row, one-word logits head and a three-word vocabulary;
* position ids of a row that is a single image (no text at all) and of the longest row
  the library accepts (COMPASS_MAX_TOKENS_PER_ROW tokens, images spread over it), bit-exact
  against the C++ reference, plus one token more rejected on the host.
"""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from oracle import ref as R
from synth import workloads as W
from tests import helpers as H
from tests.test_gpu_small import check_layer_out, layer_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["sliding", "full"])
@pytest.mark.parametrize("Bn,L", [(1, 1), (3, 1), (2, 2)])
def test_tiny_prefill(dt, kind, Bn, L):
    sh = H.small_shape(dt, kind, 64, 4, 2, 256, 256, 3)
    w, x, pos = layer_case(sh, Bn, L, seed=30 + L)
    ref, st = O.layer_prefill(sh, w, x, pos, return_stages=True)
    td = H.tdtype(sh)
    kc = torch.full((Bn, 2, L, 64), float("nan"), dtype=td, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = H.run_prefill(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kv=(kc, vc))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x, ref, f"prefill B={Bn} L={L}")
    assert H.rel_err(H.np64(kc), st["k"]) <= H.tol(sh)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_over_empty_cache_and_single_row(dt, kind):
    sh = H.small_shape(dt, kind, 128, 4, 1, 256, 512, 16)
    bf = dt == "bf16"
    w, _, _ = layer_case(sh, 1, 8, seed=41)
    for lens in (np.array([0], np.int32), np.array([0, 0, 5], np.int32)):
        Bn, cap = len(lens), 8
        x = H.rand_np(42, (Bn, sh.hidden), bf16=bf)
        kc = H.rand_np(43, (Bn, 1, cap, 128), bf16=bf)
        vc = H.rand_np(44, (Bn, 1, cap, 128), bf16=bf)
        pos = O.decode_positions(lens, np.zeros(Bn, np.int64))
        ref, _, vnew = O.layer_decode(sh, w, x, pos, kc, vc, lens)
        td = H.tdtype(sh)
        out = H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), H.to_dev(kc, td),
                           H.to_dev(vc, td), H.ints_to_dev(lens))
        torch.cuda.synchronize()
        check_layer_out(sh, out, x, ref, f"decode lens={lens.tolist()}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("win", [1, 2])
def test_decode_window_of_one_or_two_keys_and_last_cache_slot(dt, win):
    """A sliding decode layer whose window holds only the new key (or it and one more), with
    one row writing the cache's last slot (lens = capacity - 1)."""
    sh = H.small_shape(dt, "sliding", 128, 4, 1, 256, 512, win)
    bf = dt == "bf16"
    w, _, _ = layer_case(sh, 1, 8, seed=47 + win)
    lens = np.array([0, 1, 2, 37, 299], np.int32)
    Bn, cap = len(lens), 300
    x = H.rand_np(48, (Bn, sh.hidden), bf16=bf)
    kc = H.rand_np(49, (Bn, 1, cap, 128), bf16=bf)
    vc = H.rand_np(50, (Bn, 1, cap, 128), bf16=bf)
    pos = O.decode_positions(lens, np.array([0, 3, -2, 10, -100], np.int64))
    ref, knew, vnew = O.layer_decode(sh, w, x, pos, kc, vc, lens)
    td = H.tdtype(sh)
    kd, vd = H.to_dev(kc, td), H.to_dev(vc, td)
    out = H.run_decode(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kd, vd,
                       H.ints_to_dev(lens))
    torch.cuda.synchronize()
    check_layer_out(sh, out, x, ref, f"decode window {win}")
    kg = H.np64(kd)
    for i, n in enumerate(lens):
        assert H.rel_err(kg[i, :, n], knew[i]) <= H.tol(sh), f"row {i} new K"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 3])
def test_logits_one_row_tiny_vocab(dt, V):
    bf = dt == "bf16"
    h = H.rand_np(50, (1, 64), bf16=bf)
    nw = H.rand_np(51, (64,), std=0.1, mean=1.0, bf16=bf)
    E = H.rand_np(52, (V, 64), bf16=bf)
    td = torch.bfloat16 if bf else torch.float32
    cd = 1 if bf else 0
    got = H.run_logits(H.to_dev(h, td), H.to_dev(nw, td), 1e-5, H.to_dev(E, td), 0.25, cd)
    b = H.B()
    ws = H.workspace(b.compass_logits_argmax_workspace_size(1, 64, V, cd))
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    b.compass_logits_argmax(H.to_dev(h, td), H.to_dev(nw, td), 1e-5, H.to_dev(E, td), 0.25, tok, None, ws, cd)
    torch.cuda.synchronize()
    ref = O.logits(h, nw, 1e-5, E, 0.25)
    assert H.rel_err(H.np64(got), ref) <= (2e-2 if bf else 1e-4)
    assert int(tok.item()) == int(np.argmax(got.cpu().numpy()[0]))


def gpu_positions(tok, grid, off):
    b = H.B()
    Bn, L = tok.shape
    pos = torch.full((3, Bn, L), -7, dtype=torch.int32, device="cuda")
    delta = torch.full((Bn,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((Bn,), -7, dtype=torch.int32, device="cuda")
    b.compass_mrope_positions(H.ints_to_dev(tok), W.IMAGE_TOKEN_ID, H.ints_to_dev(grid), H.ints_to_dev(off), 2,
                              pos, delta, status)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), delta.cpu().numpy(), status.cpu().numpy()


def test_positions_row_that_is_one_image():
    img = W.IMAGE_TOKEN_ID
    tok = np.full((1, 12), img, np.int32)  # two images, merged grids (3, 2, 1) and (1, 2, 3): 6 pads each
    grid = np.array([[3, 4, 2], [1, 4, 6]], np.int32)
    off = np.array([0, 2], np.int32)
    pos, delta, status = gpu_positions(tok, grid, off)
    ref_pos, ref_delta = O.mrope_positions(tok, img, grid, off, 2)
    assert status.tolist() == [0]
    np.testing.assert_array_equal(pos, ref_pos)
    np.testing.assert_array_equal(delta, ref_delta)


def test_positions_longest_row():
    """COMPASS_MAX_TOKENS_PER_ROW tokens with 40 images of assorted grids spread over the row."""
    L = 524288
    img = W.IMAGE_TOKEN_ID
    tok = W.text_tokens(61, L).reshape(1, L).copy()
    grids = []
    r = np.random.default_rng(62)
    p = 100
    for _ in range(40):
        g = (int(r.integers(1, 4)), 2 * int(r.integers(1, 20)), 2 * int(r.integers(1, 20)))
        n = g[0] * (g[1] // 2) * (g[2] // 2)
        tok[0, p:p + n] = img
        grids.append(g)
        p += n + int(r.integers(0, 9000))
    assert p < L
    grid = np.array(grids, np.int32)
    off = np.array([0, len(grids)], np.int32)
    pos, delta, status = gpu_positions(tok, grid, off)
    code, ref_pos, ref_delta = R.mrope_positions(tok, img, grid, off, 2)
    assert code == 0 and status.tolist() == [0]
    np.testing.assert_array_equal(pos, ref_pos)
    np.testing.assert_array_equal(delta, ref_delta)
    b = H.B()
    longer = torch.zeros((1, L + 1), dtype=torch.int32, device="cuda")
    out = torch.zeros((3, 1, L + 1), dtype=torch.int32, device="cuda")
    d1 = torch.zeros((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(b.CompassError) as e:
        b.compass_mrope_positions(longer, img, H.ints_to_dev(grid), H.ints_to_dev(np.array([0, 0])), 2, out, d1, d1)
    assert e.value.code == b.COMPASS_E_UNSUPPORTED


def test_prefill_large_logits():
    """Scores spread over ~33 log2 units (q and k weights x5, gate / up x0.1 so attention
    dominates the branch sum): near one-hot rows and repeated raises of the softmax reference.

    At this spread the storage roundings decide the result by percents: the layer feeds the
    bf16-rounded LayerNorm output to the projection and stores q / k / v in bf16, and that
    alone moves the fp64 oracle's output by 2.2e-2 here. So the reference, built from the
    oracle's functions alone, follows the same storage steps: a = bf16(LN(x)), q = bf16(a Wq^T),
    k = bf16(a Wk^T), v = bf16(a Wv^T), act = bf16(silu(a Wg^T) * (a Wu^T)), then the oracle's
    attention in fp64 and the bf16-rounded attention output through Wo; the kernel's cache is
    checked against that k and v. What remains is the softmax arithmetic
    (bf16 P) plus rare one-ulp differences: 3.2e-3 measured. A softmax that loses precision fails
    the 8e-3 gate (re-rounding q * log2(e) / sqrt(hd) to bf16, for one, gives 2.5e-2 here in a
    CPU emulation). A full-attention (NoPE) layer, so no rotation angle enters q."""
    sh = H.small_shape("bf16", "full", 128, 4, 1, 256, 512, 0)
    Bn, L, Hq, hd = 1, 400, 4, 128
    w, x, pos = layer_case(sh, Bn, L, seed=77)
    w = dict(w)
    for name, f in (("wq", 5.0), ("wk", 5.0), ("w_gate", 0.1), ("w_up", 0.1)):
        w[name] = H.bf16_round(w[name] * f)
    td = H.tdtype(sh)
    kc = torch.zeros((Bn, sh.n_kv_heads, L, hd), dtype=td, device="cuda")
    vc = torch.zeros_like(kc)
    out = H.run_prefill(sh, H.weights_to_dev(sh, w), H.to_dev(x, td), H.ints_to_dev(pos), kv=(kc, vc))
    torch.cuda.synchronize()
    f64 = lambda n: w[n].astype(np.float64)
    a = H.bf16_round(O.layer_norm(x[0], w["ln_w"], sh.ln_eps))
    q = H.bf16_round(a @ f64("wq").T).reshape(L, Hq, hd).transpose(1, 0, 2)
    k = H.bf16_round(a @ f64("wk").T).reshape(L, sh.n_kv_heads, hd).transpose(1, 0, 2)
    v = H.bf16_round(a @ f64("wv").T).reshape(L, sh.n_kv_heads, hd).transpose(1, 0, 2)
    assert H.rel_err(H.np64(kc)[0], k) <= 2e-2 and H.rel_err(H.np64(vc)[0], v) <= 2e-2
    s = np.einsum("hqd,hkd->hqk", q, np.repeat(k, Hq // sh.n_kv_heads, axis=0)) / np.sqrt(hd)
    spread = np.log2(np.e) * float(np.std(s[:, np.tril(np.ones((L, L), bool))]))
    assert spread > 25.0, f"score spread {spread:.1f} log2 units: the case is not large-logit"
    o_flat = H.bf16_round(O.attention(q, k, v, sh.kind, sh.window))   # [L, Hq * hd]
    act = H.bf16_round(O.silu(a @ f64("w_gate").T) * (a @ f64("w_up").T))
    d_ref = o_flat @ f64("wo").T + act @ f64("w_down").T
    ref = x[0].astype(np.float64) + d_ref
    d_gpu = H.np64(out)[0] - x[0]
    e_branch = float(np.max(np.abs(d_gpu - d_ref) - 2.0 ** -8 * np.abs(ref)) / np.max(np.abs(d_ref)))
    print(f"large-logit layer: branch-sum rel err {e_branch:.3e} at score spread {spread:.1f}")
    assert e_branch <= 8e-3, f"branch-sum rel err {e_branch:.3e} at score spread {spread:.1f}"
