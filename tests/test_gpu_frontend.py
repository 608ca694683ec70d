"""GPU parity of the token-id front end and the greedy head, through the C ABI:
compass_embed (table gather + image-row replacement), compass_decode_positions,
compass_logits_argmax, and a whole greedy generation (positions, embedding, a 4-layer
prefill with deepstack, then decode steps feeding each argmax token back) against
oracle.greedy_generate.

Gates: embedding and positions are copies / integer arithmetic, compared bit-exactly.
Greedy tokens: where the oracle's top-2 logit gap exceeds twice the logits tolerance
(1e-4 fp32, 2e-2 bf16, relative to the largest |logit|) the token must equal the
oracle's; elsewhere several tokens are correct and the chosen one must be within that
tolerance of the oracle's maximum. Tokens also equal the first argmax of compass_logits'
own output (the same fp32 values).
"""
import numpy as np
import pytest
import torch

from oracle import compass_oracle as O
from synth import stream_seed
from synth import workloads as W
import synth.rng_torch as RT
from tests import helpers as H
import cohere2_block_mrope_amd.stack as S

pytestmark = pytest.mark.gpu


def embed_dev(tokens, E, rows=None, feats=None, dtype=1):
    b = H.B()
    R, D = tokens.numel(), E.shape[1]
    h = torch.full((R, D), float("nan"), dtype=E.dtype, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    b.compass_embed(tokens, E, rows, feats, h, st, dtype)
    return h, st


def argmax_dev(h, nw, eps, E, scale, dtype):
    b = H.B()
    R, D = h.shape
    ws = H.workspace(b.compass_logits_argmax_workspace_size(R, D, E.shape[0], dtype))
    tok = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    mx = torch.empty((R,), dtype=torch.float32, device="cuda")
    b.compass_logits_argmax(h, nw, eps, E, scale, tok, mx, ws, dtype)
    return tok, mx


def check_tokens(tok, ref_logits, tol):
    """tok [R] from the GPU; ref_logits [R, V] fp64 from the oracle."""
    tok = np.asarray(tok)
    srt = np.sort(ref_logits, axis=1)
    scale = np.max(np.abs(ref_logits), axis=1)
    gap = srt[:, -1] - srt[:, -2]
    best = np.argmax(ref_logits, axis=1)
    clear = gap > 2 * tol * scale
    assert np.array_equal(tok[clear], best[clear]), (tok[clear], best[clear])
    picked = ref_logits[np.arange(len(tok)), tok]
    assert np.all(srt[:, -1] - picked <= 2 * tol * scale)
    return int(clear.sum())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_embed_parity_with_image_rows(dtype):
    r = np.random.default_rng(11)
    V, D, R = 777, 192, 301
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cd = 1 if dtype == "bf16" else 0
    E = H.rand_np(20, (V, D))
    tokens = r.integers(0, V, R)
    rows = np.sort(r.choice(R, 40, replace=False))
    feats = H.rand_np(21, (40, D))
    h, st = embed_dev(H.ints_to_dev(tokens), H.to_dev(E, tdt), H.ints_to_dev(rows), H.to_dev(feats, tdt), cd)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    np.testing.assert_array_equal(H.np64(h), O.embed(tokens, E, rows, feats))
    # no image rows, one token
    h1, st1 = embed_dev(H.ints_to_dev(tokens[:1]), H.to_dev(E, tdt), None, None, cd)
    torch.cuda.synchronize()
    assert int(st1.item()) == 0
    np.testing.assert_array_equal(H.np64(h1), O.embed(tokens[:1], E))


def test_embed_status_bits():
    """Ids outside [0, V) give zero rows and bit 0; image rows outside [0, R) are skipped, bit 1."""
    V, D = 100, 64
    E = H.rand_np(30, (V, D))
    tokens = np.array([3, -1, 99, 100, 7])
    feats = H.rand_np(31, (2, D))
    h, st = embed_dev(H.ints_to_dev(tokens), H.to_dev(E, torch.bfloat16), H.ints_to_dev([4, 5]),
                      H.to_dev(feats, torch.bfloat16))
    torch.cuda.synchronize()
    assert int(st.item()) == 3
    got = H.np64(h)
    np.testing.assert_array_equal(got[[0, 2]], E[[3, 99]])
    assert not got[[1, 3]].any()
    np.testing.assert_array_equal(got[4], feats[0])
    h, st = embed_dev(H.ints_to_dev(tokens[[0, 2, 4]]), H.to_dev(E, torch.bfloat16), H.ints_to_dev([-1]),
                      H.to_dev(feats[:1], torch.bfloat16))
    torch.cuda.synchronize()
    assert int(st.item()) == 2
    np.testing.assert_array_equal(H.np64(h), E[[3, 99, 7]])


@pytest.mark.parametrize("B", [1, 64, 300])
def test_decode_positions(B):
    b = H.B()
    r = np.random.default_rng(B)
    lens = r.integers(0, 9000, B)
    delta = r.integers(-2000, 50, B)
    ld, dd = H.ints_to_dev(lens), H.ints_to_dev(delta)
    pos = torch.full((3, B), -1, dtype=torch.int32, device="cuda")
    b.compass_decode_positions(ld, dd, 0, pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pos.cpu().numpy(), O.decode_positions(lens, delta))
    np.testing.assert_array_equal(ld.cpu().numpy(), lens)
    b.compass_decode_positions(ld, dd, 1, pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pos.cpu().numpy(), O.decode_positions(lens + 1, delta))
    np.testing.assert_array_equal(ld.cpu().numpy(), lens + 1)
    b.compass_decode_positions(ld, None, 3, pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pos.cpu().numpy(), O.decode_positions(lens + 4, np.zeros(B, np.int64)))


@pytest.mark.parametrize("R,V", [(1, 1000), (37, 1001), (100, 777), (300, 513)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logits_argmax_small(dtype, R, V):
    """Row counts that take each logits tile shape (<= 64, <= 128, > 128 rows) and a ragged vocab."""
    D = 256
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cd, tol = (1, 2e-2) if dtype == "bf16" else (0, 1e-4)
    h = H.rand_np(40 + R, (R, D))
    nw = H.rand_np(41, (D,), std=0.1, mean=1.0)
    E = H.rand_np(42, (V, D), std=0.5)
    scale = 0.0625
    hd, nd, Ed = H.to_dev(h, tdt), H.to_dev(nw, tdt), H.to_dev(E, tdt)
    tok, mx = argmax_dev(hd, nd, 1e-5, Ed, scale, cd)
    lg = H.run_logits(hd, nd, 1e-5, Ed, scale, cd)
    torch.cuda.synchronize()
    ref = O.logits(h, nw, 1e-5, E, scale)
    assert H.rel_err(H.np64(lg), ref) <= tol
    lgn = lg.cpu().numpy()
    tk = tok.cpu().numpy()
    np.testing.assert_array_equal(tk, np.argmax(lgn, axis=1))
    np.testing.assert_array_equal(mx.cpu().numpy(), lgn.max(axis=1))
    check_tokens(tk, ref, tol)


def test_logits_argmax_ties_and_strided_rows():
    """Equal logits go to the smallest id; rows taken with a stride (the last token of each
    [L, D] batch row) give the tokens of the same rows copied out."""
    D, V, Bn, L = 128, 900, 5, 7
    h3 = H.rand_np(50, (Bn, L, D))
    nw = H.rand_np(51, (D,), std=0.1, mean=1.0)
    E = H.rand_np(52, (V, D), std=0.5)
    hd3 = H.to_dev(h3, torch.bfloat16)
    nd = H.to_dev(nw, torch.bfloat16)
    tok_s, mx_s = argmax_dev(hd3[:, -1], nd, 1e-5, H.to_dev(E, torch.bfloat16), 0.25, 1)
    tok_c, mx_c = argmax_dev(hd3[:, -1].contiguous(), nd, 1e-5, H.to_dev(E, torch.bfloat16), 0.25, 1)
    torch.cuda.synchronize()
    assert torch.equal(tok_s, tok_c) and torch.equal(mx_s, mx_c)
    t0 = int(tok_c[0])
    E2 = E.copy()
    lo, hi = t0 // 2, min(t0 + 1 + (V - t0) // 2, V - 1)
    E2[lo] = E2[t0]   # an equal column below: it wins
    if hi != t0:
        E2[hi] = E2[t0]  # an equal column above: it does not
    tok2, mx2 = argmax_dev(hd3[:, -1], nd, 1e-5, H.to_dev(E2, torch.bfloat16), 0.25, 1)
    allzero, _ = argmax_dev(hd3[:, -1], nd, 1e-5, torch.zeros((V, D), dtype=torch.bfloat16, device="cuda"), 0.25, 1)
    torch.cuda.synchronize()
    assert int(tok2[0]) == (lo if t0 > 0 else 0)
    assert float(mx2[0]) == float(mx_c[0])
    assert not allzero.any()


def test_logits_argmax_decode_batch_full_vocab():
    """Decode-batch greedy head: 64 rows, hidden 2048, tied 256000-vocab table, logit_scale 0.0625."""
    R, D, V, scale = 64, 2048, 256000, 0.0625
    h = RT.normal(stream_seed(W.Stream.DECODE_STACK, 0, W.TensorId.X), R * D).to(torch.bfloat16).view(R, D)
    E = RT.normal(stream_seed(W.Stream.STACK_LOGITS, 0, W.TensorId.EMBED), V * D, std=0.02).to(torch.bfloat16).view(V, D)
    nw = torch.ones(D, dtype=torch.bfloat16, device="cuda")
    tok, mx = argmax_dev(h, nw, 1e-5, E, scale, 1)
    lg = H.run_logits(h, nw, 1e-5, E, scale, 1)
    torch.cuda.synchronize()
    lgn = lg.cpu().numpy()
    assert np.array_equal(mx.cpu().numpy(), lgn.max(axis=1))
    assert np.array_equal(tok.cpu().numpy(), np.argmax(lgn, axis=1))
    rows = [0, 17, 63]
    ref = O.logits(H.np64(h)[rows], np.ones(D), 1e-5, H.np64(E), scale)
    check_tokens(tok.cpu().numpy()[rows], ref, 2e-2)
    # the stored logits themselves are within the bf16 gate
    assert H.rel_err(H.np64(lg[rows]), ref) <= 2e-2


def gpu_greedy_generate(sh, layer_w, E, nw, scale, tokens, grid, off, feats, ds, img_id, merge, n_new):
    """The greedy loop on the device through the C ABI; returns tokens [B, n_new] and the
    final hidden row of each step [B, n_new, D]."""
    b = H.B()
    tdt, cd = H.tdtype(sh), H.cdtype(sh)
    Bn, L = tokens.shape
    D = sh.hidden
    td = H.ints_to_dev(tokens)
    pos = torch.empty((3, Bn, L), dtype=torch.int32, device="cuda")
    delta = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    st = torch.empty((Bn,), dtype=torch.int32, device="cuda")
    b.compass_mrope_positions(td, img_id, H.ints_to_dev(grid), H.ints_to_dev(off), merge, pos, delta, st)
    pad = np.flatnonzero(tokens.reshape(-1) == img_id)
    pad_d = H.ints_to_dev(pad)
    Ed, nd = H.to_dev(E, tdt), H.to_dev(nw, tdt)
    h, est = embed_dev(td.view(-1), Ed, pad_d, H.to_dev(feats, tdt), cd)
    h = h.view(Bn, L, D)
    cap = L + n_new
    caches = []
    for i, w in enumerate(layer_w):
        shi = sh.with_kind(S.layer_kind(i))
        kc = torch.zeros((Bn, sh.n_kv_heads, cap, sh.head_dim), dtype=tdt, device="cuda")
        vc = torch.zeros_like(kc)
        dsd = H.to_dev(ds[i], tdt) if i < 3 else None
        H.run_prefill(shi, w, h, pos, kv=(kc, vc), ds_rows=pad_d if i < 3 else None, ds=dsd, out=h)
        caches.append((kc, vc))
    out = torch.empty((Bn, n_new), dtype=torch.int32, device="cuda")
    hid = torch.empty((Bn, n_new, D), dtype=tdt, device="cuda")
    hid[:, 0] = h[:, -1]
    tok, _ = argmax_dev(h[:, -1], nd, sh.ln_eps, Ed, scale, cd)
    lens = torch.full((Bn,), L, dtype=torch.int32, device="cuda")
    p3 = torch.empty((3, Bn), dtype=torch.int32, device="cuda")
    for step in range(n_new):
        out[:, step] = tok
        if step == n_new - 1:
            break
        x, _ = embed_dev(tok, Ed, None, None, cd)
        b.compass_decode_positions(lens, delta, 0 if step == 0 else 1, p3)
        for i, w in enumerate(layer_w):
            shi = sh.with_kind(S.layer_kind(i))
            H.run_decode(shi, w, x, p3, caches[i][0], caches[i][1], lens, out=x)
        hid[:, step + 1] = x
        tok, _ = argmax_dev(x, nd, sh.ln_eps, Ed, scale, cd)
    torch.cuda.synchronize()
    assert not st.any() and int(est.item()) == 0
    return out.cpu().numpy(), H.np64(hid)


def test_greedy_generation_fp32():
    """Prompt [2, 24] with a 2 x 2 merged image in row 0 (rope_delta -2), 4-layer [S, S, S, F]
    fp32 stack with deepstack, window 8, then 6 greedy tokens fed back through decode."""
    sh = H.small_shape("f32", "sliding", hd=64, Hq=4, Hkv=1, D=256, I=512, window=8)
    V, IMG, n_new = 500, 499, 6
    # Matrices scaled to std 0.2 so that the layers, not the last token's own embedding row,
    # decide the next token (the generated sequence changes from step to step).
    layer_w = [{k: (v if k == "ln_w" else 10.0 * v) for k, v in W.make_layer_weights(sh, 90, i).items()}
               for i in range(4)]
    r = np.random.default_rng(91)
    E = H.rand_np(92, (V, sh.hidden), std=0.5)
    nw = H.rand_np(93, (sh.hidden,), std=0.1, mean=1.0)
    tokens = r.integers(0, V - 1, (2, 24))
    tokens[0, 5:9] = IMG
    grid, off = np.array([[1, 4, 4]]), np.array([0, 1, 1])
    feats = H.rand_np(94, (4, sh.hidden))
    ds = [H.rand_np(95 + i, (4, sh.hidden), std=0.5) for i in range(3)]
    scale = 0.25
    ref_tok, ref_hid = O.greedy_generate(sh, layer_w, E, nw, scale, tokens, grid, off, feats, ds, IMG, 2, n_new,
                                         return_hidden=True)
    wdev = [H.weights_to_dev(sh, w) for w in layer_w]
    got_tok, got_hid = gpu_greedy_generate(sh, wdev, E, nw, scale, tokens, grid, off, feats, ds, IMG, 2, n_new)
    # Compare step by step while the generated prefixes agree (after a legitimately
    # different pick of a near-tied token the two sequences continue differently).
    compared = 0
    for k in range(n_new):
        assert H.rel_err(got_hid[:, k], ref_hid[:, k]) <= 1e-4, k
        ref_l = O.logits(ref_hid[:, k], nw, sh.ln_eps, E, scale)
        compared += check_tokens(got_tok[:, k], ref_l, 1e-4)
        if not np.array_equal(got_tok[:, k], ref_tok[:, k]):
            break
    assert compared >= 2 * n_new - 2, compared
    assert len(set(ref_tok[0].tolist())) > 1
