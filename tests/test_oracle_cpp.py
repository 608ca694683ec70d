"""The plain fp32 C++ reference (oracle/compass_ref.cpp) against the pinned fp64 numpy
oracle: two independent CPU implementations of the same definitions. Position ids
bit-exact (including the error cases); layer outputs, rotated keys and logits within
2e-5 relative (fp32 storage of every intermediate). CPU only."""
import dataclasses

import numpy as np
import pytest

from oracle import compass_oracle as O
from oracle import ref as R
from synth import workloads as W
from tests.test_oracle_pins import mixed_pos, rand_weights, tiny_shape

TOL = 2e-5


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.fixture(scope="module", autouse=True)
def built():
    R.build()


def token_rows(B, L, seed):
    """Rows with text, images of a few merged grids (back to back too) and text."""
    layouts = [[(3, (1, 4, 6)), (2, (2, 4, 4)), (0, (1, 2, 2))], [(7, (1, 8, 12))], [], [(0, (1, 6, 2))]]
    toks, grids, offs = [], [], [0]
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
    return np.array(toks, np.int32), np.array(grids, np.int32).reshape(-1, 3), np.array(offs, np.int32)


def test_positions_bit_exact():
    tok, grid, off = token_rows(4, 90, 3)
    code, pos, delta = R.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    ref_pos, ref_delta = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    assert code == 0
    np.testing.assert_array_equal(pos, ref_pos)
    np.testing.assert_array_equal(delta, ref_delta)
    tok, grid, off = W.image_text_row(seed=5, L=4096)
    code, pos, delta = R.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    ref_pos, ref_delta = O.mrope_positions(tok, W.IMAGE_TOKEN_ID, grid, off, 2)
    assert code == 0 and int(delta[0]) == -992
    np.testing.assert_array_equal(pos, ref_pos)


@pytest.mark.parametrize("case,code", [("extra pads", O.POS_EXTRA_PADS), ("bad grid", O.POS_BAD_GRID),
                                       ("span", O.POS_SPAN_MISMATCH), ("unused", O.POS_UNUSED_IMAGES),
                                       ("grid past int64", O.POS_SPAN_MISMATCH)])
def test_position_errors_match(case, code):
    img = W.IMAGE_TOKEN_ID
    tok = np.array([[5, img, img, img, img, 6]], np.int32)
    grid, off = np.array([[1, 4, 4]], np.int32), np.array([0, 1], np.int32)
    if case == "extra pads":
        off = np.array([0, 0], np.int32)
    elif case == "bad grid":
        grid = np.array([[1, 3, 4]], np.int32)
    elif case == "grid past int64":  # merged grid 2^21 x 2^21 x 2^22: 2^64 pads
        grid = np.array([[1 << 21, 1 << 22, 1 << 23]], np.int32)
    elif case == "span":
        tok = np.array([[5, img, img, 7, img, 6]], np.int32)
    else:
        grid, off = np.array([[1, 4, 4], [1, 2, 2]], np.int32), np.array([0, 2], np.int32)
    got, _, _ = R.mrope_positions(tok, img, grid, off, 2)
    with pytest.raises(O.PositionError) as e:
        O.mrope_positions(tok, img, grid, off, 2)
    assert got == code == e.value.code


SHAPES = [
    ("sliding", "interleaved", dict(window=3, Hq=4, Hkv=2, hd=8, D=32, I=48, section=(2, 1, 1))),
    ("full", "interleaved", dict(window=3, Hq=4, Hkv=1, hd=16, D=64, I=64, section=(4, 2, 2))),
    ("sliding", "sections", dict(window=5, Hq=4, Hkv=2, hd=16, D=64, I=64, section=(4, 2, 2))),
    ("sliding", "interleaved", dict(window=40, Hq=8, Hkv=2, hd=64, D=128, I=96, section=(12, 10, 10))),
]


def shape_of(kind, layout, kw):
    sh = tiny_shape(kind, **kw)
    return dataclasses.replace(sh, rope_layout=layout)


@pytest.mark.parametrize("kind,layout,kw", SHAPES, ids=[f"{s[0]}-{s[1]}-hd{s[2]['hd']}" for s in SHAPES])
def test_layer_prefill_matches(kind, layout, kw):
    sh = shape_of(kind, layout, kw)
    w = rand_weights(sh, seed=kw["hd"], std=0.2)
    r = np.random.default_rng(kw["D"])
    B, L = 2, 23
    x = r.standard_normal((B, L, sh.hidden)).astype(np.float32)
    pos = mixed_pos(B, L, seed=4)
    rows = np.array([1, 5, 30], np.int32)
    ds = r.standard_normal((3, sh.hidden)).astype(np.float32)
    ref, st = O.layer_prefill(sh, w, x, pos, rows, ds, return_stages=True)
    out, kn, vn = R.layer_forward(sh, w, x, pos, ds_rows=rows, ds=ds)
    assert rel(out, ref) <= TOL
    assert rel(kn, st["k"]) <= TOL and rel(vn, st["v"]) <= TOL


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_chunk_and_decode_match(kind):
    sh = shape_of(kind, "interleaved", dict(window=6, Hq=4, Hkv=2, hd=16, D=64, I=64, section=(4, 2, 2)))
    w = rand_weights(sh, seed=9, std=0.2)
    r = np.random.default_rng(10)
    cap = 40
    kc = r.standard_normal((3, 2, cap, 16))
    vc = r.standard_normal((3, 2, cap, 16))
    start = np.array([0, 9, 30])
    L = 7
    x = r.standard_normal((3, L, 64)).astype(np.float32)
    pos = mixed_pos(3, L, seed=11)
    ref = O.layer_prefill_chunk(sh, w, x, pos, kc, vc, start)
    got = R.layer_forward(sh, w, x, pos, kc, vc, start)
    for a, b in zip(got, ref):
        assert rel(a, b) <= TOL
    lens = np.array([0, 17, 39])
    xd = r.standard_normal((3, 64)).astype(np.float32)
    p1 = O.decode_positions(lens, np.array([0, -2, 5]))
    ref_d, knew, vnew = O.layer_decode(sh, w, xd, p1, kc, vc, lens)
    out_d, kn, vn = R.layer_forward(sh, w, xd[:, None], p1[:, :, None], kc, vc, lens)
    assert rel(out_d[:, 0], ref_d) <= TOL
    assert rel(kn[:, :, 0], knew) <= TOL and rel(vn[:, :, 0], vnew) <= TOL


def test_logits_match():
    r = np.random.default_rng(12)
    h = r.standard_normal((5, 64)).astype(np.float32)
    nw = (1 + 0.1 * r.standard_normal(64)).astype(np.float32)
    E = r.standard_normal((77, 64)).astype(np.float32)
    got = R.logits(h, nw, 1e-5, E, 0.0625)
    assert rel(got, O.logits(h, nw, 1e-5, E, 0.0625)) <= TOL
    one = R.logits(h, nw, 1e-5, E, 1.0)
    assert np.array_equal(got, one * np.float32(0.0625))   # the scale is the last fp32 multiply
