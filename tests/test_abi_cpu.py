"""The C-ABI library loads, exports every symbol include/compass.h declares, and its
host-side argument checks return the documented codes (no GPU needed: every
failing call here is rejected before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "compass.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(compass_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def b():
    from cohere2_block_mrope_amd import binding
    return binding


def test_header_symbols_exported(b):
    lib = ctypes.CDLL(b.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in compass.h but not exported"
    assert set(names) == set(b.EXPORTED)


def compass_shape(b, **kw):
    args = dict(hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, intermediate=8192,
                kind=b.COMPASS_SLIDING, window=1024, mrope_section=(24, 20, 20), rope_theta=50000.0,
                ln_eps=1e-5, dtype=b.COMPASS_BF16)
    args.update(kw)
    return b.make_desc(**args)


def test_workspace_sizes(b):
    d = compass_shape(b)
    T, D, qd, K2 = 4096, 2048, 2048, 10240
    need = 2 * (T * D + T * qd + 2 * 4 * 4096 * 128 + T * K2)
    got = b.compass_workspace_size(d, 1, 4096, 0, 0)
    assert need <= got <= need + 8 * 256
    assert b.compass_workspace_size(d, 64, 1, 8200, 1) > 0
    assert b.compass_workspace_size(compass_shape(b, head_dim=96), 1, 16, 0, 0) == 0
    assert b._lib.compass_workspace_size(None, 1, 1, 0, 0) == 0
    assert b.compass_logits_workspace_size(4096, 2048, b.COMPASS_BF16) == 4096 * 2048 * 2
    assert b.compass_logits_workspace_size(0, 2048, 1) == 0


class FakePtr:
    """Stands in for a tensor: only data_ptr() is read by the binding on these paths."""
    def __init__(self, p, shape=(1, 16, 2048), n=1 << 40, esz=1):
        self.p, self.shape, self.n, self.esz = p, shape, n, esz

    def data_ptr(self):
        return self.p

    def numel(self):
        return self.n

    def element_size(self):
        return self.esz


def weights(b, p=0x10000):
    return b.make_weights({k: FakePtr(p + 0x1000 * i) for i, k in enumerate(
        ["ln_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"])})


CASES = [
    ("head_dim 96", dict(head_dim=96), "UNSUPPORTED"),
    ("heads not grouped", dict(n_q_heads=6), "INVALID"),
    ("group of 16", dict(n_q_heads=64), "UNSUPPORTED"),
    ("hidden not /64", dict(hidden=2000), "UNSUPPORTED"),
    ("section sum", dict(mrope_section=(24, 20, 21)), "INVALID"),
    ("section not interleavable", dict(mrope_section=(4, 30, 30)), "INVALID"),
    ("window 0", dict(window=0), "INVALID"),
    ("dtype 7", dict(dtype=7), "UNSUPPORTED"),
    ("kind 2", dict(kind=2), "INVALID"),
    ("eps nan", dict(ln_eps=float("nan")), "INVALID"),
    ("odd head mix", dict(n_q_heads=3, n_kv_heads=1, head_dim=64), "UNSUPPORTED"),
    ("rope layout 2", dict(rope_layout=2), "INVALID"),
    ("ln_fuse 2", dict(ln_fuse=2), "INVALID"),
]


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_descriptor_rejected_before_launch(b, name, kw, code):
    d = compass_shape(b, **kw)
    x = FakePtr(0x100000)
    with pytest.raises(b.CompassError) as e:
        b.compass_layer_prefill(d, weights(b), x, FakePtr(0x200000), None, None, None, FakePtr(0x300000),
                                FakePtr(0x400000), stream=0)
    assert e.value.code == getattr(b, "COMPASS_E_" + code)
    assert b.compass_last_error()


def test_argument_errors(b):
    d = compass_shape(b)
    x, out, ws = FakePtr(0x100000), FakePtr(0x300000), FakePtr(0x400000)
    pos = FakePtr(0x200000)
    call = lambda **k: b.compass_layer_prefill(d, k.get("w", weights(b)), k.get("x", x), k.get("pos", pos),
                                               k.get("kv"), None, None, k.get("out", out), k.get("ws", ws), stream=0)
    with pytest.raises(b.CompassError) as e:
        call(pos=None)
    assert e.value.code == b.COMPASS_E_INVALID
    with pytest.raises(b.CompassError) as e:
        call(x=FakePtr(0x100008))
    assert e.value.code == b.COMPASS_E_ALIGN
    with pytest.raises(b.CompassError) as e:
        call(w=weights(b, 0x10004))
    assert e.value.code == b.COMPASS_E_ALIGN
    with pytest.raises(b.CompassError) as e:
        call(ws=FakePtr(0x400000, n=1024))
    assert e.value.code == b.COMPASS_E_WORKSPACE
    with pytest.raises(b.CompassError) as e:
        call(out=FakePtr(0x100000 + 4096))  # partial overlap with x
    assert e.value.code == b.COMPASS_E_INVALID
    kv = b.compass_kv()
    kv.k, kv.v, kv.capacity = 0x500000, 0x600000, 8
    with pytest.raises(b.CompassError) as e:
        call(kv=kv)  # capacity 8 < L = 16
    assert e.value.code == b.COMPASS_E_INVALID
    kv.capacity = 1 << 23  # 2^23 rows x 128 x 2 bytes = a 2 GiB (row, kv head) slice
    with pytest.raises(b.CompassError) as e:
        call(kv=kv)
    assert e.value.code == b.COMPASS_E_UNSUPPORTED


def test_decode_and_logits_argument_errors(b):
    d = compass_shape(b)
    x = FakePtr(0x100000, shape=(4, 2048))
    with pytest.raises(b.CompassError) as e:
        b.compass_layer_decode(d, weights(b), x, FakePtr(0x200000), b.compass_kv(), FakePtr(0x300000),
                               FakePtr(0x400000), stream=0)
    assert e.value.code == b.COMPASS_E_INVALID
    h = FakePtr(0x100000, shape=(16, 2048))
    emb = FakePtr(0x800000, shape=(1000, 2048))
    with pytest.raises(b.CompassError) as e:
        b.compass_logits(h, FakePtr(0x200000), 1e-5, emb, 0.25, FakePtr(0x300000), FakePtr(0x400000, n=16), 1,
                         stream=0)
    assert e.value.code == b.COMPASS_E_WORKSPACE
    h2 = FakePtr(0x100000, shape=(16, 2000))
    with pytest.raises(b.CompassError) as e:
        b.compass_logits(h2, FakePtr(0x200000), 1e-5, emb, 0.25, FakePtr(0x300000), FakePtr(0x400000), 1, stream=0)
    assert e.value.code == b.COMPASS_E_UNSUPPORTED


def test_positions_argument_errors(b):
    tok = FakePtr(0x100000, shape=(2, 0))
    with pytest.raises(b.CompassError) as e:
        b.compass_mrope_positions(tok, 255031, FakePtr(0x1000), FakePtr(0x2000), 2, FakePtr(0x3000),
                                  FakePtr(0x4000), FakePtr(0x5000), stream=0)
    assert e.value.code == b.COMPASS_E_INVALID
    tok = FakePtr(0x100000, shape=(2, 5))
    with pytest.raises(b.CompassError) as e:
        b.compass_mrope_positions(tok, 255031, FakePtr(0x1000), FakePtr(0x2000), 0, FakePtr(0x3000),
                                  FakePtr(0x4000), FakePtr(0x5000), stream=0)
    assert e.value.code == b.COMPASS_E_INVALID


def test_version(b):
    assert "gfx950" in b.compass_version()


def test_chunk_argument_errors(b):
    """compass_layer_prefill_chunk needs a cache with lens; the rest is checked as in prefill."""
    d = compass_shape(b)
    x, out, ws = FakePtr(0x100000), FakePtr(0x300000), FakePtr(0x400000)
    kv = b.compass_kv()
    kv.k, kv.v, kv.capacity = 0x500000, 0x600000, 64
    with pytest.raises(b.CompassError) as e:  # no lens
        b.compass_layer_prefill_chunk(d, weights(b), x, FakePtr(0x200000), kv, None, None, out, ws, stream=0)
    assert e.value.code == b.COMPASS_E_INVALID
    kv.lens = 0x700000
    kv.capacity = 8
    with pytest.raises(b.CompassError) as e:  # capacity 8 < L = 16
        b.compass_layer_prefill_chunk(d, weights(b), x, FakePtr(0x200000), kv, None, None, out, ws, stream=0)
    assert e.value.code == b.COMPASS_E_INVALID


def test_front_end_argument_errors(b):
    """compass_embed / compass_decode_positions / compass_logits_argmax reject bad arguments
    on the host with the documented codes."""
    L = b._lib
    # embed: D not a multiple of 8, NULL table, image pointers missing, misaligned h, h over embed
    assert L.compass_embed(4, 12, 100, 1, 0x1000, 0x2000, None, None, 0, 0x3000, None, None) == b.COMPASS_E_UNSUPPORTED
    assert L.compass_embed(4, 64, 100, 1, 0x1000, None, None, None, 0, 0x3000, None, None) == b.COMPASS_E_INVALID
    assert L.compass_embed(4, 64, 100, 1, 0x1000, 0x2000, None, None, 3, 0x3000, None, None) == b.COMPASS_E_INVALID
    assert L.compass_embed(4, 64, 100, 1, 0x1000, 0x2000, None, None, 0, 0x3008, None, None) == b.COMPASS_E_ALIGN
    assert L.compass_embed(4, 64, 100, 1, 0x1000, 0x100000, None, None, 0, 0x100000 + 1024, None,
                           None) == b.COMPASS_E_INVALID
    assert L.compass_embed(0, 64, 100, 1, 0x1000, 0x2000, None, None, 0, 0x3000, None, None) == b.COMPASS_E_INVALID
    assert L.compass_embed(4, 64, 100, 5, 0x1000, 0x2000, None, None, 0, 0x3000, None, None) == b.COMPASS_E_UNSUPPORTED
    # decode positions: B < 1, advance < 0, NULL lens, pos over lens
    assert L.compass_decode_positions(0, 0x1000, None, 0, 0x2000, None) == b.COMPASS_E_INVALID
    assert L.compass_decode_positions(4, 0x1000, None, -1, 0x2000, None) == b.COMPASS_E_INVALID
    assert L.compass_decode_positions(4, None, None, 0, 0x2000, None) == b.COMPASS_E_INVALID
    assert L.compass_decode_positions(4, 0x1000, None, 0, 0x1008, None) == b.COMPASS_E_INVALID
    # logits argmax
    # bf16: LayerNorm rows, then (value, id) partials of the 2000 128-column spans per row
    assert b.compass_logits_argmax_workspace_size(64, 2048, 256000, 1) == 64 * 2048 * 2 + 2 * 64 * 2000 * 4
    # fp32: LayerNorm rows, the logits, then the winners of 4096-column chunks
    assert b.compass_logits_argmax_workspace_size(64, 2048, 256000, 0) == \
        64 * 2048 * 4 + 64 * 256000 * 4 + 2 * 256 * 63
    assert b.compass_logits_argmax_workspace_size(64, 2048, 256000, 9) == 0
    ws = 0x10000000
    need = b.compass_logits_argmax_workspace_size(8, 2048, 1000, 1)

    def am(R=8, D=2048, V=1000, dt=1, h=0x100000, ldh=0, nw=0x200000, emb=0x400000, tok=0x300000,
           w=ws, n=need):
        return L.compass_logits_argmax(R, D, V, dt, h, ldh, nw, 1e-5, emb, 0.0625, tok, None, w, n, None)

    assert am(D=2000) == b.COMPASS_E_UNSUPPORTED
    assert am(ldh=1000) == b.COMPASS_E_INVALID          # ldh < D
    assert am(ldh=2052) == b.COMPASS_E_ALIGN            # rows not 16-byte aligned
    assert am(tok=None) == b.COMPASS_E_INVALID
    assert am(n=need - 1) == b.COMPASS_E_WORKSPACE
    assert am(w=ws + 16) == b.COMPASS_E_ALIGN
    assert am(dt=3) == b.COMPASS_E_UNSUPPORTED
    assert "ldh" in (am(ldh=1000) and b.compass_last_error())
    assert am(R=70000, n=1 << 40) == b.COMPASS_E_UNSUPPORTED  # R above the grid limit
    # pre-normalized rows (norm_w NULL): the GEMM reads h with 32-bit offsets
    assert am(nw=None, ldh=1 << 29) == b.COMPASS_E_UNSUPPORTED
    assert am(nw=None, h=None) == b.COMPASS_E_INVALID


def test_q4_decode_argument_errors(b):
    """compass_layer_decode_q4: bf16 only, every matrix pointer set, codes 16-byte aligned."""
    def wq4(p=0x10000, bad=None, misalign=None):
        w = b.compass_layer_weights_q4()
        w.ln_w = p
        for i, (name, _) in enumerate(b.compass_layer_weights_q4._fields_[1:]):
            base = p + 0x100000 * (i + 1)
            m = b.compass_q4_matrix(base, base + 0x40000, base + 0x80000)
            if name == bad:
                m.scales = None
            if name == misalign:
                m.q = base + 8
            setattr(w, name, m)
        return w
    kv = b.compass_kv()
    kv.k, kv.v, kv.capacity, kv.lens = 0x5000000, 0x6000000, 64, 0x7000000
    x, pos, out, ws = FakePtr(0x100000, shape=(4, 2048)), FakePtr(0x200000), FakePtr(0x300000), FakePtr(0x400000)
    for d, w, code in [(compass_shape(b, dtype=b.COMPASS_F32), wq4(), b.COMPASS_E_UNSUPPORTED),
                       (compass_shape(b), wq4(bad="w_up"), b.COMPASS_E_INVALID),
                       (compass_shape(b), wq4(misalign="wo"), b.COMPASS_E_ALIGN)]:
        with pytest.raises(b.CompassError) as e:
            b.compass_layer_decode_q4(d, w, x, pos, kv, out, ws, stream=0)
        assert e.value.code == code
    with pytest.raises(b.CompassError) as e:  # workspace too small
        b.compass_layer_decode_q4(compass_shape(b), wq4(), x, pos, kv, out, FakePtr(0x400000, n=64), stream=0)
    assert e.value.code == b.COMPASS_E_WORKSPACE


def test_noalloc_decode_checks_before_any_launch(b):
    """The no-allocation decode validates like compass_layer_decode and rejects a step whose
    workspace exceeds the scratch, all before any HIP call."""
    d = compass_shape(b, kind=b.COMPASS_FULL, window=0)
    x = FakePtr(0x100000, shape=(64, 2048))
    kv = b.compass_kv()
    kv.k, kv.v, kv.lens, kv.capacity = 0x500000, 0x600000, 0x700000, 1 << 16
    assert b.compass_workspace_size(d, 64, 1, 1 << 16, 1) > b.COMPASS_NOALLOC_SCRATCH_BYTES
    with pytest.raises(b.CompassError) as e:
        b.compass_layer_decode_noalloc(d, weights(b), x, None, kv, FakePtr(0x300000), stream=0)
    assert e.value.code == b.COMPASS_E_WORKSPACE and "no-allocation maximum" in b.compass_last_error()
    with pytest.raises(b.CompassError) as e:
        b.compass_layer_decode_noalloc(d, weights(b, 0x10004), x, None, kv, FakePtr(0x300000), stream=0)
    assert e.value.code == b.COMPASS_E_ALIGN
    with pytest.raises(b.CompassError) as e:
        b.compass_layer_decode_noalloc(d, weights(b), x, None, b.compass_kv(), FakePtr(0x300000), stream=0)
    assert e.value.code == b.COMPASS_E_INVALID


def test_chained_decode_checks(b):
    """LayerNorm outputs are handed between bf16 layers only, 16-byte aligned, never over x or
    out, out_norm needs the next layer's weight, and the chained call validates like
    compass_layer_decode (all rejected before any HIP call)."""
    kv = b.compass_kv()
    kv.k, kv.v, kv.capacity, kv.lens = 0x5000000, 0x6000000, 64, 0x7000000
    x, pos, out, ws = FakePtr(0x100000, shape=(4, 2048)), FakePtr(0x200000), FakePtr(0x300000), FakePtr(0x400000)
    nrm, lnw = FakePtr(0x800000), FakePtr(0x900000)
    f32 = compass_shape(b, dtype=b.COMPASS_F32)
    for d, xn, nw, on, code in [(f32, nrm, None, None, b.COMPASS_E_UNSUPPORTED),
                                (f32, None, lnw, nrm, b.COMPASS_E_UNSUPPORTED),
                                (compass_shape(b), None, None, nrm, b.COMPASS_E_INVALID),
                                (compass_shape(b), FakePtr(0x800008), None, None, b.COMPASS_E_ALIGN),
                                (compass_shape(b), None, lnw, FakePtr(0x800008), b.COMPASS_E_ALIGN),
                                (compass_shape(b), None, FakePtr(0x900008), nrm, b.COMPASS_E_ALIGN),
                                (compass_shape(b), None, lnw, FakePtr(0x100000 + 4096), b.COMPASS_E_INVALID),
                                (compass_shape(b), None, lnw, FakePtr(0x300000 - 4096), b.COMPASS_E_INVALID)]:
        with pytest.raises(b.CompassError) as e:
            b.compass_layer_decode_chained(d, weights(b), x, xn, pos, kv, out, nw, 1e-5, on, ws, stream=0)
        assert e.value.code == code, (xn, nw, on)
    with pytest.raises(b.CompassError) as e:  # workspace too small
        b.compass_layer_decode_chained(compass_shape(b), weights(b), x, nrm, pos, kv, out, lnw, 1e-5, nrm,
                                       FakePtr(0x400000, n=64), stream=0)
    assert e.value.code == b.COMPASS_E_WORKSPACE
    with pytest.raises(b.CompassError) as e:  # no kv
        b.compass_layer_decode_chained(compass_shape(b), weights(b), x, nrm, pos, b.compass_kv(), out, lnw, 1e-5,
                                       nrm, ws, stream=0)
    assert e.value.code == b.COMPASS_E_INVALID
