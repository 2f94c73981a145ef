"""The C-ABI library loads without a GPU, exports every entry point include/atlas.h
declares, and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

from swa_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    with open(os.path.join(ROOT, "include", "atlas.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"ATLAS_API\s+[\w\s\*]+?\b(atlas_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from swa_attention_amd import build
        build.build()
    return L.lib()


def test_every_declared_symbol_is_exported(lib):
    syms = header_symbols()
    assert len(syms) >= 15
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(L.exported_symbols())


def test_stream_read_validation(lib):
    def sr(buf=FAKE, n=1 << 20, sink=FAKE, blocks=512):
        return lib.atlas_stream_read(buf, n, sink, blocks, None)
    assert sr(buf=None) == L.ATLAS_ERR_INVALID_ARG
    assert sr(sink=None) == L.ATLAS_ERR_INVALID_ARG
    assert sr(n=0) == L.ATLAS_ERR_INVALID_ARG
    assert sr(n=100) == L.ATLAS_ERR_INVALID_ARG           # not a multiple of 16
    assert sr(buf=FAKE + 8) == L.ATLAS_ERR_INVALID_ARG    # misaligned
    assert sr(blocks=0) == L.ATLAS_ERR_INVALID_ARG
    assert sr(blocks=70000) == L.ATLAS_ERR_INVALID_ARG
    assert b"blocks" in lib.atlas_last_error()


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.atlas_version()
    assert lib.atlas_status_string(0) == b"ok"
    assert lib.atlas_status_string(3) == b"workspace too small"


FAKE = 0x10000   # a non-null, 16-byte aligned address; never dereferenced by validation


def w4(N=64, K=256, group=128, qweight=FAKE, scales=FAKE, zeros=FAKE, scale_dtype=0):
    return L.atlas_w4(qweight, scales, zeros, N, K, group, scale_dtype)


def test_w4_gemv_validation(lib):
    def gemv(W, ws_bytes=1 << 20, ws=FAKE, x=FAKE, y=FAKE):
        return lib.atlas_w4_gemv(ctypes.byref(W) if W is not None else None, x, y, ws, ws_bytes, None)
    assert gemv(None) == L.ATLAS_ERR_INVALID_ARG
    assert gemv(w4(qweight=None)) == L.ATLAS_ERR_INVALID_ARG
    assert gemv(w4(K=100)) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert gemv(w4(group=48)) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert gemv(w4(scale_dtype=3)) == L.ATLAS_ERR_INVALID_ARG
    assert gemv(w4(qweight=FAKE + 4)) == L.ATLAS_ERR_INVALID_ARG
    assert gemv(w4(), x=None) == L.ATLAS_ERR_INVALID_ARG
    assert gemv(w4(), ws=None) == L.ATLAS_ERR_INVALID_ARG
    need = lib.atlas_w4_gemv_workspace_bytes(ctypes.byref(w4()))
    assert need > 0
    assert gemv(w4(), ws_bytes=need - 1) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in lib.atlas_last_error()


def test_w4_gemv_batch_validation(lib):
    def gb(W, B=4, ws_bytes=1 << 24, ws=FAKE, x=FAKE, y=FAKE):
        return lib.atlas_w4_gemv_batch(ctypes.byref(W) if W is not None else None, x, B, y, ws, ws_bytes, None)
    assert gb(None) == L.ATLAS_ERR_INVALID_ARG
    assert gb(w4(), B=0) == L.ATLAS_ERR_INVALID_ARG
    assert gb(w4(), B=9) == L.ATLAS_ERR_INVALID_ARG
    assert gb(w4(K=96)) == L.ATLAS_ERR_UNSUPPORTED_SHAPE            # K % 64 != 0
    assert gb(w4(group=64)) == L.ATLAS_ERR_UNSUPPORTED_SHAPE        # group not a multiple of 128
    assert gb(w4(group=32)) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert gb(w4(), x=None) == L.ATLAS_ERR_INVALID_ARG
    assert gb(w4(), ws=None) == L.ATLAS_ERR_INVALID_ARG
    assert lib.atlas_w4_gemv_batch_workspace_bytes(ctypes.byref(w4(group=64)), 4) == 0
    assert lib.atlas_w4_gemv_batch_workspace_bytes(ctypes.byref(w4()), 9) == 0
    for N, K, B in ((7168, 5120, 8), (5120, 27648, 8), (640, 1728, 3), (64, 256, 1)):
        need = lib.atlas_w4_gemv_batch_workspace_bytes(ctypes.byref(w4(N, K)), B)
        assert need > 0
        assert gb(w4(N, K), B=B, ws_bytes=need - 1) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL


def test_workspace_sizes_are_positive_for_real_shapes(lib):
    for N, K in ((7168, 5120), (5120, 5120), (27648, 5120), (5120, 27648), (896, 640), (640, 1728)):
        assert lib.atlas_w4_gemv_workspace_bytes(ctypes.byref(w4(N, K))) > 0
    assert lib.atlas_gqa_decode_workspace_bytes(40, 8, 128, 16385) > 0
    assert lib.atlas_gqa_decode_workspace_bytes(40, 8, 64, 16385) == 0


def test_attention_and_norm_validation(lib):
    g = lib.atlas_gqa_decode
    ok_ws = lib.atlas_gqa_decode_workspace_bytes(40, 8, 128, 4097)
    assert g(FAKE, FAKE, FAKE, 40, 8, 64, 4097, FAKE, 0, 0.1, FAKE, FAKE, ok_ws, None) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert g(FAKE, FAKE, FAKE, 40, 7, 128, 4097, FAKE, 0, 0.1, FAKE, FAKE, ok_ws, None) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert g(FAKE, FAKE, FAKE, 40, 8, 128, 4097, FAKE, -1, 0.1, FAKE, FAKE, ok_ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, 40, 8, 128, 4097, None, 0, 0.1, FAKE, FAKE, ok_ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, 40, 8, 128, 4097, FAKE, 0, 0.1, FAKE, FAKE, 16, None) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL
    n = lib.atlas_rmsnorm_residual
    assert n(None, FAKE, None, FAKE, 10, 1e-6, None) == L.ATLAS_ERR_INVALID_ARG
    assert n(FAKE, FAKE, None, FAKE, 0, 1e-6, None) == L.ATLAS_ERR_INVALID_ARG
    assert n(FAKE, FAKE, None, FAKE, 20000, 1e-6, None) == L.ATLAS_ERR_INVALID_ARG
    rope = L.atlas_rope(500000.0, 1.0, 8192.0, 32.0, 1.0, 0.0)
    q = lib.atlas_qk_norm_rope
    assert q(FAKE, FAKE, FAKE, FAKE, 40, 8, 127, FAKE, ctypes.byref(rope), 1e-6, None) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert q(FAKE, FAKE, FAKE, FAKE, 40, 8, 128, None, ctypes.byref(rope), 1e-6, None) == L.ATLAS_ERR_INVALID_ARG


def test_kv_layout_attention_validation(lib):
    g = lib.atlas_gqa_decode_kv
    ws = lib.atlas_gqa_decode_workspace_bytes(40, 8, 128, 4096)

    def call(layout, D=128, window=4096, ws_bytes=ws, pos=FAKE):
        lay = None if layout is None else ctypes.byref(L.atlas_kv_layout(*layout))
        return g(FAKE, FAKE, FAKE, lay, 40, 8, D, pos, window, 0.1, FAKE, FAKE, ws_bytes, None)
    assert call(None) == L.ATLAS_ERR_INVALID_ARG
    assert call((2, 1, 4096)) == L.ATLAS_ERR_INVALID_ARG              # element type
    assert call((1, 1, 4096), window=0) == L.ATLAS_ERR_INVALID_ARG     # a ring needs a window
    assert call((1, 1, 4096), window=4097) == L.ATLAS_ERR_INVALID_ARG  # ... that fits its slots
    assert call((1, 1, 0)) == L.ATLAS_ERR_INVALID_ARG
    assert call((1, 1, 4096), D=64) == L.ATLAS_ERR_UNSUPPORTED_SHAPE
    assert call((1, 1, 4096), ws_bytes=16) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL
    assert call((1, 1, 4096), pos=None) == L.ATLAS_ERR_INVALID_ARG


def test_sample_validation(lib):
    ws = lib.atlas_sample_workspace_bytes(100278)
    assert ws > 100278 * 4
    assert lib.atlas_sample_workspace_bytes(0) == 0
    s = lib.atlas_sample
    assert s(None, 100278, 0.6, 0.95, FAKE, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert s(FAKE, 0, 0.6, 0.95, FAKE, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert s(FAKE, 100278, -1.0, 0.95, FAKE, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert s(FAKE, 100278, float("nan"), 0.95, FAKE, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert s(FAKE, 100278, 0.6, 0.0, FAKE, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert s(FAKE, 100278, 0.6, 1.5, FAKE, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG
    assert s(FAKE, 100278, 0.6, 0.95, None, FAKE, FAKE, ws, None) == L.ATLAS_ERR_INVALID_ARG   # needs u
    assert s(FAKE, 100278, 0.6, 0.95, FAKE, FAKE, FAKE, ws - 1, None) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL


def _fake_model(n_layers=2, **over):
    m = dict(d=640, hq=5, hkv=1, hd=128, dff=1728)
    m.update(over)
    nqkv = (m["hq"] + 2 * m["hkv"]) * m["hd"]

    def lay(t=0, qkv_K=None):
        return L.atlas_layer(w4(nqkv, qkv_K or m["d"]), w4(m["d"], m["hq"] * m["hd"]), w4(m["dff"], m["d"]),
                             w4(m["dff"], m["d"]), w4(m["d"], m["dff"]), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, t)
    layers = (L.atlas_layer * n_layers)(*[lay(over.get("type", 0), over.get("qkv_K")) for _ in range(n_layers)])
    rope = L.atlas_rope(500000.0, 1.0, 8192.0, 32.0, 1.0, 0.0)
    mm = L.atlas_model(m["d"], m["hq"], m["hkv"], m["hd"], m["dff"], n_layers, 64, 1000, 1e-6, 300, rope, rope,
                       ctypes.cast(layers, ctypes.POINTER(L.atlas_layer)), FAKE, FAKE, FAKE)
    return mm, layers


def test_decode_step_noalloc_validation(lib):
    """The no-allocation decode step checks its arguments like atlas_decode_step and
    rejects a model whose workspace exceeds its fixed scratch area before touching
    the device."""
    mm, keep = _fake_model()
    step = lib.atlas_decode_step_noalloc
    assert step(None, FAKE, None, FAKE, None, None, None, None, None) == L.ATLAS_ERR_INVALID_ARG
    assert step(ctypes.byref(mm), None, None, FAKE, None, None, None, None, None) == L.ATLAS_ERR_INVALID_ARG
    assert step(ctypes.byref(mm), FAKE, None, None, None, None, None, None, None) == L.ATLAS_ERR_INVALID_ARG
    bad, keep2 = _fake_model(type=2)
    assert step(ctypes.byref(bad), FAKE, None, FAKE, None, None, None, None, None) == L.ATLAS_ERR_INVALID_ARG
    big, keep3 = _fake_model()
    big.vocab = 2_000_000                                  # logits alone: 8 MB of workspace
    need = lib.atlas_decode_workspace_bytes(ctypes.byref(big))
    assert need > 4 << 20
    assert step(ctypes.byref(big), FAKE, None, FAKE, None, FAKE, FAKE, None, None) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in lib.atlas_last_error()
    assert lib.atlas_decode_workspace_bytes(ctypes.byref(mm)) <= 4 << 20


def test_decode_step_validation(lib):
    mm, keep = _fake_model()
    need = lib.atlas_decode_workspace_bytes(ctypes.byref(mm))
    assert need > 0
    step = lib.atlas_decode_step
    assert step(None, FAKE, None, FAKE, None, None, None, FAKE, need, None) == L.ATLAS_ERR_INVALID_ARG
    assert step(ctypes.byref(mm), None, None, FAKE, None, None, None, FAKE, need, None) == L.ATLAS_ERR_INVALID_ARG
    assert step(ctypes.byref(mm), FAKE, None, None, None, None, None, FAKE, need, None) == L.ATLAS_ERR_INVALID_ARG
    assert step(ctypes.byref(mm), FAKE, None, FAKE, None, None, None, FAKE, need - 1, None) == \
        L.ATLAS_ERR_WORKSPACE_TOO_SMALL
    bad, keep2 = _fake_model(type=2)
    assert step(ctypes.byref(bad), FAKE, None, FAKE, None, None, None, FAKE, need, None) == L.ATLAS_ERR_INVALID_ARG
    bad, keep3 = _fake_model(qkv_K=1280)
    assert step(ctypes.byref(bad), FAKE, None, FAKE, None, None, None, FAKE, need, None) == \
        L.ATLAS_ERR_UNSUPPORTED_SHAPE
    bad, keep4 = _fake_model(hd=64)
    assert lib.atlas_decode_workspace_bytes(ctypes.byref(bad)) == 0
    wide, keep5 = _fake_model(d=6176, hq=1, hkv=1)          # the GEMV input vectors hold d <= 6144
    assert step(ctypes.byref(wide), FAKE, None, FAKE, None, None, None, FAKE, need, None) == \
        L.ATLAS_ERR_UNSUPPORTED_SHAPE
    kvbad, keep6 = _fake_model()
    kvbad.kv_dtype = 2
    assert step(ctypes.byref(kvbad), FAKE, None, FAKE, None, None, None, FAKE, need, None) == L.ATLAS_ERR_INVALID_ARG
    ringbad, keep7 = _fake_model()
    ringbad.swa_ring, ringbad.window = 1, 0
    assert step(ctypes.byref(ringbad), FAKE, None, FAKE, None, None, None, FAKE, need, None) == \
        L.ATLAS_ERR_INVALID_ARG
    bat = lib.atlas_decode_batch
    bneed = lib.atlas_decode_batch_workspace_bytes(ctypes.byref(mm), 4)
    assert bneed > 0
    assert lib.atlas_decode_batch_workspace_bytes(ctypes.byref(mm), 0) == 0
    assert lib.atlas_decode_batch_workspace_bytes(ctypes.byref(mm), 17) == 0
    assert bat(ctypes.byref(mm), FAKE, FAKE, 0, None, None, None, FAKE, bneed, None) == L.ATLAS_ERR_INVALID_ARG
    assert bat(ctypes.byref(mm), None, FAKE, 4, None, None, None, FAKE, bneed, None) == L.ATLAS_ERR_INVALID_ARG
    assert bat(ctypes.byref(mm), FAKE, None, 4, None, None, None, FAKE, bneed, None) == L.ATLAS_ERR_INVALID_ARG
    assert bat(ctypes.byref(mm), FAKE, FAKE, 4, None, None, None, FAKE, bneed - 1, None) == \
        L.ATLAS_ERR_WORKSPACE_TOO_SMALL
    pre = lib.atlas_prefill
    pneed = lib.atlas_prefill_workspace_bytes(ctypes.byref(mm), 8)
    bf, keep8 = _fake_model()
    bf.kv_dtype = 1
    assert 0 < lib.atlas_prefill_workspace_bytes(ctypes.byref(bf), 8) < pneed   # half-size prompt KV buffers
    assert pneed > 0
    assert pre(ctypes.byref(mm), FAKE, 8, 295, None, None, FAKE, pneed, None) == L.ATLAS_ERR_INVALID_ARG
    assert pre(ctypes.byref(mm), FAKE, 0, 0, None, None, FAKE, pneed, None) == L.ATLAS_ERR_INVALID_ARG
    assert pre(ctypes.byref(mm), FAKE, 8, 0, None, None, FAKE, pneed - 1, None) == L.ATLAS_ERR_WORKSPACE_TOO_SMALL
