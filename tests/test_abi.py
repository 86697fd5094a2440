"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before anything is enqueued.

Only validation paths are exercised here: every call below fails its checks,
so no kernel is launched and no pointer is dereferenced (the fake device
addresses are never touched)."""
import ctypes
import os
import re

import pytest

from moe_denoise_forward_amd import dgmoe as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 40  # a 256-byte aligned address that is never dereferenced


def test_header_symbols_are_exported():
    hdr = open(os.path.join(ROOT, "include", "dgmoe.h")).read()
    declared = set(re.findall(r"\b(dgmoe_[a-z_]+)\s*\(", hdr))
    assert declared == set(dg.EXPORTS)
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert dg.dgmoe_abi_version() == dg.ABI_VERSION


def test_status_strings():
    for s in range(8):
        assert dg.dgmoe_status_str(s) not in ("", "unknown status")
    assert dg.dgmoe_status_str(99) == "unknown status"


def _dims(**kw):
    d = dict(D=256, E=16, k=4, I=128, Id=192, eps=1e-6)
    d.update(kw)
    return dg.make_dims(d["D"], d["E"], d["k"], d["I"], d["Id"], d["eps"])


def test_workspace_size_and_invalid_dims():
    assert dg.dgmoe_workspace_size(_dims(), 100) > 0
    assert dg.dgmoe_workspace_size(_dims(), 0) >= 0
    for bad in (dict(D=100), dict(D=0), dict(I=96), dict(Id=32), dict(E=0), dict(E=300),
                dict(k=0), dict(k=17, E=16), dict(k=33, E=64), dict(eps=float("nan")),
                dict(D=8256)):
        assert dg.dgmoe_workspace_size(_dims(**bad), 10) == 0, bad
    assert dg.dgmoe_workspace_size(_dims(), -1) == 0
    assert dg.dgmoe_workspace_size(_dims(), (1 << 20) + 1) == 0


def test_packed_bytes():
    assert dg.dgmoe_packed_bytes(10, 128, dg.DGMOE_Q4G64) == 640
    assert dg.dgmoe_packed_bytes(10, 128, dg.DGMOE_Q8G64) == 1280
    assert dg.dgmoe_packed_bytes(64, 128, dg.DGMOE_Q4G32) == 4096
    assert dg.dgmoe_packed_bytes(64, 128, dg.DGMOE_NVFP4) == 4096
    assert dg.dgmoe_packed_bytes(64, 128, dg.DGMOE_Q6G32) == 6144
    assert dg.dgmoe_packed_bytes(10, 100, dg.DGMOE_Q4G64) == 0
    assert dg.dgmoe_packed_bytes(10, 128, dg.DGMOE_BF16) == 0


def _mat(fmt, base):
    packed = fmt in (dg.DGMOE_Q4G64, dg.DGMOE_Q8G64, dg.DGMOE_Q4G32, dg.DGMOE_NVFP4, dg.DGMOE_Q6G32)
    return dg.dgmoe_matrix(fmt, base, base + 4096 if packed else None)


def _weights(router=dg.DGMOE_Q8G64, experts=dg.DGMOE_Q4G64, dense=dg.DGMOE_Q4G64, **override):
    w = dg.dgmoe_block_weights(
        _mat(router, FAKE), FAKE + 64, FAKE + 128, None,
        _mat(experts, FAKE + (1 << 20)), _mat(experts, FAKE + (2 << 20)),
        _mat(dense, FAKE + (3 << 20)), _mat(dense, FAKE + (4 << 20)),
        FAKE + 256, FAKE + 512, FAKE + 768, FAKE + 1024, FAKE + 1280, 0.5)
    for k, v in override.items():
        setattr(w, k, v)
    return w


def _block(dims=None, w=None, x=FAKE, x_dtype=dg.DGMOE_BF16, L=10, y=FAKE, y_dtype=dg.DGMOE_F32,
           ws=FAKE, ws_bytes=None):
    dims = dims or _dims()
    w = w or _weights()
    if ws_bytes is None:
        ws_bytes = dg.dgmoe_workspace_size(dims, L)
    return dg._lib.dgmoe_block_forward(ctypes.byref(dims), ctypes.byref(w), x, x_dtype, L, None,
                                       None, y, y_dtype, None, None, ws, ws_bytes, None)


def test_block_forward_validation():
    assert _block(dims=_dims(D=100)) == dg.DGMOE_ERR_BAD_DIMS
    assert _block(L=-3) == dg.DGMOE_ERR_BAD_DIMS
    assert _block(x=None) == dg.DGMOE_ERR_NULL_ARG
    assert _block(x=FAKE + 2) == dg.DGMOE_ERR_MISALIGNED
    assert _block(x_dtype=dg.DGMOE_F16) == dg.DGMOE_ERR_BAD_DTYPE
    assert _block(y=None) == dg.DGMOE_ERR_NULL_ARG
    assert _block(y_dtype=dg.DGMOE_Q4G64) == dg.DGMOE_ERR_BAD_DTYPE
    assert _block(ws=None) == dg.DGMOE_ERR_NULL_ARG
    assert _block(ws=FAKE + 64) == dg.DGMOE_ERR_MISALIGNED
    assert _block(ws_bytes=100) == dg.DGMOE_ERR_WORKSPACE
    # gate_up / down format mismatch
    w = _weights()
    w.expert_down = _mat(dg.DGMOE_BF16, FAKE + (2 << 20))
    assert _block(w=w) == dg.DGMOE_ERR_BAD_DTYPE
    # unsupported expert format
    assert _block(w=_weights(experts=dg.DGMOE_F32)) == dg.DGMOE_ERR_BAD_DTYPE
    # the dense MLP may take its own format, but its two matrices share one
    w = _weights(experts=dg.DGMOE_Q4G32, dense=dg.DGMOE_BF16)
    w.dense_down = _mat(dg.DGMOE_Q4G32, FAKE + (4 << 20))
    assert _block(w=w) == dg.DGMOE_ERR_BAD_DTYPE
    w = _weights(experts=dg.DGMOE_Q4G32, dense=dg.DGMOE_Q4G64)
    w.expert_down = _mat(dg.DGMOE_Q4G64, FAKE + (2 << 20))
    assert _block(w=w) == dg.DGMOE_ERR_BAD_DTYPE
    # 8-bit and f32 MLP weights are not MLP formats
    assert _block(w=_weights(dense=dg.DGMOE_F32)) == dg.DGMOE_ERR_BAD_DTYPE
    assert _block(w=_weights(experts=dg.DGMOE_Q8G64)) == dg.DGMOE_ERR_BAD_DTYPE
    # misaligned packed weight data or scales (64-byte rule)
    w = _weights()
    w.expert_gate_up = dg.dgmoe_matrix(dg.DGMOE_Q4G64, FAKE + (1 << 20) + 32, FAKE + 4096)
    assert _block(w=w) == dg.DGMOE_ERR_MISALIGNED
    w = _weights()
    w.expert_gate_up = dg.dgmoe_matrix(dg.DGMOE_Q4G64, FAKE + (1 << 20), FAKE + 4096 + 16)
    assert _block(w=w) == dg.DGMOE_ERR_MISALIGNED
    # missing scales of a packed matrix
    w = _weights()
    w.dense_down = dg.dgmoe_matrix(dg.DGMOE_Q4G64, FAKE + (4 << 20), None)
    assert _block(w=w) == dg.DGMOE_ERR_NULL_ARG
    # a q4 router is not a supported router format
    assert _block(w=_weights(router=dg.DGMOE_Q4G64)) == dg.DGMOE_ERR_BAD_DTYPE
    assert _block(w=_weights(router=dg.DGMOE_Q4G32)) == dg.DGMOE_ERR_BAD_DTYPE
    # an unknown format code
    assert _block(w=_weights(experts=8, dense=8)) == dg.DGMOE_ERR_BAD_DTYPE
    assert _block(w=_weights(router=dg.DGMOE_Q6G32)) == dg.DGMOE_ERR_BAD_DTYPE
    assert _block(w=_weights(router=dg.DGMOE_NVFP4)) == dg.DGMOE_ERR_BAD_DTYPE
    # missing norm weight
    assert _block(w=_weights(post_ff_norm=None)) == dg.DGMOE_ERR_NULL_ARG
    # L == 0 is a no-op that succeeds without touching anything
    assert _block(L=0, x=None, y=None, ws=None, ws_bytes=0) == dg.DGMOE_OK


def test_route_and_moe_ffn_validation():
    dims = _dims()
    w = _weights()
    n = dg.dgmoe_workspace_size(dims, 10)
    r = dg._lib.dgmoe_route(ctypes.byref(dims), ctypes.byref(w), FAKE, dg.DGMOE_BF16, 10, None,
                            FAKE, None, FAKE, n, None)
    assert r == dg.DGMOE_ERR_NULL_ARG
    r = dg._lib.dgmoe_route(ctypes.byref(dims), ctypes.byref(w), FAKE, dg.DGMOE_BF16, 10, FAKE + 2,
                            FAKE, None, FAKE, n, None)
    assert r == dg.DGMOE_ERR_MISALIGNED
    w2 = _weights(router=dg.DGMOE_F16)
    r = dg._lib.dgmoe_route(ctypes.byref(dims), ctypes.byref(w2), FAKE, dg.DGMOE_BF16, 10, FAKE,
                            FAKE, None, FAKE, n, None)
    assert r == dg.DGMOE_ERR_BAD_DTYPE
    r = dg._lib.dgmoe_moe_ffn(ctypes.byref(dims), ctypes.byref(w), FAKE, dg.DGMOE_BF16, 10, FAKE,
                              FAKE, None, FAKE, n, None)
    assert r == dg.DGMOE_ERR_NULL_ARG
    r = dg._lib.dgmoe_moe_ffn(ctypes.byref(dims), ctypes.byref(w), FAKE, dg.DGMOE_BF16, 10, FAKE,
                              FAKE, FAKE, FAKE, n - 1, None)
    assert r == dg.DGMOE_ERR_WORKSPACE


def test_pack_unpack_validation():
    lib = dg._lib
    Q4, Q8 = dg.DGMOE_Q4G64, dg.DGMOE_Q8G64
    assert lib.dgmoe_pack(FAKE, 16, 100, Q4, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_pack(FAKE, 4, 128, Q4, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS  # rows % 64
    assert lib.dgmoe_pack(FAKE, 48, 128, Q4, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_pack(FAKE, 16, 128, dg.DGMOE_BF16, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DTYPE
    assert lib.dgmoe_pack(None, 64, 128, Q4, FAKE, FAKE, None) == dg.DGMOE_ERR_NULL_ARG
    assert lib.dgmoe_pack(FAKE, 64, 128, Q4, FAKE + 32, FAKE, None) == dg.DGMOE_ERR_MISALIGNED
    assert lib.dgmoe_pack(FAKE, 0, 128, Q8, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_unpack(FAKE, FAKE, 16, 128, Q4, dg.DGMOE_BF16, FAKE, None) == dg.DGMOE_ERR_BAD_DTYPE
    assert lib.dgmoe_unpack(FAKE, FAKE, 64, 128, Q4, dg.DGMOE_F32, FAKE + 8, None) == dg.DGMOE_ERR_MISALIGNED
    assert lib.dgmoe_unpack(FAKE, FAKE, 5, 128, Q4, dg.DGMOE_F32, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS
    G32 = dg.DGMOE_Q4G32
    assert lib.dgmoe_pack(FAKE, 32, 128, G32, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS  # rows % 64
    assert lib.dgmoe_pack(FAKE, 64, 96, G32, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS  # cols % 64
    assert lib.dgmoe_pack(FAKE, 64, 128, G32, FAKE, FAKE + 16, None) == dg.DGMOE_ERR_MISALIGNED
    assert lib.dgmoe_unpack(FAKE, FAKE, 96, 128, G32, dg.DGMOE_F16, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_pack(FAKE, 64, 128, 8, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DTYPE
    assert lib.dgmoe_pack(FAKE, 96, 128, dg.DGMOE_Q6G32, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS
    F4 = dg.DGMOE_NVFP4
    assert lib.dgmoe_pack(FAKE, 32, 128, F4, FAKE, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS  # rows % 64
    assert lib.dgmoe_unpack(FAKE, FAKE, 64, 100, F4, dg.DGMOE_F32, FAKE, None) == dg.DGMOE_ERR_BAD_DIMS


def test_check_workspace_validation():
    # argument errors are reported before any HIP call
    flags = ctypes.c_uint32(0)
    lib = dg._lib
    assert lib.dgmoe_check_workspace(None, 10, FAKE, ctypes.byref(flags), None) == dg.DGMOE_ERR_NULL_ARG
    assert lib.dgmoe_check_workspace(ctypes.byref(_dims()), 10, None, ctypes.byref(flags), None) == dg.DGMOE_ERR_NULL_ARG
    assert lib.dgmoe_check_workspace(ctypes.byref(_dims()), 10, FAKE, None, None) == dg.DGMOE_ERR_NULL_ARG
    assert lib.dgmoe_check_workspace(ctypes.byref(_dims(D=100)), 10, FAKE, ctypes.byref(flags), None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_check_workspace(ctypes.byref(_dims()), 0, FAKE, ctypes.byref(flags), None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_check_workspace(ctypes.byref(_dims()), 10, FAKE + 64, ctypes.byref(flags), None) == dg.DGMOE_ERR_MISALIGNED


def test_hidden_limit_matches_header():
    # the header promises hidden up to 8192 (the front kernel stages router_scale
    # for 8192 inputs in LDS; the combine runs one thread per 8 columns)
    assert dg.dgmoe_workspace_size(_dims(D=8192), 4) > 0
    assert dg.dgmoe_workspace_size(_dims(D=8256), 4) == 0
    hdr = open(os.path.join(ROOT, "include", "dgmoe.h")).read()
    assert "hidden: a multiple of 64 in [64, 8192]" in hdr


# ------------------------------------------------------------------ head
def _hdims(**kw):
    d = dict(D=256, V=4160, Isc=192, eps=1e-6)
    d.update(kw)
    return dg.make_head_dims(d["D"], d["V"], d["Isc"], d["eps"])


def _hweights(embed=dg.DGMOE_Q4G64, **override):
    w = dg.dgmoe_head_weights(_mat(embed, FAKE + (1 << 20)), FAKE + 256,
                              _mat(dg.DGMOE_Q4G64, FAKE + (2 << 20)),
                              _mat(dg.DGMOE_Q4G64, FAKE + (3 << 20)), FAKE + 512)
    for k, v in override.items():
        setattr(w, k, v)
    return w


def test_head_workspace_size_and_invalid_dims():
    assert dg.dgmoe_head_workspace_size(_hdims(), 100) > 0
    for bad in (dict(D=100), dict(D=8256), dict(V=4100), dict(V=(1 << 20) + 64), dict(V=0),
                dict(Isc=96), dict(Isc=16448), dict(eps=float("inf")), dict(eps=-1.0)):
        assert dg.dgmoe_head_workspace_size(_hdims(**bad), 10) == 0, bad
    assert dg.dgmoe_head_workspace_size(_hdims(), -1) == 0
    assert dg.dgmoe_head_workspace_size(_hdims(), (1 << 20) + 1) == 0
    # the soft embedding's probabilities alone take 2 L V bytes
    assert dg.dgmoe_head_workspace_size(_hdims(), 100) >= 2 * 100 * 4160


def _tail(h=None, w=None, x=FAKE, x_dtype=dg.DGMOE_F32, L=10, T=0.6, H=FAKE, am=FAKE, lg=None,
          ws=FAKE, ws_bytes=None):
    h = h or _hdims()
    w = w or _hweights()
    if ws_bytes is None:
        ws_bytes = dg.dgmoe_head_workspace_size(h, L)
    return dg._lib.dgmoe_tail(ctypes.byref(h), ctypes.byref(w), x, x_dtype, L, T, H, am, None, None,
                              lg, ws, ws_bytes, None)


def test_tail_validation():
    assert _tail(h=_hdims(V=100)) == dg.DGMOE_ERR_BAD_DIMS
    assert _tail(T=0.0) == dg.DGMOE_ERR_BAD_DIMS
    assert _tail(T=float("nan")) == dg.DGMOE_ERR_BAD_DIMS
    assert _tail(T=-0.5) == dg.DGMOE_ERR_BAD_DIMS
    assert _tail(x_dtype=dg.DGMOE_F16) == dg.DGMOE_ERR_BAD_DTYPE
    assert _tail(w=_hweights(embed=dg.DGMOE_BF16)) == dg.DGMOE_ERR_BAD_DTYPE
    assert _tail(w=_hweights(final_norm=None)) == dg.DGMOE_ERR_NULL_ARG
    assert _tail(w=_hweights(final_norm=FAKE + 4)) == dg.DGMOE_ERR_MISALIGNED
    assert _tail(x=None) == dg.DGMOE_ERR_NULL_ARG
    assert _tail(H=None) == dg.DGMOE_ERR_NULL_ARG
    assert _tail(am=None) == dg.DGMOE_ERR_NULL_ARG
    assert _tail(x=FAKE + 8) == dg.DGMOE_ERR_MISALIGNED
    assert _tail(lg=FAKE + 4) == dg.DGMOE_ERR_MISALIGNED
    assert _tail(ws=None) == dg.DGMOE_ERR_NULL_ARG
    assert _tail(ws=FAKE + 128) == dg.DGMOE_ERR_MISALIGNED
    assert _tail(ws_bytes=1000) == dg.DGMOE_ERR_WORKSPACE
    w = _hweights()
    w.embed = dg.dgmoe_matrix(dg.DGMOE_Q4G64, FAKE + (1 << 20) + 32, FAKE + 4096)
    assert _tail(w=w) == dg.DGMOE_ERR_MISALIGNED
    assert _tail(L=0, x=None, H=None, am=None, ws=None, ws_bytes=0) == dg.DGMOE_OK


def test_soft_embed_and_sc_input_validation():
    lib, h, w = dg._lib, _hdims(), _hweights()
    n = dg.dgmoe_head_workspace_size(h, 10)
    assert lib.dgmoe_soft_embed(ctypes.byref(h), ctypes.byref(w), None, 10, FAKE, FAKE, n, None) == dg.DGMOE_ERR_NULL_ARG
    assert lib.dgmoe_soft_embed(ctypes.byref(h), ctypes.byref(w), FAKE + 4, 10, FAKE, FAKE, n, None) == dg.DGMOE_ERR_MISALIGNED
    assert lib.dgmoe_soft_embed(ctypes.byref(h), ctypes.byref(w), FAKE, 10, FAKE, FAKE, n - 1, None) == dg.DGMOE_ERR_WORKSPACE
    assert lib.dgmoe_sc_input(ctypes.byref(h), ctypes.byref(w), None, FAKE, 10, FAKE, FAKE, n, None) == dg.DGMOE_ERR_NULL_ARG
    assert lib.dgmoe_sc_input(ctypes.byref(h), ctypes.byref(w), FAKE + 2, FAKE, 10, FAKE, FAKE, n, None) == dg.DGMOE_ERR_MISALIGNED
    # the MLP weights are needed only with a signal
    w2 = _hweights(sc_pre_norm=None)
    assert lib.dgmoe_sc_input(ctypes.byref(h), ctypes.byref(w2), FAKE, FAKE, 10, FAKE, FAKE, n, None) == dg.DGMOE_ERR_NULL_ARG
    w3 = _hweights()
    w3.sc_down = _mat(dg.DGMOE_BF16, FAKE + (3 << 20))
    assert lib.dgmoe_sc_input(ctypes.byref(h), ctypes.byref(w3), FAKE, FAKE, 10, FAKE, FAKE, n, None) == dg.DGMOE_ERR_BAD_DTYPE
    assert lib.dgmoe_sc_input(ctypes.byref(h), ctypes.byref(w), FAKE, None, 0, None, None, 0, None) == dg.DGMOE_OK
    flags = ctypes.c_uint32(0)
    assert lib.dgmoe_head_check_workspace(ctypes.byref(h), 0, FAKE, ctypes.byref(flags), None) == dg.DGMOE_ERR_BAD_DIMS
    assert lib.dgmoe_head_check_workspace(ctypes.byref(h), 10, None, ctypes.byref(flags), None) == dg.DGMOE_ERR_NULL_ARG


# ------------------------------------------------------------------ denoise attention
def _adims(**kw):
    d = dict(H=16, Hkv=8, hd=256, window=1023, pairs=128, stride=128, theta=1e4, den=256.0, eps=1e-6)
    d.update(kw)
    return dg.make_attn_dims(d["H"], d["Hkv"], d["hd"], d["window"], d["pairs"], d["stride"],
                             d["theta"], d["den"], d["eps"])


def test_attn_workspace_size_and_invalid_dims():
    n = dg.dgmoe_attn_workspace_size(_adims(), 256, 4096)
    # prepared q / k / v in fp16 at least, plus the key-range partials
    assert n >= (16 + 2 * 8) * 256 * 256 * 2
    assert dg.dgmoe_attn_workspace_size(_adims(), 100, 0) > 0
    for bad in [dict(hd=96), dict(hd=1024), dict(H=12, Hkv=8), dict(Hkv=0), dict(window=-1),
                dict(pairs=129), dict(pairs=64, stride=32), dict(pairs=128, stride=129),
                dict(theta=0.0), dict(theta=float("inf")), dict(den=0.0), dict(eps=-1.0),
                dict(eps=float("nan"))]:
        assert dg.dgmoe_attn_workspace_size(_adims(**bad), 16, 16) == 0, bad
    assert dg.dgmoe_attn_workspace_size(_adims(), -1, 16) == 0
    assert dg.dgmoe_attn_workspace_size(_adims(), 16, -1) == 0
    assert dg.dgmoe_attn_workspace_size(_adims(), (1 << 20) + 1, 16) == 0
    # a partial rotation whose partner stride reaches the last dimension is valid
    assert dg.dgmoe_attn_workspace_size(_adims(hd=512, Hkv=2, pairs=64, stride=448), 16, 16) > 0


def _attn(a=None, q=FAKE, k=FAKE, v=FAKE, ind=None, L=16, wq=FAKE, wk=FAKE, kc=FAKE, vc=FAKE,
          rows=64, kv=32, out=FAKE, od=None, ws=FAKE, ws_bytes=None):
    a = a or _adims()
    ind = dg.DGMOE_BF16 if ind is None else ind
    od = dg.DGMOE_F32 if od is None else od
    if ws_bytes is None:
        ws_bytes = dg.dgmoe_attn_workspace_size(a, L, kv)
    return dg._lib.dgmoe_attn_denoise(ctypes.byref(a), q, k, v, ind, L, wq, wk, kc, vc, rows, kv,
                                      out, od, ws, ws_bytes, None)


def test_attn_validation():
    assert dg._lib.dgmoe_attn_denoise(None, FAKE, FAKE, FAKE, 1, 16, FAKE, FAKE, FAKE, FAKE, 64, 32,
                                      FAKE, 0, FAKE, 1 << 30, None) == dg.DGMOE_ERR_NULL_ARG
    assert _attn(a=_adims(hd=100)) == dg.DGMOE_ERR_BAD_DIMS
    assert _attn(kv=65, rows=64) == dg.DGMOE_ERR_BAD_DIMS            # kv_len past the cache
    assert _attn(kv=-1) == dg.DGMOE_ERR_BAD_DIMS
    assert _attn(L=-1) == dg.DGMOE_ERR_BAD_DIMS
    # the row tiles of a query group are a grid dimension of at most 65535
    assert _attn(a=_adims(H=16, Hkv=1), L=(65535 * 64) // 16 + 1, ws_bytes=1 << 40) == dg.DGMOE_ERR_BAD_DIMS
    assert _attn(ind=dg.DGMOE_F16) == dg.DGMOE_ERR_BAD_DTYPE
    assert _attn(od=dg.DGMOE_Q4G64) == dg.DGMOE_ERR_BAD_DTYPE
    for name in ("q", "k", "wq", "wk", "out", "ws"):
        assert _attn(**{name: None}) == dg.DGMOE_ERR_NULL_ARG, name
    assert _attn(kc=None) == dg.DGMOE_ERR_NULL_ARG
    assert _attn(vc=None) == dg.DGMOE_ERR_NULL_ARG
    assert _attn(q=FAKE + 2) == dg.DGMOE_ERR_MISALIGNED
    assert _attn(kc=FAKE + 8) == dg.DGMOE_ERR_MISALIGNED
    assert _attn(out=FAKE + 8) == dg.DGMOE_ERR_MISALIGNED
    assert _attn(ws=FAKE + 128) == dg.DGMOE_ERR_MISALIGNED
    assert _attn(ws_bytes=1000) == dg.DGMOE_ERR_WORKSPACE
    # no committed rows: the caches are not needed; L = 0 is a no-op
    assert _attn(kv=0, kc=None, vc=None, ws_bytes=100) == dg.DGMOE_ERR_WORKSPACE
    assert _attn(L=0, q=None, k=None, out=None, ws=None, ws_bytes=0) == dg.DGMOE_OK
