"""The C-ABI library loads and exports every function include/td.h declares
(no GPU needed: nothing is called that touches a device)."""
import ctypes
import os
import re

import pytest

from decode_persistent_megakernel_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "td.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(td_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("td_create", "td_decode_step", "td_destroy", "td_status", "td_strerror", "td_token_ptr"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(_lib.SO_PATH):
        pytest.fail("libtd.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(_lib.SO_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_strerror_without_device():
    assert _lib.strerror(_lib.TD_OK) == "ok"
    assert "range" in _lib.strerror(_lib.TD_E_RANGE)
    assert _lib.strerror(12345) == "unknown error"


def test_create_rejects_bad_config_before_touching_the_device():
    L = _lib.lib()
    h = ctypes.c_void_p()
    cfg = _lib.TdConfig(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=3, head_dim=64, intermediate=512,
                        vocab=100, max_ctx=16, rope_theta=1e4, rms_eps=1e-5, weight_format=0, qkv_bias=0)
    w = _lib.TdWeights()
    assert L.td_create(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.byref(h)) == _lib.TD_E_INVALID_ARG
    cfg.n_kv_heads = 2
    cfg.head_dim = 96
    assert L.td_create(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.byref(h)) == _lib.TD_E_INVALID_ARG
    assert not h.value


def _valid_config(**over):
    kw = dict(n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=64, intermediate=512, vocab=1000,
              max_ctx=64, rope_theta=1e4, rms_eps=1e-5, weight_format=_lib.TD_WF_BF16, qkv_bias=0)
    kw.update(over)
    return _lib.TdConfig(**kw)


def _fake_weights(n_layers, scales=False, bias=False, drop=None):
    """Non-null fake device addresses (td_create validates them before any device call)."""
    p = 0x10000
    fields = ["attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gu", "w_d"]
    if scales:
        fields += ["s_qkv", "s_o", "s_gu", "s_d"]
    if bias:
        fields += ["b_qkv"]
    arr = (_lib.TdLayerWeights * n_layers)()
    for i in range(n_layers):
        arr[i] = _lib.TdLayerWeights(**{f: (None if f == drop else p) for f in fields})
    w = _lib.TdWeights(embed=None if drop == "embed" else p, final_norm=p, head=p, layers=arr)
    return w, arr


@pytest.mark.parametrize("over", [
    dict(n_layers=0), dict(hidden=-256), dict(vocab=0), dict(max_ctx=0), dict(intermediate=0),
    dict(head_dim=96), dict(head_dim=32), dict(n_kv_heads=3), dict(n_q_heads=32, n_kv_heads=2),
    dict(hidden=320), dict(intermediate=520), dict(weight_format=7),
    dict(weight_format=_lib.TD_WF_INT4_G64, intermediate=576),
    dict(rope_theta=0.0), dict(rms_eps=-1.0),
])
def test_create_rejects_each_bad_config_field(over):
    L = _lib.lib()
    cfg = _valid_config(**over)
    w, keep = _fake_weights(max(1, cfg.n_layers), scales=True, bias=True)
    h = ctypes.c_void_p(123)
    assert L.td_create(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.byref(h)) == _lib.TD_E_INVALID_ARG
    assert h.value is None  # *out is cleared on error


@pytest.mark.parametrize("drop,fmt,bias", [
    ("embed", 0, 0), ("w_qkv", 0, 0), ("w_d", 0, 0), ("mlp_norm", 0, 0),
    ("s_gu", _lib.TD_WF_INT4_G64, 0), ("b_qkv", 0, 1),
])
def test_create_rejects_missing_weights(drop, fmt, bias):
    L = _lib.lib()
    cfg = _valid_config(weight_format=fmt, qkv_bias=bias)
    w, keep = _fake_weights(cfg.n_layers, scales=True, bias=True, drop=drop)
    h = ctypes.c_void_p()
    assert L.td_create(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.byref(h)) == _lib.TD_E_INVALID_ARG


def test_null_arguments_are_rejected():
    L = _lib.lib()
    assert L.td_create(None, None, 0, None) == _lib.TD_E_INVALID_ARG
    kv = _lib.TdKV(k=None, v=None, max_ctx=64)
    assert L.td_decode_step(None, None, 0, ctypes.byref(kv), None, None) == _lib.TD_E_INVALID_ARG
    assert L.td_decode_loop(None, None, 0, 4, -1, ctypes.byref(kv), None, None, None, None) == _lib.TD_E_INVALID_ARG
    assert L.td_forward_block(None, None, 4, 0, ctypes.byref(kv), None, 0, None, None) == _lib.TD_E_INVALID_ARG
    assert L.td_status(None, None) == _lib.TD_E_INVALID_ARG
    assert L.td_set_step_clock(None, None, 0) == _lib.TD_E_INVALID_ARG
    ms = ctypes.c_float()
    assert L.td_measure_stream(None, 1 << 20, 1, ctypes.byref(ms), None) == _lib.TD_E_INVALID_ARG
    # sizes and alignment are checked before any device call (the pointer is never dereferenced)
    fake = ctypes.c_void_p(1 << 40)
    assert L.td_measure_stream(fake, 8, 1, ctypes.byref(ms), None) == _lib.TD_E_INVALID_ARG
    assert L.td_measure_stream(fake, (1 << 20) + 4, 1, ctypes.byref(ms), None) == _lib.TD_E_INVALID_ARG
    assert L.td_measure_stream(ctypes.c_void_p((1 << 40) + 8), 1 << 20, 1, ctypes.byref(ms), None) == _lib.TD_E_INVALID_ARG
    assert L.td_measure_stream(fake, 1 << 20, 0, ctypes.byref(ms), None) == _lib.TD_E_INVALID_ARG
    assert L.td_measure_stream(fake, 1 << 20, 1, None, None) == _lib.TD_E_INVALID_ARG
    L.td_destroy(None)  # a no-op


@pytest.mark.parametrize("field", ["attn_norm", "w_qkv", "s_o", "b_qkv", "w_gu", "embed", "head", "final_norm"])
def test_create_rejects_weight_pointers_not_16_byte_aligned(field):
    """The kernels read weight rows and norm gains in 16-byte pieces, so td_create
    refuses a weight pointer that is not 16-byte aligned (8-byte aligned here),
    before any device call; the same weights aligned get past this check (and
    fail later, at the device query, on a host without a GPU)."""
    L = _lib.lib()
    cfg = _valid_config(weight_format=_lib.TD_WF_INT4_G64, qkv_bias=1)
    w, arr = _fake_weights(cfg.n_layers, scales=True, bias=True)
    h = ctypes.c_void_p()
    rc_aligned = L.td_create(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.byref(h))
    assert rc_aligned != _lib.TD_E_INVALID_ARG
    if field in ("embed", "head", "final_norm"):
        setattr(w, field, 0x10008)
    else:
        setattr(arr[1], field, 0x10008)
    assert L.td_create(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.byref(h)) == _lib.TD_E_INVALID_ARG
    assert b"16-byte aligned" in L.td_last_error()
    assert not h.value
