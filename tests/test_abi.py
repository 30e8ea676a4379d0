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
