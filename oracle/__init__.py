"""Python binding of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports or links it, and
this module imports nothing from the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

WF_BF16 = 0
WF_INT4_G64 = 1
E_ARG = -1
E_NONFINITE = -6


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    hdr = os.path.join(_HERE, "oracle.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < newest:
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-semantic-interposition",
                               "-ffp-contract=off", "-Wall", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                              "intermediate", "vocab", "max_ctx")] + \
               [("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("weight_format", ctypes.c_int32), ("qkv_bias", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class _Layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "w_qkv", "s_qkv", "b_qkv", "w_o", "s_o", "mlp_norm",
                                               "w_gu", "s_gu", "w_d", "s_d", "w_router")]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(_Layer))]


class _Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x_in", "qkv", "attn", "x_mid", "act", "x_out", "h_final",
                                               "expert_ids", "expert_w")]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        d, i32, i64, vp = ctypes.c_double, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.orc_bf16_value.restype = d
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_value.restype = d
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16.argtypes = [d]
        L.orc_rmsnorm.argtypes = [vp, vp, i32, d, vp]
        L.orc_weight.restype = d
        L.orc_weight.argtypes = [vp, vp, i32, i32, i64, i32]
        L.orc_linear.argtypes = [vp, vp, i32, i32, i32, vp, vp, i32]
        L.orc_rope.argtypes = [vp, i32, i32, d]
        L.orc_attention.argtypes = [vp, vp, vp, i32, i32, vp]
        L.orc_silu.restype = d
        L.orc_silu.argtypes = [d]
        L.orc_argmax.restype = i32
        L.orc_argmax.argtypes = [vp, i32, vp]
        L.orc_route.restype = i32
        L.orc_route.argtypes = [vp, i32, i32, vp, vp]
        L.orc_step.restype = i32
        L.orc_step.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), i32, i32, vp, vp, vp, i32]
        L.orc_step_traced.restype = i32
        L.orc_step_traced.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), i32, i32, vp, vp, vp,
                                      i32, ctypes.POINTER(_Trace)]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]) -> Optional[int]:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def default_threads() -> int:
    return max(1, int(os.environ.get("ORACLE_THREADS", os.cpu_count() or 1)))


# --------------------------------------------------------------------------- pieces

def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(int(b))


def f16_value(h: int) -> float:
    return lib().orc_f16_value(int(h))


def round_bf16(v: float) -> int:
    return int(lib().orc_round_bf16(float(v)))


def rmsnorm(x: np.ndarray, gain_bf16: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(gain_bf16, dtype=np.uint16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(y))
    return y


def linear(w: np.ndarray, s: Optional[np.ndarray], fmt: int, rows: int, cols: int, x: np.ndarray,
           nthreads: Optional[int] = None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.size == cols
    w = np.ascontiguousarray(w)
    s = None if s is None else np.ascontiguousarray(s, dtype=np.uint16)
    y = np.empty(rows, dtype=np.float64)
    lib().orc_linear(_p(w), _p(s), fmt, rows, cols, _p(x), _p(y), nthreads or default_threads())
    return y


def weight(w: np.ndarray, s: Optional[np.ndarray], fmt: int, cols: int, r: int, k: int) -> float:
    return lib().orc_weight(_p(np.ascontiguousarray(w)), _p(s), fmt, cols, r, k)


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    out = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_p(out), out.size, pos, theta)
    return out


def attention(q: np.ndarray, K_bf16: np.ndarray, V_bf16: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K_bf16, dtype=np.uint16)
    V = np.ascontiguousarray(V_bf16, dtype=np.uint16)
    n, d = K.shape
    out = np.empty(d, dtype=np.float64)
    lib().orc_attention(_p(q), _p(K), _p(V), n, d, _p(out))
    return out


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def argmax(logits: np.ndarray):
    x = np.ascontiguousarray(logits, dtype=np.float64)
    bad = ctypes.c_int32(0)
    i = lib().orc_argmax(_p(x), x.size, ctypes.byref(bad))
    return int(i), bool(bad.value)


def route(z: np.ndarray, k: int):
    """MoE routing of router logits z[E]: (status, ids[k], weights[k])."""
    x = np.ascontiguousarray(z, dtype=np.float64)
    ids = np.zeros(max(k, 1), dtype=np.int32)
    w = np.zeros(max(k, 1), dtype=np.float64)
    r = lib().orc_route(_p(x), x.size, int(k), _p(ids), _p(w))
    return int(r), ids[:k], w[:k]


# --------------------------------------------------------------------------- whole step

class Oracle:
    """The oracle decoder over a synthetic model (synth.Model) with its own K/V caches."""

    def __init__(self, model, max_ctx: Optional[int] = None, nthreads: Optional[int] = None):
        cfg = model.cfg
        self.model = model
        self.cfg = cfg
        self.nthreads = nthreads or default_threads()
        self.c = _Config(n_layers=cfg.n_layers, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads,
                         n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, intermediate=cfg.intermediate,
                         vocab=cfg.vocab, max_ctx=max_ctx or cfg.max_ctx, rope_theta=cfg.rope_theta,
                         rms_eps=cfg.rms_eps, weight_format=cfg.weight_format, qkv_bias=int(cfg.qkv_bias),
                         n_experts=cfg.n_experts, top_k=cfg.top_k)
        self._layers = (_Layer * cfg.n_layers)()
        for i, L in enumerate(model.layers):
            self._layers[i] = _Layer(attn_norm=_p(L.attn_norm), w_qkv=_p(L.qkv.w), s_qkv=_p(L.qkv.s),
                                     b_qkv=_p(L.qkv_bias), w_o=_p(L.o.w), s_o=_p(L.o.s), mlp_norm=_p(L.mlp_norm),
                                     w_gu=_p(L.gate_up.w), s_gu=_p(L.gate_up.s), w_d=_p(L.down.w),
                                     s_d=_p(L.down.s), w_router=_p(L.router))
        self.w = _Weights(embed=_p(model.embed), head=_p(model.head), final_norm=_p(model.final_norm),
                          layers=self._layers)
        ctx = self.c.max_ctx
        shape = (cfg.n_layers, cfg.n_kv_heads, ctx, cfg.head_dim)
        self.k = np.zeros(shape, dtype=np.uint16)
        self.v = np.zeros(shape, dtype=np.uint16)

    def set_kv(self, k: np.ndarray, v: np.ndarray) -> None:
        assert k.shape == self.k.shape and v.shape == self.v.shape
        self.k[...] = k
        self.v[...] = v

    def step(self, token: int, pos: int, want_logits: bool = True):
        """Returns (next_token_or_error, logits or None)."""
        logits = np.empty(self.cfg.vocab, dtype=np.float64) if want_logits else None
        r = lib().orc_step(ctypes.byref(self.c), ctypes.byref(self.w), int(token), int(pos), _p(self.k),
                           _p(self.v), _p(logits) if logits is not None else None, self.nthreads)
        return int(r), logits

    def step_traced(self, token: int, pos: int):
        cfg = self.cfg
        L, H, I = cfg.n_layers, cfg.hidden, cfg.intermediate
        t = {
            "x_in": np.zeros(H), "qkv": np.zeros((L, cfg.qkv_rows)), "attn": np.zeros((L, cfg.q_dim)),
            "x_mid": np.zeros((L, H)), "act": np.zeros((L, I)), "x_out": np.zeros((L, H)), "h_final": np.zeros(H),
        }
        if cfg.n_experts:
            t["expert_ids"] = np.zeros((L, cfg.top_k), dtype=np.int32)
            t["expert_w"] = np.zeros((L, cfg.top_k))
        tr = _Trace(**{k: _p(v) for k, v in t.items()})
        logits = np.empty(cfg.vocab, dtype=np.float64)
        r = lib().orc_step_traced(ctypes.byref(self.c), ctypes.byref(self.w), int(token), int(pos), _p(self.k),
                                  _p(self.v), _p(logits), self.nthreads, ctypes.byref(tr))
        t["logits"] = logits
        return int(r), t

    def prefill(self, tokens, start: int = 0) -> None:
        """Runs the prompt through the decode step at positions start.. (logits skipped)."""
        for i, t in enumerate(tokens):
            r, _ = self.step(int(t), start + i, want_logits=False)
            assert r >= 0, r
