"""Batch-1 decode step of a Llama-style decoder on MI355X (gfx950).

Thin Python binding over the C ABI in include/td.h.  It only moves arguments:
device buffers come from PyTorch tensors (PyTorch is used for device memory and
streams), and every step of the decode runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import (TD_E_HIP, TD_E_INVALID_ARG, TD_E_NONFINITE, TD_E_PLAN, TD_E_RANGE, TD_E_TIMEOUT,
                   TD_E_UNSUPPORTED, TD_EXEC_GRAPH, TD_EXEC_MEGAKERNEL, TD_EXEC_PER_OP, TD_OK, TD_WF_BF16,
                   TD_WF_INT4_G64, TdError)

__all__ = ["DeviceModel", "Decoder", "KVCache", "gemv", "attention", "TdError"]


def _torch():
    import torch
    return torch


def _dev(arr: Optional[np.ndarray], device):
    """A device copy of a host array of stored-format bits (bf16/fp16 bits or bytes)."""
    if arr is None:
        return None
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class DeviceModel:
    """Weights of one model in device memory, in the stored formats of td.h.

    `model` is any object with `cfg` (n_layers, hidden, n_q_heads, n_kv_heads,
    head_dim, intermediate, vocab, rope_theta, rms_eps, weight_format, qkv_bias,
    tied), `embed`, `head`, `final_norm` and `layers` (attn_norm, qkv, qkv_bias,
    o, mlp_norm, gate_up, down; each linear with `.w` and `.s`) as host arrays.
    """

    def __init__(self, model, device: str = "cuda"):
        c = model.cfg
        self.cfg = c
        self.device = device
        self.embed = _dev(model.embed, device)
        self.head = self.embed if c.tied else _dev(model.head, device)
        self.final_norm = _dev(model.final_norm, device)
        self.layers = []
        for L in model.layers:
            self.layers.append({
                "attn_norm": _dev(L.attn_norm, device), "mlp_norm": _dev(L.mlp_norm, device),
                "w_qkv": _dev(L.qkv.w, device), "s_qkv": _dev(L.qkv.s, device),
                "b_qkv": _dev(L.qkv_bias, device),
                "w_o": _dev(L.o.w, device), "s_o": _dev(L.o.s, device),
                "w_gu": _dev(L.gate_up.w, device), "s_gu": _dev(L.gate_up.s, device),
                "w_d": _dev(L.down.w, device), "s_d": _dev(L.down.s, device),
                "w_router": _dev(getattr(L, "router", None), device),
            })

    def td_config(self, max_ctx: int) -> _lib.TdConfig:
        c = self.cfg
        return _lib.TdConfig(n_layers=c.n_layers, hidden=c.hidden, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
                             head_dim=c.head_dim, intermediate=c.intermediate, vocab=c.vocab, max_ctx=max_ctx,
                             rope_theta=c.rope_theta, rms_eps=c.rms_eps, weight_format=c.weight_format,
                             qkv_bias=int(c.qkv_bias), n_experts=getattr(c, "n_experts", 0),
                             top_k=getattr(c, "top_k", 0))

    def td_weights(self):
        n = len(self.layers)
        arr = (_lib.TdLayerWeights * n)()
        for i, L in enumerate(self.layers):
            arr[i] = _lib.TdLayerWeights(**{k: _ptr(v) for k, v in L.items()})
        w = _lib.TdWeights(embed=_ptr(self.embed), final_norm=_ptr(self.final_norm), head=_ptr(self.head),
                           layers=arr)
        return w, arr


class KVCache:
    """K and V caches in device memory: bf16 bits [n_layers][n_kv_heads][max_ctx][head_dim]."""

    def __init__(self, cfg, max_ctx: int, device: str = "cuda", k: Optional[np.ndarray] = None,
                 v: Optional[np.ndarray] = None):
        torch = _torch()
        shape = (cfg.n_layers, cfg.n_kv_heads, max_ctx, cfg.head_dim)
        self.max_ctx = max_ctx
        self.k = _dev(k, device) if k is not None else torch.zeros(shape, dtype=torch.int16, device=device)
        self.v = _dev(v, device) if v is not None else torch.zeros(shape, dtype=torch.int16, device=device)
        assert tuple(self.k.shape) == shape and tuple(self.v.shape) == shape

    def td_kv(self) -> _lib.TdKV:
        return _lib.TdKV(k=_ptr(self.k), v=_ptr(self.v), max_ctx=self.max_ctx)

    def host(self):
        return (self.k.cpu().numpy().view(np.uint16), self.v.cpu().numpy().view(np.uint16))


class Decoder:
    """One td_ctx: td_create at construction, td_decode_step per step (or
    td_decode_loop for several greedy steps in one launch)."""

    def __init__(self, dm: DeviceModel, max_ctx: int, executor: int = TD_EXEC_MEGAKERNEL):
        self.dm = dm
        self.max_ctx = max_ctx
        self._cfg = dm.td_config(max_ctx)
        self._w, self._layers = dm.td_weights()
        h = ctypes.c_void_p()
        _lib.check(_lib.lib().td_create(ctypes.byref(self._cfg), ctypes.byref(self._w), executor, ctypes.byref(h)),
                   "td_create")
        self._h = h

    @property
    def handle(self) -> int:
        return self._h.value

    def token_ptr(self) -> int:
        return _lib.lib().td_token_ptr(self._h)

    def routing(self):
        """The last step's MoE routing as host arrays (ids [L][top_k] int32, weights
        [L][top_k] float32), or None for a dense model (synchronous copy)."""
        c = self.dm.cfg
        if not getattr(c, "n_experts", 0):
            return None
        n = c.n_layers * c.top_k
        ids = np.empty(n, dtype=np.int32)
        w = np.empty(n, dtype=np.float32)
        for dst, src in ((ids, _lib.lib().td_expert_ids(self._h)), (w, _lib.lib().td_expert_weights(self._h))):
            e = _hip_rt().hipMemcpy(dst.ctypes.data, src, dst.nbytes, 2)
            if e != 0:
                raise RuntimeError(f"hipMemcpy failed: {e}")
        return ids.reshape(c.n_layers, c.top_k), w.reshape(c.n_layers, c.top_k)

    def step(self, token_ptr: int, pos: int, kv: KVCache, logits, stream=None) -> None:
        """One decode step; `token_ptr` is a device int32 address, `logits` a float32 device tensor [vocab]."""
        kvs = kv.td_kv()
        _lib.check(_lib.lib().td_decode_step(self._h, token_ptr, int(pos), ctypes.byref(kvs), _ptr(logits),
                                             _stream_handle(stream)), "td_decode_step")

    def loop(self, token_ptr: int, pos: int, n_steps: int, kv: KVCache, logits, tokens=None, count=None,
             eos: int = -1, stream=None) -> None:
        """Up to n_steps greedy steps in one launch (td_decode_loop); `tokens` (int32 device
        tensor [n_steps]) and `count` (int32 device tensor [1]) are optional outputs."""
        kvs = kv.td_kv()
        _lib.check(_lib.lib().td_decode_loop(self._h, token_ptr, int(pos), int(n_steps), int(eos), ctypes.byref(kvs),
                                             _ptr(logits), _ptr(tokens), _ptr(count), _stream_handle(stream)),
                   "td_decode_loop")

    def forward_block(self, tokens, pos0: int, kv: KVCache, logits, all_logits: bool = False, argmax=None,
                      stream=None) -> None:
        """len(tokens) consecutive tokens at positions pos0.. in one pass (td_forward_block);
        `tokens` is an int32 device tensor, `logits` float32 [vocab] (or [n][vocab] with
        all_logits), `argmax` an optional int32 device tensor ([n] with all_logits, else [1])."""
        kvs = kv.td_kv()
        _lib.check(_lib.lib().td_forward_block(self._h, _ptr(tokens), int(tokens.numel()), int(pos0),
                                               ctypes.byref(kvs), _ptr(logits), int(bool(all_logits)), _ptr(argmax),
                                               _stream_handle(stream)), "td_forward_block")

    def status(self) -> int:
        err = ctypes.c_int32(0)
        return int(_lib.lib().td_status(self._h, ctypes.byref(err)))

    def set_step_clock(self, buf) -> None:
        """Following loop launches write their per-step clock into buf (uint64/int64 device tensor), or off."""
        _lib.check(_lib.lib().td_set_step_clock(self._h, None if buf is None else buf.data_ptr(),
                                                0 if buf is None else int(buf.numel())), "td_set_step_clock")

    def set_timing(self, enable: bool) -> None:
        _lib.check(_lib.lib().td_set_timing(self._h, int(enable)), "td_set_timing")

    def last_step_ms(self) -> float:
        return float(_lib.lib().td_last_step_ms(self._h))

    def enable_trace(self, on: bool = True):
        """Returns the device trace tensor (uint64 [ncu, n_stages, 32]) that following steps fill."""
        torch = _torch()
        if not on:
            _lib.check(_lib.lib().td_set_trace(self._h, None, 0), "td_set_trace")
            self._trace = None
            return None
        n = int(_lib.lib().td_trace_bytes(self._h))
        c = self.dm.cfg
        stages = (6 if getattr(c, "n_experts", 0) else 5) * c.n_layers + 1  # a MoE layer adds the router stage
        self._trace = torch.zeros(n // 8, dtype=torch.int64, device=self.dm.device)
        _lib.check(_lib.lib().td_set_trace(self._h, self._trace.data_ptr(), n), "td_set_trace")
        return self._trace.view(-1, stages, 32)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _lib.lib().td_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_step_noalloc(dm: "DeviceModel", max_ctx: int, token_ptr: int, pos: int, kv: "KVCache", logits,
                        token_out, error_out, stream=None) -> None:
    """One decode step with no context and no device allocation (td_decode_step_noalloc):
    the library's fixed scratch array holds every intermediate; token_out and error_out
    are int32 device tensors [1]."""
    cfg = dm.td_config(max_ctx)
    w, _layers = dm.td_weights()
    kvs = kv.td_kv()
    _lib.check(_lib.lib().td_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(w), token_ptr, int(pos),
                                                 ctypes.byref(kvs), _ptr(logits), _ptr(token_out), _ptr(error_out),
                                                 _stream_handle(stream)), "td_decode_step_noalloc")


def measure_stream(buf, reps: int = 5, stream=None) -> float:
    """The stream-read yardstick over a device tensor: GB/s of reps timed read passes."""
    ms = ctypes.c_float(0.0)
    nbytes = buf.numel() * buf.element_size()
    _lib.check(_lib.lib().td_measure_stream(buf.data_ptr(), nbytes, int(reps), ctypes.byref(ms),
                                            _stream_handle(stream)), "td_measure_stream")
    return nbytes * reps / (ms.value * 1e-3) / 1e9


def gemv(fmt: int, w, s, rows: int, cols: int, x, y, stream=None) -> None:
    """y = W x on device tensors through the test hook (same chunk arithmetic as the step)."""
    _lib.check(_lib.lib().td_test_gemv(fmt, _ptr(w), _ptr(s), rows, cols, _ptr(x), _ptr(y), _stream_handle(stream)),
               "td_test_gemv")


def attention(q, k, v, n_pos: int, head_dim: int, out, chunk_len: int = 0, waves: int = 1, stream=None) -> None:
    """One query head over n_pos K/V rows through the step's tile, wave-fold and merge
    routines, as `waves` waves of the head run them in the step (test hook)."""
    _lib.check(_lib.lib().td_test_attention(_ptr(q), _ptr(k), _ptr(v), n_pos, head_dim, int(chunk_len), int(waves),
                                            _ptr(out), _stream_handle(stream)), "td_test_attention")



def rope(x, n_heads: int, head_dim: int, pos: int, theta: float, out, stream=None) -> None:
    """Half-split RoPE at one position through the step's rotation (test hook)."""
    _lib.check(_lib.lib().td_test_rope(_ptr(x), n_heads, head_dim, int(pos), float(theta), _ptr(out),
                                       _stream_handle(stream)), "td_test_rope")


def argmax(logits, n: int, groups: int, work, token, nonfinite, stream=None) -> None:
    """The step's greedy selection over n logits in `groups` workgroups (test hook)."""
    _lib.check(_lib.lib().td_test_argmax(_ptr(logits), n, groups, _ptr(work), _ptr(token), _ptr(nonfinite),
                                         _stream_handle(stream)), "td_test_argmax")


_hip = None


def _hip_rt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return _hip


def read_device_i32(ptr: int) -> int:
    """Reads one int32 from a device address (synchronous copy on the null stream)."""
    v = ctypes.c_int32(0)
    e = _hip_rt().hipMemcpy(ctypes.byref(v), ptr, 4, 2)  # hipMemcpyDeviceToHost
    if e != 0:
        raise RuntimeError(f"hipMemcpy failed: {e}")
    return int(v.value)
