"""ctypes declarations of the C ABI in include/td.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_PKG, "libtd.so")

TD_OK = 0
TD_E_INVALID_ARG = -1
TD_E_UNSUPPORTED = -2
TD_E_PLAN = -3
TD_E_RANGE = -4
TD_E_HIP = -5
TD_E_NONFINITE = -6
TD_E_NOMEM = -7
TD_E_TIMEOUT = -8

TD_WF_BF16 = 0
TD_WF_INT4_G64 = 1

TD_EXEC_MEGAKERNEL = 0
TD_EXEC_PER_OP = 1
TD_EXEC_GRAPH = 2

TD_MAX_LOOP_STEPS = 256
TD_MAX_BLOCK = 64
TD_MAX_EXPERTS = 256
TD_MAX_TOPK = 16
TD_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTED = [
    "td_create", "td_decode_step", "td_decode_step_noalloc", "td_decode_loop", "td_forward_block", "td_token_ptr", "td_expert_ids", "td_expert_weights", "td_status", "td_destroy", "td_strerror", "td_last_error",
    "td_plan_partition", "td_plan_check",
    "td_test_gemv", "td_test_attention", "td_test_rope", "td_test_argmax", "td_set_timing", "td_last_step_ms", "td_set_step_clock", "td_measure_stream", "td_trace_bytes", "td_set_trace",
]


class TdConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                              "intermediate", "vocab", "max_ctx")] + \
               [("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("weight_format", ctypes.c_int32), ("qkv_bias", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class TdLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "w_qkv", "s_qkv", "b_qkv", "w_o", "s_o", "mlp_norm",
                                               "w_gu", "s_gu", "w_d", "s_d", "w_router")]


class TdWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(TdLayerWeights))]


class TdKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("max_ctx", ctypes.c_int32)]


class TdError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {code} ({strerror(code)}) {last_error()}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtd.so.  There is no fallback: without the built library the
    decode step cannot run, and this raises."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(f"{SO_PATH} is not built; run decode_persistent_megakernel_amd/build.py "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(SO_PATH)
        i32, vp, f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        L.td_create.restype = i32
        L.td_create.argtypes = [ctypes.POINTER(TdConfig), ctypes.POINTER(TdWeights), i32, ctypes.POINTER(vp)]
        L.td_decode_step.restype = i32
        L.td_decode_step.argtypes = [vp, vp, i32, ctypes.POINTER(TdKV), vp, vp]
        L.td_decode_step_noalloc.restype = i32
        L.td_decode_step_noalloc.argtypes = [ctypes.POINTER(TdConfig), ctypes.POINTER(TdWeights), vp, i32,
                                             ctypes.POINTER(TdKV), vp, vp, vp, vp]
        L.td_decode_loop.restype = i32
        L.td_decode_loop.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(TdKV), vp, vp, vp, vp]
        L.td_forward_block.restype = i32
        L.td_forward_block.argtypes = [vp, vp, i32, i32, ctypes.POINTER(TdKV), vp, i32, vp, vp]
        L.td_token_ptr.restype = vp
        L.td_expert_ids.restype = vp
        L.td_expert_ids.argtypes = [vp]
        L.td_expert_weights.restype = vp
        L.td_expert_weights.argtypes = [vp]
        L.td_token_ptr.argtypes = [vp]
        L.td_status.restype = i32
        L.td_status.argtypes = [vp, ctypes.POINTER(i32)]
        L.td_destroy.restype = None
        L.td_destroy.argtypes = [vp]
        L.td_strerror.restype = ctypes.c_char_p
        L.td_strerror.argtypes = [i32]
        L.td_last_error.restype = ctypes.c_char_p
        L.td_last_error.argtypes = []
        L.td_plan_partition.restype = i32
        L.td_plan_partition.argtypes = [ctypes.POINTER(TdConfig), i32, vp, i32]
        L.td_plan_check.restype = i32
        L.td_plan_check.argtypes = [ctypes.POINTER(TdConfig), i32, vp, i32]
        L.td_test_gemv.restype = i32
        L.td_test_gemv.argtypes = [i32, vp, vp, i32, i32, vp, vp, vp]
        L.td_test_attention.restype = i32
        L.td_test_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
        L.td_test_rope.restype = i32
        L.td_test_rope.argtypes = [vp, i32, i32, i32, f32, vp, vp]
        L.td_test_argmax.restype = i32
        L.td_test_argmax.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.td_set_step_clock.restype = i32
        L.td_set_step_clock.argtypes = [vp, vp, i32]
        L.td_measure_stream.restype = i32
        L.td_measure_stream.argtypes = [vp, ctypes.c_int64, i32, ctypes.POINTER(f32), vp]
        L.td_set_timing.restype = i32
        L.td_set_timing.argtypes = [vp, i32]
        L.td_last_step_ms.restype = f32
        L.td_last_step_ms.argtypes = [vp]
        L.td_trace_bytes.restype = ctypes.c_int64
        L.td_trace_bytes.argtypes = [vp]
        L.td_set_trace.restype = i32
        L.td_set_trace.argtypes = [vp, vp, ctypes.c_int64]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    try:
        return lib().td_strerror(code).decode()
    except RuntimeError:
        return "?"


def last_error() -> str:
    try:
        return lib().td_last_error().decode()
    except RuntimeError:
        return ""


def check(code: int, what: str) -> None:
    if code != TD_OK:
        raise TdError(code, what)
