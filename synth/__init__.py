"""Seeded synthetic inputs for the batch-1 decode step.

This module draws the random-init weights, prompts and K/V prefixes that the
workloads below are defined on, and nothing else: it holds none of the
decoder's arithmetic.  The CPU oracle (test infrastructure) and the GPU library
consume the same bytes from here.

The five workloads are the decoder shapes the pages measure (Llama-3.2-1B in
"Decoding in tiles" sec. 2; TinyLlama-1.1B int4 in tinyinfer's "speed limit"
section; Qwen2.5-1.5B in "One launch per token"), plus a tiny model and a
long-context stress case.  Trained checkpoints are not used: weights are
random, with the shapes, formats and value distributions listed per config.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

WF_BF16 = 0
WF_INT4_G64 = 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rope_theta: float
    rms_eps: float
    weight_format: int          # WF_BF16 or WF_INT4_G64 (layer linears only)
    qkv_bias: bool
    tied: bool
    prompt_len: int             # tokens prefilled before decoding (0: random K/V prefix)
    kv_prefix: int              # random K/V positions (long-context stress), else 0
    decode_steps: int
    max_ctx: int
    seed: int
    n_experts: int = 0          # mixture-of-experts MLP: experts per layer (0: dense MLP)
    top_k: int = 0              # experts each token is routed to

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def start_pos(self) -> int:
        return self.prompt_len + self.kv_prefix


def _cfg(**kw) -> Config:
    return Config(**kw)


# c0 .. c4: the workloads.  rms_eps: 1e-5 for the Llama family, 1e-6 for Qwen2.5.
CONFIGS: Dict[str, Config] = {
    "tiny": _cfg(name="tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 intermediate=1024, vocab=4096, rope_theta=10000.0, rms_eps=1e-5,
                 weight_format=WF_BF16, qkv_bias=False, tied=True, prompt_len=16, kv_prefix=0,
                 decode_steps=16, max_ctx=32, seed=1000),
    "llama1b": _cfg(name="llama1b", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8,
                    head_dim=64, intermediate=8192, vocab=128256, rope_theta=500000.0,
                    rms_eps=1e-5, weight_format=WF_BF16, qkv_bias=False, tied=True,
                    prompt_len=512, kv_prefix=0, decode_steps=128, max_ctx=640, seed=1001),
    "tinyllama_int4": _cfg(name="tinyllama_int4", n_layers=22, hidden=2048, n_q_heads=32,
                           n_kv_heads=4, head_dim=64, intermediate=5632, vocab=32000,
                           rope_theta=10000.0, rms_eps=1e-5, weight_format=WF_INT4_G64,
                           qkv_bias=False, tied=False, prompt_len=256, kv_prefix=0,
                           decode_steps=128, max_ctx=384, seed=1002),
    "qwen1p5b": _cfg(name="qwen1p5b", n_layers=28, hidden=1536, n_q_heads=12, n_kv_heads=2,
                     head_dim=128, intermediate=8960, vocab=151936, rope_theta=1e6,
                     rms_eps=1e-6, weight_format=WF_BF16, qkv_bias=True, tied=True,
                     prompt_len=1024, kv_prefix=0, decode_steps=64, max_ctx=1088, seed=1003),
    "llama1b_int4_long": _cfg(name="llama1b_int4_long", n_layers=16, hidden=2048, n_q_heads=32,
                              n_kv_heads=8, head_dim=64, intermediate=8192, vocab=128256,
                              rope_theta=500000.0, rms_eps=1e-5, weight_format=WF_INT4_G64,
                              qkv_bias=False, tied=True, prompt_len=0, kv_prefix=8192,
                              decode_steps=64, max_ctx=8256, seed=1004),
    # f3: a mixture-of-experts decoder of the OLMoE-1B-7B shape (64 experts of
    # intermediate 1024, 8 routed per token; 16 query and 16 kv heads of 128;
    # vocab 50304; untied), with a random K/V prefix of 512 positions.
    "olmoe": _cfg(name="olmoe", n_layers=16, hidden=2048, n_q_heads=16, n_kv_heads=16, head_dim=128,
                  intermediate=1024, vocab=50304, rope_theta=10000.0, rms_eps=1e-5, weight_format=WF_BF16,
                  qkv_bias=False, tied=False, prompt_len=0, kv_prefix=512, decode_steps=64, max_ctx=576,
                  seed=1005, n_experts=64, top_k=8),
}
# the workloads of the native driver (td_bench)
CONFIG_ORDER: List[str] = ["tiny", "llama1b", "tinyllama_int4", "qwen1p5b", "llama1b_int4_long", "olmoe"]


def shrink(cfg: Config, **over) -> Config:
    """A copy of `cfg` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **over)


# --------------------------------------------------------------------------- build / load

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, i32, ctypes.c_char_p]
        L.synth_fill_bf16_normal.argtypes = [vp, i64, u64, ctypes.c_double, ctypes.c_double]
        L.synth_fill_bf16_const.argtypes = [vp, i64, ctypes.c_float]
        L.synth_fill_f16_absnormal.argtypes = [vp, i64, u64, ctypes.c_double]
        L.synth_fill_u8_uniform.argtypes = [vp, i64, u64]
        L.synth_fill_i32_uniform.argtypes = [vp, i64, u64, i32]
        L.synth_stream_at.restype = u64
        L.synth_stream_at.argtypes = [u64, u64]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_f32_to_f16.restype = ctypes.c_uint16
        L.synth_f32_to_f16.argtypes = [ctypes.c_float]
        _lib = L
    return _lib


def key(seed: int, layer: int, name: str) -> int:
    return int(lib().synth_key(seed, layer, name.encode()))


def bf16_normal(n: int, k: int, std: float, mean: float = 0.0) -> np.ndarray:
    a = np.empty(n, dtype=np.uint16)
    lib().synth_fill_bf16_normal(a.ctypes.data, n, k, mean, std)
    return a


def bf16_const(n: int, v: float) -> np.ndarray:
    a = np.empty(n, dtype=np.uint16)
    lib().synth_fill_bf16_const(a.ctypes.data, n, v)
    return a


def f16_absnormal(n: int, k: int, std: float) -> np.ndarray:
    a = np.empty(n, dtype=np.uint16)
    lib().synth_fill_f16_absnormal(a.ctypes.data, n, k, std)
    return a


def u8_uniform(n: int, k: int) -> np.ndarray:
    a = np.empty(n, dtype=np.uint8)
    lib().synth_fill_u8_uniform(a.ctypes.data, n, k)
    return a


def i32_uniform(n: int, k: int, hi: int) -> np.ndarray:
    a = np.empty(n, dtype=np.int32)
    lib().synth_fill_i32_uniform(a.ctypes.data, n, k, hi)
    return a


# --------------------------------------------------------------------------- model

WEIGHT_STD = 0.02      # linear layers, embedding, head, QKV bias
SCALE_STD = 0.003      # int4 group scales: |N(0, 0.003)| in fp16
KV_STD = 1.0           # random K/V prefix of the long-context stress case


@dataclasses.dataclass
class Linear:
    """One linear layer's stored weight.

    bf16:  `w` is uint16 [rows, K] (bf16 bits), `s` is None.
    int4:  `w` is uint8 [rows, K/2] (element k in byte k/2, low nibble for even k,
           stored code u in 0..15 standing for q = u - 8), `s` is uint16 [rows, K/64]
           (fp16 bits, one scale per 64 consecutive elements along K).
    """
    w: np.ndarray
    s: Optional[np.ndarray]
    rows: int
    cols: int


@dataclasses.dataclass
class Layer:
    attn_norm: np.ndarray      # bf16 [H]
    qkv: Linear                # [(nq + 2 nkv) d, H]: q rows, then k rows, then v rows
    qkv_bias: Optional[np.ndarray]  # bf16 [(nq + 2 nkv) d]
    o: Linear                  # [H, nq d]
    mlp_norm: np.ndarray       # bf16 [H]
    gate_up: Linear            # [2 I, H]: gate rows, then up rows; MoE: [E][2 I][H], expert e's block at rows 2 I e
    down: Linear               # [H, I]; MoE: [E][H][I], expert e's block at rows H e
    router: Optional[np.ndarray] = None  # MoE only: bf16 [E, H]


@dataclasses.dataclass
class Model:
    cfg: Config
    embed: np.ndarray          # bf16 [V, H]
    head: np.ndarray           # bf16 [V, H]; the same array as embed when tied
    final_norm: np.ndarray     # bf16 [H]
    layers: List[Layer]

    def nbytes(self) -> int:
        tot = self.embed.nbytes + self.final_norm.nbytes + (0 if self.cfg.tied else self.head.nbytes)
        for L in self.layers:
            tot += L.attn_norm.nbytes + L.mlp_norm.nbytes
            for lin in (L.qkv, L.o, L.gate_up, L.down):
                tot += lin.w.nbytes + (lin.s.nbytes if lin.s is not None else 0)
            if L.qkv_bias is not None:
                tot += L.qkv_bias.nbytes
            if L.router is not None:
                tot += L.router.nbytes
        return tot

    def active_nbytes(self) -> int:
        """Bytes one decode step reads from the weights: a MoE layer reads the router
        and the top_k routed experts only."""
        c = self.cfg
        if not c.n_experts:
            return self.nbytes()
        tot = self.nbytes()
        for L in self.layers:
            for lin in (L.gate_up, L.down):
                per = (lin.w.nbytes + (lin.s.nbytes if lin.s is not None else 0)) // c.n_experts
                tot -= per * (c.n_experts - c.top_k)
        return tot


def _linear(cfg: Config, layer: int, name: str, rows: int, cols: int) -> Linear:
    seed = cfg.seed
    if cfg.weight_format == WF_BF16:
        w = bf16_normal(rows * cols, key(seed, layer, name), WEIGHT_STD).reshape(rows, cols)
        return Linear(w=w, s=None, rows=rows, cols=cols)
    assert cols % 64 == 0, "int4 group-64 needs K divisible by 64"
    w = u8_uniform(rows * cols // 2, key(seed, layer, name)).reshape(rows, cols // 2)
    s = f16_absnormal(rows * cols // 64, key(seed, layer, name + ".scale"), SCALE_STD)
    return Linear(w=w, s=s.reshape(rows, cols // 64), rows=rows, cols=cols)


def make_model(cfg: Config) -> Model:
    H, I, V = cfg.hidden, cfg.intermediate, cfg.vocab
    seed = cfg.seed
    embed = bf16_normal(V * H, key(seed, -1, "embed"), WEIGHT_STD).reshape(V, H)
    head = embed if cfg.tied else bf16_normal(V * H, key(seed, -1, "head"), WEIGHT_STD).reshape(V, H)
    layers = []
    for l in range(cfg.n_layers):
        bias = None
        if cfg.qkv_bias:
            bias = bf16_normal(cfg.qkv_rows, key(seed, l, "qkv_bias"), WEIGHT_STD)
        E = max(cfg.n_experts, 1)
        router = None
        if cfg.n_experts:
            router = bf16_normal(E * H, key(seed, l, "router"), WEIGHT_STD).reshape(E, H)
        layers.append(Layer(
            attn_norm=bf16_const(H, 1.0),
            qkv=_linear(cfg, l, "qkv", cfg.qkv_rows, H),
            qkv_bias=bias,
            o=_linear(cfg, l, "o", H, cfg.q_dim),
            mlp_norm=bf16_const(H, 1.0),
            gate_up=_linear(cfg, l, "gate_up", E * 2 * I, H),
            down=_linear(cfg, l, "down", E * H, I),
            router=router,
        ))
    return Model(cfg=cfg, embed=embed, head=head, final_norm=bf16_const(H, 1.0), layers=layers)


def prompt(cfg: Config) -> np.ndarray:
    return i32_uniform(cfg.prompt_len, key(cfg.seed, -1, "prompt"), cfg.vocab)


def first_token(cfg: Config) -> int:
    """The first decode input when there is no prompt (random K/V prefix case)."""
    return int(i32_uniform(1, key(cfg.seed, -1, "first_token"), cfg.vocab)[0])


def kv_cache(cfg: Config) -> tuple:
    """Zeroed K and V caches, uint16 (bf16 bits) [L, n_kv, max_ctx, d] each; with a
    random prefix of `kv_prefix` positions drawn from N(0, 1) when the config asks."""
    shape = (cfg.n_layers, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
    k = np.zeros(shape, dtype=np.uint16)
    v = np.zeros(shape, dtype=np.uint16)
    if cfg.kv_prefix:
        P = cfg.kv_prefix
        for l in range(cfg.n_layers):
            for g in range(cfg.n_kv_heads):
                k[l, g, :P] = bf16_normal(P * cfg.head_dim, key(cfg.seed, l * 1000 + g, "k_prefix"),
                                          KV_STD).reshape(P, cfg.head_dim)
                v[l, g, :P] = bf16_normal(P * cfg.head_dim, key(cfg.seed, l * 1000 + g, "v_prefix"),
                                          KV_STD).reshape(P, cfg.head_dim)
    return k, v


def random_kv_prefix(cfg: Config, n_pos: int, seed_tag: str = "kv_stand_in", std: float = KV_STD):
    """K/V caches whose first `n_pos` positions are seeded random bf16 values.

    Stands in for a prompt prefill where running the prompt through the CPU
    oracle would take minutes; the decode step reads the cache the same way
    whatever produced it."""
    shape = (cfg.n_layers, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
    k = np.zeros(shape, dtype=np.uint16)
    v = np.zeros(shape, dtype=np.uint16)
    for l in range(cfg.n_layers):
        for g in range(cfg.n_kv_heads):
            k[l, g, :n_pos] = bf16_normal(n_pos * cfg.head_dim,
                                          key(cfg.seed, l * 1000 + g, seed_tag + ".k"), std).reshape(n_pos, cfg.head_dim)
            v[l, g, :n_pos] = bf16_normal(n_pos * cfg.head_dim,
                                          key(cfg.seed, l * 1000 + g, seed_tag + ".v"), std).reshape(n_pos, cfg.head_dim)
    return k, v
