"""Algorithmic HBM bytes of one batch-1 decode step.

A decode step reads every weight once ("Decoding in tiles", sec. 2: the bytes
of the weights over the bandwidth are the floor), plus one embedding row, the
K/V cache up to the current position, and writes one K/V row and the logits.
These are the bytes the metric counts; partial sums, barrier counters and
re-reads are not counted (hardware counters show those separately).
"""
from __future__ import annotations

WF_BF16 = 0
WF_INT4_G64 = 1


def linear_bytes(rows: int, cols: int, fmt: int) -> int:
    """Stored bytes of one [rows, cols] linear: bf16, or 4-bit codes plus one
    fp16 scale per 64 weights along cols."""
    if fmt == WF_BF16:
        return rows * cols * 2
    return rows * cols // 2 + rows * (cols // 64) * 2


def layer_weight_bytes(cfg) -> int:
    H, d = cfg.hidden, cfg.head_dim
    qkv_rows = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d
    b = linear_bytes(qkv_rows, H, cfg.weight_format)
    b += linear_bytes(H, cfg.n_q_heads * d, cfg.weight_format)
    # a mixture-of-experts layer streams its router and the top_k routed experts only
    # ("One launch per token", 64-expert section: the floor is set by the active weights)
    n_mlp = cfg.top_k if getattr(cfg, "n_experts", 0) else 1
    b += n_mlp * linear_bytes(2 * cfg.intermediate, H, cfg.weight_format)
    b += n_mlp * linear_bytes(H, cfg.intermediate, cfg.weight_format)
    if getattr(cfg, "n_experts", 0):
        b += cfg.n_experts * H * 2          # bf16 router
    b += 2 * H * 2                      # two bf16 norm gains
    if cfg.qkv_bias:
        b += qkv_rows * 2
    return b


def kv_bytes_per_position(cfg) -> int:
    """bf16 K and V rows of one position over all layers."""
    return cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * 2


def head_bytes(cfg) -> int:
    return cfg.vocab * cfg.hidden * 2


def weight_bytes_per_token(cfg) -> int:
    """Weights a token streams: all layers, the head, the final norm and one embedding row."""
    return cfg.n_layers * layer_weight_bytes(cfg) + head_bytes(cfg) + cfg.hidden * 2 + cfg.hidden * 2


def step_bytes(cfg, pos: int) -> int:
    """Algorithmic bytes of the step at position `pos` (reads K/V rows 0..pos)."""
    kv = kv_bytes_per_position(cfg)
    return weight_bytes_per_token(cfg) + (pos + 1) * kv + kv + 4 * cfg.vocab


def mean_step_bytes(cfg, first_pos: int, n_steps: int) -> float:
    return sum(step_bytes(cfg, first_pos + i) for i in range(n_steps)) / n_steps
