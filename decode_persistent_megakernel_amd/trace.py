"""Summary of the in-kernel stage trace (td_set_trace): where one step's time goes.

For each stage of the step and each CU the kernel stamps (100 MHz device
clock): start, inputs staged, compute finished, epilogue finished, barrier
passed.  The summary splits the step into, per stage kind, the time to stage
inputs, the compute (weight streaming and arithmetic), the epilogue and the
wait at the grid barrier, averaged over CUs, and the critical path (the last
CU to finish the compute of each stage)."""
from __future__ import annotations

import numpy as np

KINDS = ["qkv", "attn", "o", "gu", "down", "head"]
TICK_US = 0.01  # 100 MHz


def summarize(trace: np.ndarray, n_layers: int) -> dict:
    full = trace.astype(np.int64)  # [ncu, stages, 32]
    t = full[:, :, :5]
    wv = full[:, :, 8:8 + 24].reshape(full.shape[0], full.shape[1], 8, 3)
    ns = t.shape[1]
    kinds = [KINDS[s % 5] if s < 5 * n_layers else "head" for s in range(ns)]
    t0 = t[:, 0, 0].min()
    step_us = (t[:, -1, 3].max() - t0) * TICK_US
    seg = np.diff(t, axis=2) * TICK_US  # [ncu, stages, 4]: prepare, compute, epilogue, barrier
    out = {"step_us": float(step_us), "stages": {}}
    for k in KINDS:
        idx = [i for i, kk in enumerate(kinds) if kk == k]
        if not idx:
            continue
        s = seg[:, idx, :]
        # critical-path view: per stage, time from the last CU's barrier exit of the
        # previous stage to the last CU's compute end
        prev_end = np.array([t[:, i - 1, 4].max() if i > 0 else t0 for i in idx])
        comp_end = np.array([t[:, i, 2].max() for i in idx])
        w = wv[:, idx]  # [ncu, n, 8, 3]
        has = w[..., 2] > 0
        first_wait = np.where(has, w[..., 1] - w[..., 0], 0) * TICK_US
        stream = np.where(has, w[..., 2] - w[..., 1], 0) * TICK_US
        nh = max(1, int(has.sum()))
        out["stages"][k] = {
            "wave_first_chunk_wait_us": float(first_wait.sum() / nh),
            "wave_stream_us": float(stream.sum() / nh),
            "count": len(idx),
            "prepare_us": float(s[..., 0].mean()),
            "compute_us_mean": float(s[..., 1].mean()),
            "compute_us_max": float(s[..., 1].max(axis=0).mean()),
            "epilogue_us": float(s[..., 2].mean()),
            "barrier_us_mean": float(s[..., 3].mean()),
            "span_us": float(((comp_end - prev_end) * TICK_US).mean()),
        }
    return out


def format_summary(s: dict) -> str:
    lines = [f"step {s['step_us']:.1f} us"]
    lines.append(f"{'stage':6} {'n':>3} {'prep':>7} {'comp':>7} {'compmax':>8} {'epi':>7} {'bar':>7} {'span':>7}"
                 f" {'w1st':>6} {'wstrm':>6}")
    for k, v in s["stages"].items():
        lines.append(f"{k:6} {v['count']:3d} {v['prepare_us']:7.2f} {v['compute_us_mean']:7.2f} "
                     f"{v['compute_us_max']:8.2f} {v['epilogue_us']:7.2f} {v['barrier_us_mean']:7.2f} "
                     f"{v['span_us']:7.2f} {v['wave_first_chunk_wait_us']:6.2f} {v['wave_stream_us']:6.2f}")
    return "\n".join(lines)
