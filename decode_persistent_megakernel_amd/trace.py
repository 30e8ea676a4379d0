"""Summary of the in-kernel stage trace (td_set_trace): where one step's time goes.

For each CU and each stage of the step, every compute wave stamps (100 MHz
device clock): stage entered, inputs staged (the workgroup rendezvous passed),
first weight chunk in LDS (first attention tile done), last output published.
The summary gives, per stage kind and averaged over the layers:

  span      critical-path time the stage adds: from the last output of the
            previous stage to the last output of this one, over all CUs
  handoff   from the last output of the previous stage to the moment a CU has
            its inputs staged (minimum and median over CUs): the cross-CU
            hand-off latency
  work      per CU, from inputs staged to its last output (median and maximum
            over CUs): streaming plus arithmetic plus epilogue
"""
from __future__ import annotations

import numpy as np

KINDS = ["qkv", "attn", "o", "gu", "down", "head", "router"]
LAYER_KINDS = {5: ["qkv", "attn", "o", "gu", "down"], 6: ["qkv", "attn", "o", "router", "gu", "down"]}
TICK_US = 0.01  # 100 MHz


def summarize(trace: np.ndarray, n_layers: int, spl: int = 5) -> dict:
    """spl: stages per layer, 5 for a dense layer, 6 for a mixture-of-experts one (with the router)."""
    raw = trace.astype(np.int64).reshape(trace.shape[0], trace.shape[1], 8, 4)  # [ncu, stages, wave, stamp]
    ns = raw.shape[1]
    kinds = [LAYER_KINDS[spl][s % spl] if s < spl * n_layers else "head" for s in range(ns)]
    valid = raw > 0
    t0 = raw[..., 0][valid[..., 0]].min()
    t = (raw - t0) * TICK_US
    entered = np.where(valid[..., 0], t[..., 0], np.inf).min(axis=2)         # [ncu, stages]
    staged = np.where(valid[..., 1], t[..., 1], np.inf).min(axis=2)
    end = np.where(valid[..., 3], t[..., 3], -np.inf).max(axis=2)
    part = np.isfinite(entered)  # the CU took part in the stage
    stage_end = np.array([end[part[:, s], s].max() for s in range(ns)])
    out = {"step_us": float(stage_end[-1]), "stages": {}}
    for k in KINDS:
        idx = [i for i, kk in enumerate(kinds) if kk == k]
        if not idx:
            continue
        span, hmin, hmed, wmed, wmax = [], [], [], [], []
        for s in idx:
            prev = stage_end[s - 1] if s > 0 else 0.0
            span.append(stage_end[s] - prev)
            p = part[:, s]
            h = staged[p, s] - prev
            hmin.append(h.min())
            hmed.append(np.median(h))
            w = end[p, s] - staged[p, s]
            wmed.append(np.median(w))
            wmax.append(w.max())
        out["stages"][k] = {
            "count": len(idx),
            "span_us": float(np.mean(span)),
            "handoff_min_us": float(np.mean(hmin)),
            "handoff_med_us": float(np.mean(hmed)),
            "work_med_us": float(np.mean(wmed)),
            "work_max_us": float(np.mean(wmax)),
        }
    return out


def format_summary(s: dict) -> str:
    lines = [f"step {s['step_us']:.1f} us (first stamp to last output)"]
    lines.append(f"{'stage':6} {'n':>3} {'span':>7} {'hoffmin':>8} {'hoffmed':>8} {'workmed':>8} {'workmax':>8}")
    for k, v in s["stages"].items():
        lines.append(f"{k:6} {v['count']:3d} {v['span_us']:7.2f} {v['handoff_min_us']:8.2f} {v['handoff_med_us']:8.2f} "
                     f"{v['work_med_us']:8.2f} {v['work_max_us']:8.2f}")
    return "\n".join(lines)
