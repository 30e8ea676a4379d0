#!/usr/bin/env python3
"""Benchmark of the batch-1 decode step on one MI355X.

Workload (default): the Llama-3.2-1B-shaped bf16 decoder (16 layers, hidden
2048, 32 q / 8 kv heads of 64, intermediate 8192, vocab 128256, tied
embeddings, RoPE theta 500000) with seeded random-init weights ~N(0, 0.02).
A seeded random 512-token prompt is prefilled into the K/V cache by the block
forward (td_forward_block, 64 tokens per call on the matrix cores; its rate is
reported as "prefill"); then greedy decode steps run at positions 512, 513, ...
with the token chained on the device.  A "step" is one decode
step (one token).  W warmup steps run first (positions 512..), then the K timed
steps restart at position 512 (each step rewrites its own cache row first).

Printed: one JSON line with tokens/s, ms/token, the roofline of the decode
kernel (algorithmic HBM bytes per step / measured kernel time, against the
8 TB/s HBM peak) and the CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def source_hash() -> str:
    """sha256 (first 16 hex digits) of the sources that define the decode kernel
    and its launch plan; a counter summary taken on other sources is stale."""
    from decode_persistent_megakernel_amd.profile import sources_hash
    return sources_hash()


def read_traffic(workload: str, kernel_hash: str):
    """HBM bytes per decode step from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"megakernel_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != kernel_hash:
        return None
    try:
        return int(float(vals["fetch_bytes_per_step"]) + float(vals["write_bytes_per_step"]))
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(model, cfg, pos0: int, budget_s: float):
    """The CPU oracle (fp64, all host threads) on decode steps of the same model
    at the same positions, for about `budget_s` seconds (at least 2 steps)."""
    import oracle
    import synth

    nthreads = int(os.environ.get("ORACLE_THREADS", os.cpu_count() or 1))
    o = oracle.Oracle(model, nthreads=nthreads)
    k, v = synth.random_kv_prefix(cfg, pos0, seed_tag="cpu_baseline")
    o.set_kv(k, v)
    t = synth.first_token(cfg)
    n = 0
    t0 = time.perf_counter()
    while True:
        r, _ = o.step(t, pos0 + n)
        t = r if r >= 0 else 0
        n += 1
        el = time.perf_counter() - t0
        if (n >= 2 and el >= budget_s) or pos0 + n >= cfg.max_ctx:
            break
    # the same oracle on one thread, for two more steps: after the last position
    # when the cache has room, else again at the first two (timing only)
    o.nthreads = 1
    p1 = pos0 + n if pos0 + n + 2 <= cfg.max_ctx else pos0
    n1 = 0
    t1 = time.perf_counter()
    while n1 < 2 and p1 + n1 < cfg.max_ctx:
        r, _ = o.step(t, p1 + n1)
        t = r if r >= 0 else 0
        n1 += 1
    el1 = time.perf_counter() - t1
    return {"value": round(n / el, 4), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"{n} decode steps of the same workload at positions {pos0}..{pos0 + n - 1}, "
                      f"fp64 scalar C oracle, {nthreads} OpenMP threads, K/V prefix random",
            "ms_per_token": round(el / n * 1e3, 2),
            "single_thread": ({"ms_per_token": round(el1 / n1 * 1e3, 2), "steps": n1,
                               "positions": [p1, p1 + n1 - 1]} if n1 else None)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 128, or fewer where the workload's cache holds fewer)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="llama1b")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--trace", default=None, help="write the in-kernel stage trace summary of one step here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (a known-size kernel for counter calibration)")
    ap.add_argument("--baseline-steps", type=int, default=32,
                    help="timed steps of each baseline (one launch per step, per-op launches, graph replay); 0 = skip")
    ap.add_argument("--steps-per-launch", type=int, default=64,
                    help="greedy steps per td_decode_loop launch (1 = one td_decode_step launch per token)")
    ap.add_argument("--prefill-block", type=int, default=64,
                    help="prompt tokens per td_forward_block call (0 = prefill through the decode step)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); the library runs on one GPU and has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import decode_persistent_megakernel_amd as td
    from decode_persistent_megakernel_amd import accounting
    import synth

    cfg = synth.CONFIGS[args.config]
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    model = synth.make_model(cfg)
    print(f"[bench] generated {model.nbytes() / 1e9:.2f} GB of weights in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    dm = td.DeviceModel(model, device=dev)
    moe = cfg.n_experts > 0
    # every model, dense or mixture-of-experts, runs on the persistent kernel and its token loop
    dec = td.Decoder(dm, cfg.max_ctx, executor=td.TD_EXEC_MEGAKERNEL)
    start = cfg.start_pos
    prefill = None
    if cfg.kv_prefix:
        k, v = synth.kv_cache(cfg)
        kv = td.KVCache(cfg, cfg.max_ctx, device=dev, k=k, v=v)
        first = torch.tensor([synth.first_token(cfg)], dtype=torch.int32, device=dev)
        del k, v
    else:
        kv = td.KVCache(cfg, cfg.max_ctx, device=dev)
        prompt = synth.prompt(cfg)
        scratch_logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
        t_pf = time.perf_counter()
        if args.prefill_block > 0:
            blk = max(1, min(args.prefill_block, td._lib.TD_MAX_BLOCK))
            ptoks = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).to(dev)
            pstream = torch.cuda.current_stream()

            def prefill_pass():
                for i in range(0, len(prompt), blk):
                    dec.forward_block(ptoks[i:i + blk], i, kv, scratch_logits, stream=pstream)

            prefill_pass()  # untimed (first-call setup)
            torch.cuda.synchronize()
            pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            pe0.record(pstream)
            prefill_pass()  # the same positions again: the cache rows are rewritten with the same values
            pe1.record(pstream)
            torch.cuda.synchronize()
            pms = pe0.elapsed_time(pe1)
            prefill = {"tokens": len(prompt), "block_rows": blk, "calls": (len(prompt) + blk - 1) // blk,
                       "ms": round(pms, 3), "tokens_per_s": round(len(prompt) / (pms / 1e3), 1),
                       "path": "td_forward_block (MFMA GEMMs, fp32 inputs split into three bf16 parts)"}
        else:
            tok = torch.empty(1, dtype=torch.int32, device=dev)
            for i, t in enumerate(prompt):
                tok.fill_(int(t))
                dec.step(tok.data_ptr(), i, kv, scratch_logits)
            torch.cuda.synchronize()
        print(f"[bench] prefilled {len(prompt)} tokens in {time.perf_counter() - t_pf:.2f}s", file=sys.stderr,
              flush=True)
        first = torch.empty(1, dtype=torch.int32, device=dev)
        first.copy_(torch.tensor([td.read_device_i32(dec.token_ptr())], dtype=torch.int32))
    st = dec.status()
    if st != 0:
        print(f"device status {st} after prefill", file=sys.stderr)
        return 1

    n_steps = args.steps if args.steps is not None else min(128, cfg.max_ctx - start)
    if start + n_steps > cfg.max_ctx:
        print(f"--steps {n_steps} exceeds the cache ({cfg.max_ctx - start} positions left)", file=sys.stderr)
        return 1
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
    tok_ptr = dec.token_ptr()
    stream = torch.cuda.current_stream()
    spl = max(1, min(args.steps_per_launch, td._lib.TD_MAX_LOOP_STEPS))

    def run(n, record, per_launch=spl, clocks=None):
        """n greedy steps from `first` at positions start.., per_launch steps per
        launch; with `record`, HIP events on the stream around every launch (and,
        with `clocks`, a per-step device clock buffer for each launch).
        Returns [(event pair, steps in the launch, first position)]."""
        evs = []
        i = 0
        while i < n:
            m = min(per_launch, n - i)
            src = first.data_ptr() if i == 0 else tok_ptr
            if clocks is not None:
                dec.set_step_clock(clocks[len(evs)])
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            if per_launch == 1:
                dec.step(src, start + i, kv, logits, stream=stream)
            else:
                dec.loop(src, start + i, m, kv, logits, stream=stream)
            if record:
                e1.record(stream)
                evs.append(((e0, e1), m, start + i))
            i += m
        return evs

    run(min(args.warmup, cfg.max_ctx - start), False)
    torch.cuda.synchronize()
    if dec.status() != 0:
        print("device error during warmup", file=sys.stderr)
        return 1
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    n_launch = (n_steps + spl - 1) // spl
    clocks = [torch.zeros(spl + 1, dtype=torch.int64, device=dev) for _ in range(n_launch)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = run(n_steps, True, clocks=clocks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = None
    if clocks is not None:
        dec.set_step_clock(None)
        d = []
        for c, (_, m, _) in zip(clocks, evs):
            t = c.cpu().numpy()[: m + 1].astype(np.int64)
            d.extend(np.diff(t) * 10.0 / 1e3)  # 100 MHz ticks -> us
        step_us = np.array(d)
    st = dec.status()
    if st != 0:
        print(f"device status {st} during the timed steps", file=sys.stderr)
        return 1
    launch_ms = np.array([a.elapsed_time(b) for (a, b), _, _ in evs])
    total_ms = float(launch_ms.sum())
    tokens_s = n_steps / (total_ms / 1e3)
    launch_bytes = [accounting.mean_step_bytes(cfg, p0, m) * m for _, m, p0 in evs]
    bytes_launch = float(np.mean(launch_bytes))
    kern_ms = float(launch_ms.mean())
    achieved = float(np.sum(launch_bytes)) / (total_ms / 1e3) / 1e9
    if args.trace:
        from decode_persistent_megakernel_amd import trace as tdtrace
        tr = dec.enable_trace(True)
        dec.step(first.data_ptr(), start, kv, logits, stream=stream)
        torch.cuda.synchronize()
        raw = tr.cpu().numpy()
        np.save(os.path.splitext(args.trace)[0] + "_raw.npy", raw)
        summ = tdtrace.summarize(raw, cfg.n_layers, 6 if moe else 5)
        dec.enable_trace(False)
        with open(args.trace, "w") as f:
            json.dump(summ, f, indent=1)
        print(tdtrace.format_summary(summ), file=sys.stderr, flush=True)
    baselines = None
    if args.baseline_steps > 0:
        # the persistent kernel launched once per token (td_decode_step); the same
        # fused ops launched one kernel each, and those launches captured once into
        # a hipGraph and replayed: timed like the headline, per launch
        baselines = {}
        nb = min(args.baseline_steps, n_steps)
        if spl > 1:
            sev = run(nb, True, per_launch=1)
            torch.cuda.synchronize()
            if dec.status() != 0:
                print("device status error in the single-step baseline", file=sys.stderr)
                return 1
            sms = np.array([a.elapsed_time(b) for (a, b), _, _ in sev])
            baselines["single_step_launch"] = {"tokens_per_s": round(nb / (sms.sum() / 1e3), 2),
                                               "ms_per_step": round(float(sms.mean()), 4), "steps": nb,
                                               "launches_per_step": 1}
        for name, ex in (("per_op", td.TD_EXEC_PER_OP), ("graph", td.TD_EXEC_GRAPH)):
            bdec = td.Decoder(dm, cfg.max_ctx, executor=ex)
            bdec.step(first.data_ptr(), start, kv, logits, stream=stream)  # warm-up (and graph capture)
            torch.cuda.synchronize()
            bev = []
            for i in range(nb):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                bdec.step(first.data_ptr() if i == 0 else bdec.token_ptr(), start + i, kv, logits, stream=stream)
                e1.record(stream)
                bev.append((e0, e1))
            torch.cuda.synchronize()
            if bdec.status() != 0:
                print(f"device status error in the {name} baseline", file=sys.stderr)
                return 1
            bms = np.array([a.elapsed_time(b) for a, b in bev])
            baselines[name] = {"tokens_per_s": round(nb / (bms.sum() / 1e3), 2), "ms_per_step": round(float(bms.mean()), 4),
                               "steps": nb,
                               "launches_per_step": (((7 if moe else 6) * cfg.n_layers + 3) if name == "per_op"
                                                     else 2)}
            bdec.close()
            del bdec
    # the stream-read yardstick: a plain read of 2 GiB, 5 timed passes
    ybuf = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    ybuf.fill_(1.0)
    yard = td.measure_stream(ybuf, reps=5, stream=stream)
    del ybuf
    khash = source_hash()
    traffic = read_traffic(args.config, khash)
    if traffic is not None:
        traffic = int(round(traffic * float(np.mean([m for _, m, _ in evs]))))  # per step -> per launch
    cpu = None
    if args.cpu_budget > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(model, cfg, start, args.cpu_budget)
    out = {
        "metric": "batch-1 decode tokens/s (ms/token) and % of MI355X peak HBM GB/s",
        "value": round(tokens_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / n_steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: Llama-style decoder, {cfg.n_layers} layers, hidden {cfg.hidden}, "
                        f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv heads x {cfg.head_dim}, intermediate "
                        f"{cfg.intermediate}, vocab {cfg.vocab}, "
                        + (f"mixture of {cfg.n_experts} experts, top {cfg.top_k}, " if moe else "")
                        + f"{'int4 g64' if cfg.weight_format else 'bf16'} weights, greedy decode at positions "
                        f"{start}..{start + n_steps - 1}, batch 1",
            "weights": "int4-g64+fp16-scales" if cfg.weight_format else "bf16",
            "arithmetic": "fp32 accumulate, fp32 activations, bf16 K/V cache",
            "executor": ((f"persistent megakernel, up to {spl} greedy steps per cooperative launch (in-kernel token loop)"
                          if spl > 1 else "persistent megakernel (one cooperative launch per token)")
                         + (": router, top-k and the chosen experts' rows inside the same launch" if moe else "")),
            "steps_per_launch": sorted({m for _, m, _ in evs}),
            "global_batch": 1,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": ("td_megakernel (" + ", ".join(str(m) for m in sorted({m for _, m, _ in evs}))
                       + " whole decode steps per launch)"),
            "launches": len(evs),
            "algorithmic_bytes_per_launch": int(round(bytes_launch)),
            "kernel_ms_mean": round(kern_ms, 4),
            "kernel_ms_p10": round(float(np.percentile(launch_ms, 10)), 4),
            "kernel_ms_p90": round(float(np.percentile(launch_ms, 90)), 4),
            "step_ms_p10": None if step_us is None else round(float(np.percentile(step_us, 10)) / 1e3, 4),
            "step_ms_p50": None if step_us is None else round(float(np.percentile(step_us, 50)) / 1e3, 4),
            "step_ms_p90": None if step_us is None else round(float(np.percentile(step_us, 90)) / 1e3, 4),
            "step_clock": "in-kernel 100 MHz clock at each step's token decision (first CU)",
            "yardstick_gbps": round(yard, 1),
            "frac_of_yardstick": round(achieved / yard, 4),
            "yardstick": "td_measure_stream: 16-byte non-temporal reads of 2 GiB, one workgroup per CU, 32 KiB contiguous per pass, 5 passes",
            "source_sha256_16": khash,
        },
        "cpu_baseline": cpu,
        "baselines": baselines,
        "prefill": prefill,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out), flush=True)
    # release every device allocation while the runtime is fully up (a profiler
    # attached to the process then has nothing left to tear down at exit)
    dec.close()
    del evs, dec, kv, dm, logits, first, model
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
