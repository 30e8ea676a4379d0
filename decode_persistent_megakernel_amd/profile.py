"""rocprofv3 profiles of the decode paths, written as short text summaries.

    python -m decode_persistent_megakernel_amd.profile --config llama1b [--config ...]
           [--what trace,pmc,stages,block] --out profiles --raw <scratch dir>

For each workload (td_bench and bench.py run as child processes; this process
never touches the GPU):

  trace   rocprofv3 --kernel-trace --stats of td_bench: per-kernel time of the
          timed td_decode_loop launches (64 steps each); with --executor graph
          the per-op kernels of the graph executor instead
  pmc     two counter runs, FETCH_SIZE then WRITE_SIZE, each followed in the
          same process by a 1 GiB device-to-device copy whose counter reading
          scales KiB-per-dispatch into bytes; HBM bytes per decode step against
          the algorithmic bytes (accounting.mean_step_bytes)
  stages  the in-kernel stage trace of one decode step (bench.py --trace):
          per stage kind, the critical-path span, the cross-CU hand-off and
          the per-CU work (see trace.py)
  block   the block forward (td_forward_block, 64-token blocks) kernel trace

Each summary states the command that produced it and the sha256 of the
sources it measured; bench.py reads `fetch_bytes_per_step` and
`write_bytes_per_step` back from a traffic summary only while that hash still
matches the sources.  The profiler itself can end with a segmentation fault in
the HIP runtime's exit-time teardown after the program has finished and the
results are written; such a run is used when the program printed its last line
and the database is complete.
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import sqlite3
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
TD_BENCH = os.path.join(PKG, "td_bench")
SHOWN_BENCH = "$REPO/decode_persistent_megakernel_amd/td_bench"
MEGAKERNEL_SOURCES = ("td_api.cpp", "td_internal.h", "td_kernels.hip")
OPS_SOURCES = ("td_api.cpp", "td_internal.h", "td_ops.hip")
BLOCK_SOURCES = ("td_api.cpp", "td_internal.h", "td_block.hip")
CAL_BYTES = 1 << 30  # td_bench --copy-calibration
PEAK_GBS = 8000.0


def sources_hash(names=MEGAKERNEL_SOURCES) -> str:
    """sha256 (first 16 hex digits) over the named csrc files, each prefixed by its name."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _say(*a):
    print("[profile]", *a, flush=True)


def _db(d: str) -> sqlite3.Connection:
    f = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not f:
        raise RuntimeError(f"no rocprofv3 database under {d}")
    return sqlite3.connect(f[0])


def _rocprof(prof_args, prog_args, outdir: str, log: str, timeout: int, last_key: str) -> None:
    """Runs rocprofv3 on td_bench (the program directly after --) from /tmp.
    Accepts the profiler's own exit-time SIGSEGV when the program's last JSON
    line (containing last_key) was printed."""
    outdir = os.path.abspath(outdir)  # the profiler runs from /tmp
    os.makedirs(outdir, exist_ok=True)
    cmd = ["rocprofv3", *prof_args, "-d", outdir, "-o", "run", "--", TD_BENCH, *prog_args]
    env = dict(os.environ, TMPDIR="/tmp")
    with open(log, "w") as f:
        p = subprocess.run(cmd, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT, timeout=timeout)
    text = open(log).read()
    done = any(last_key in line for line in text.splitlines() if line.startswith("{"))
    if p.returncode != 0 and not (p.returncode in (139, -11) and done):
        raise RuntimeError(f"rocprofv3 exited with {p.returncode}; see {log}")
    if not done:
        raise RuntimeError(f"td_bench did not finish; see {log}")
    if p.returncode != 0:
        _say(f"rocprofv3 ended with signal 11 after the program finished ({log}); results are complete")


def _short(name: str) -> str:
    return name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]


def _cfg(name):
    sys.path.insert(0, ROOT)
    import synth
    return synth.CONFIGS[name]


def _step_bytes(cfg, steps):
    from decode_persistent_megakernel_amd import accounting
    return accounting.mean_step_bytes(cfg, cfg.start_pos, steps)


def _cmd_text(prof: str, prog: str) -> str:
    return f"cd /tmp && export TMPDIR=/tmp && rocprofv3 {prof} -d <out> -o run -- {SHOWN_BENCH} {prog}"


# ---------------------------------------------------------------- kernel trace
def trace(name: str, out: str, raw: str, graph: bool = False) -> str:
    cfg = _cfg(name)
    moe = graph  # the per-op kernels (replayed as a graph) instead of the persistent kernel
    if moe:
        steps, warmup, prog = 16, 2, f"--config {name} --executor graph --steps 16 --warmup 2"
    else:
        steps, warmup, loop = min(128, cfg.decode_steps), 8, 64  # the steps must fit the cache
        prog = f"--config {name} --steps {steps} --warmup {warmup} --loop {loop}"
    d = os.path.join(raw, f"kt_{name}")
    _rocprof(["--kernel-trace", "--stats"], prog.split(), d, d + ".log", 400, "ms_per_step")
    c = _db(d)
    per = c.execute("select name, duration from kernels order by start").fetchall()
    alg = _step_bytes(cfg, steps)
    if moe:
        path = os.path.join(out, f"graph_{name}_kernel_trace.txt")
        ops = [(_short(n), du) for n, du in per if "op_" in n]
        if not cfg.n_experts:
            raise RuntimeError("the graph-executor trace summary is written for mixture-of-experts workloads")
        begins = [i for i, (n, _) in enumerate(ops) if n == "op_begin"]
        timed = ops[begins[-steps]:]
        agg = collections.OrderedDict()
        for n, du in timed:
            agg.setdefault(n, []).append(du)
        tot = sum(du for _, du in timed) / 1e3 / steps
        lines = [f"# decode step of {name} ({cfg.n_layers} layers, {cfg.n_experts} experts of {cfg.intermediate}, "
                 f"top {cfg.top_k}) on the graph executor (per-op kernels replayed as one hipGraph): "
                 "rocprofv3 kernel trace",
                 "command: " + _cmd_text("--kernel-trace --stats", prog),
                 f"per-dispatch query: select name, duration from kernels order by start (the last {steps} steps, "
                 f"positions {cfg.start_pos}..{cfg.start_pos + steps - 1})",
                 f"sources_sha256_16 ({', '.join(OPS_SOURCES)}): {sources_hash(OPS_SOURCES)}", "",
                 f"{'kernel':16} {'calls/step':>10} {'avg_us':>9} {'us/step':>9}"]
        for n, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{n:16} {len(v) / steps:10.1f} {sum(v) / len(v) / 1e3:9.2f} {sum(v) / 1e3 / steps:9.1f}")
        lines += ["", f"kernel time per step: {tot:.1f} us", f"algorithmic_bytes_per_step: {alg:.0f}",
                  f"achieved_GBps (over kernel time): {alg / (tot * 1e-6) / 1e9:.1f}",
                  f"frac_of_8TBps: {alg / (tot * 1e-6) / 1e9 / PEAK_GBS:.4f}"]
        H, I, k = cfg.hidden, cfg.intermediate, cfg.top_k
        for op, b in (("op_moe_gu", k * 2 * I * H * 2), ("op_moe_down", k * H * I * 2)):
            if op in agg:
                us = sum(agg[op]) / len(agg[op]) / 1e3
                lines.append(f"{op}: {b} routed weight bytes / {us:.2f} us = {b / us / 1e3:.0f} GB/s "
                             f"({b / us / 1e3 / PEAK_GBS:.3f} of 8000 GB/s)")
    else:
        path = os.path.join(out, f"megakernel_{name}_kernel_trace.txt")
        rows = c.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
        mk = [du for n, du in per if "td_megakernel" in n]
        nl = (steps + loop - 1) // loop
        t = sorted(mk[-nl:])
        mean = sum(t) / len(t) / 1e3
        nwl = (warmup + loop - 1) // loop
        lines = [f"# td_megakernel, workload {name}: rocprofv3 kernel trace",
                 "command: " + _cmd_text("--kernel-trace --stats", prog),
                 "summary query: select name, total_calls, total_duration, average, percentage from top_kernels; "
                 "per-dispatch: select name, duration from kernels order by start",
                 f"source_sha256_16: {sources_hash()}", "",
                 f"{'kernel':60} {'calls':>7} {'total_us':>12} {'avg_us':>10} {'pct':>6}"]
        for n, calls, tot, avg, pct in rows:
            lines.append(f"{n[:60]:60} {calls:7d} {tot:12.1f} {avg:10.2f} {pct:6.2f}")
        lines += ["",
                  f"td_megakernel dispatches: {len(mk)} = {cfg.prompt_len} prompt steps (one step each) + {nwl} "
                  f"warmup ({warmup} steps) + {nl} timed ({loop} steps each)",
                  f"timed dispatches (last {nl}): mean {mean:.1f} us, min {t[0] / 1e3:.1f}, max {t[-1] / 1e3:.1f}",
                  f"timed_us_per_dispatch: {mean:.1f}", f"steps_per_dispatch: {loop}",
                  f"timed_us_per_step: {mean / loop:.2f}",
                  f"positions: {cfg.start_pos}..{cfg.start_pos + steps - 1}",
                  f"algorithmic_bytes_per_step: {alg:.0f}",
                  f"achieved_GBps: {alg / (mean / loop * 1e-6) / 1e9:.1f}",
                  f"frac_of_8TBps: {alg / (mean / loop * 1e-6) / 1e9 / PEAK_GBS:.4f}"]
    open(path, "w").write("\n".join(lines) + "\n")
    return path


# ---------------------------------------------------------------- HBM counters
def pmc(name: str, out: str, raw: str, graph: bool = False) -> str:
    cfg = _cfg(name)
    moe = graph
    if moe:
        steps, prog = 16, f"--config {name} --executor graph --steps 16 --warmup 2 --copy-calibration"
    else:
        steps = min(64, cfg.decode_steps)
        prog = f"--config {name} --steps {steps} --warmup 8 --loop 64 --copy-calibration"
    vals = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(raw, f"{counter.lower()}_{name}")
        _rocprof(["--pmc", counter], prog.split(), d, d + ".log", 240, "copy_calibration_bytes")
        r = _db(d).execute("select dispatch_id, kernel_name, value from counters_collection "
                           "order by dispatch_id").fetchall()
        cal = [v for _, n, v in r if "copyBuffer" in n][-1]
        if moe:
            ops = [(_short(n), v) for _, n, v in r if "op_" in n]
            begins = [i for i, (n, _) in enumerate(ops) if n == "op_begin"]
            kib = sum(v for _, v in ops[begins[-steps]:])
        else:
            kib = [v for _, n, v in r if "td_megakernel" in n][-1]
        vals[counter] = (kib, cal)
    (fr, fc), (wr, wc) = vals["FETCH_SIZE"], vals["WRITE_SIZE"]
    fs, ws = CAL_BYTES / 1024 / fc, CAL_BYTES / 1024 / wc
    fb, wb = fr * 1024 * fs / steps, wr * 1024 * ws / steps
    alg = _step_bytes(cfg, steps)
    kind = "graph" if moe else "megakernel"
    srcs = OPS_SOURCES if moe else MEGAKERNEL_SOURCES
    what = (f"the per-op kernels of the last {steps} steps (graph executor), summed" if moe else
            f"the last td_megakernel dispatch: {steps} decode steps")
    lines = [f"# {'per-op decode kernels' if moe else 'td_megakernel'}, workload {name}: HBM traffic from "
             "hardware counters",
             "command_FETCH_SIZE: " + _cmd_text("--pmc FETCH_SIZE", prog),
             "command_WRITE_SIZE: " + _cmd_text("--pmc WRITE_SIZE", prog),
             "query: select dispatch_id, kernel_name, value from counters_collection order by dispatch_id "
             f"(value in KiB per dispatch; measured: {what} at positions {cfg.start_pos}..{cfg.start_pos + steps - 1}; "
             "scale: the last __amd_rocclr_copyBuffer dispatch, a 1 GiB device-to-device copy)",
             f"source_sha256_16: {sources_hash(srcs)}" + ("" if not moe else f" ({', '.join(srcs)})"),
             f"steps_measured: {steps}",
             f"fetch_kib_raw: {fr:.1f}", f"write_kib_raw: {wr:.1f}",
             f"calibration_copy_bytes: {CAL_BYTES}", f"calibration_fetch_kib_raw: {fc:.1f}",
             f"calibration_write_kib_raw: {wc:.1f}",
             f"fetch_scale: {fs:.5f}", f"write_scale: {ws:.5f}",
             f"fetch_bytes_per_step: {fb:.0f}", f"write_bytes_per_step: {wb:.0f}",
             f"algorithmic_bytes_per_step: {alg:.0f}", f"traffic_over_algorithmic: {(fb + wb) / alg:.4f}"]
    path = os.path.join(out, f"{kind}_{name}_traffic.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    return path


# ---------------------------------------------------------------- stage trace
def stages(name: str, out: str, raw: str) -> str:
    from decode_persistent_megakernel_amd import trace as tdtrace
    cfg = _cfg(name)
    js = os.path.join(raw, f"stages_{name}.json")
    args = ["--config", name, "--steps", "16", "--warmup", "4", "--cpu-budget", "0", "--baseline-steps", "0",
            "--trace", js]
    log = os.path.join(raw, f"stages_{name}.log")
    with open(log, "w") as f:
        p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, stdout=f,
                           stderr=subprocess.STDOUT, timeout=400)
    if p.returncode != 0:
        raise RuntimeError(f"bench.py --trace exited with {p.returncode}; see {log}")
    s = json.load(open(js))
    lines = [f"# td_megakernel, workload {name}: in-kernel stage trace of one decode step (td_set_trace)",
             "command: python -u bench.py " + " ".join(args[:-1]) + " <out>.json",
             f"(one td_decode_step launch at position {cfg.start_pos}, after the timed loop; 100 MHz device clock)",
             f"source_sha256_16: {sources_hash()}",
             "span: critical-path time the stage adds (last output of the previous stage to the last output of this "
             "one, over all CUs); hoff: last output of the previous stage to a CU's inputs staged (min, median over "
             "CUs); work: a CU's inputs staged to its last output (median, max over CUs); averaged over the layers; "
             "us", "", tdtrace.format_summary(s)]
    per_layer = sum(v["span_us"] for k, v in s["stages"].items() if k != "head")
    lines.append(f"per layer (sum of the layer's stage spans): {per_layer:.2f} us")
    path = os.path.join(out, f"megakernel_{name}_stage_trace.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    return path


# ---------------------------------------------------------------- block forward
def _gemm_tile_rows(kernel: str) -> int:
    """Weight rows per workgroup of a block GEMM instance, from its template
    arguments: blk_gemm<FMT, MT, NB, NORM> takes 64 NB, blk_gemm_stream<NT, XC,
    NORM> 16 NT."""
    args = [a.strip() for a in kernel.split("<", 1)[1].rstrip(">").split(",")]
    return 16 * int(args[0]) if kernel.startswith("blk_gemm_stream") else 64 * int(args[2])


def block(name: str, out: str, raw: str) -> str:
    cfg = _cfg(name)
    prog = f"--config {name} --block 64 --steps 4 --warmup 1"
    d = os.path.join(raw, f"blk_{name}")
    _rocprof(["--kernel-trace", "--stats"], prog.split(), d, d + ".log", 400, "ms_per_step")
    rows = _db(d).execute("select name, grid_x, workgroup_x, grid_y, duration from kernels order by start").fetchall()
    blk = [r for r in rows if "blk_" in r[0]]
    nblocks = sum(1 for r in blk if "blk_embed" in r[0])
    agg = collections.OrderedDict()
    for n, gx, wx, gy, du in blk:
        key = (_short(n), gx // max(wx, 1), gy)  # grid_x in workgroups
        agg.setdefault(key, []).append(du)
    H, I, V, d_ = cfg.hidden, cfg.intermediate, cfg.vocab, cfg.head_dim
    qkv_rows = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d_
    eb = 2 if cfg.weight_format == 0 else 0.5
    shapes = {qkv_rows: ("QKV", qkv_rows * H), 2 * I: ("gate/up", 2 * I * H), V: ("logits", V * H)}
    seen_h = []
    role = {}
    for (k, gx, gy) in agg:
        if "gemm" not in k:
            continue
        tile = _gemm_tile_rows(k)
        hit = [n for n in shapes if -(-n // tile) == gx]
        if hit:
            role[(k, gx, gy)] = shapes[hit[0]]
        elif -(-H // tile) == gx:  # O, then down, in a layer's launch order
            seen_h.append((k, gx, gy))
            role[(k, gx, gy)] = ("O", H * cfg.n_q_heads * d_) if len(seen_h) == 1 else ("down", H * I)
    lines = [f"# block forward (td_forward_block), workload {name}: rocprofv3 kernel trace",
             "command: " + _cmd_text("--kernel-trace --stats", prog),
             f"(the {cfg.prompt_len}-token prompt in 64-token blocks: one untimed and three timed passes = "
             f"{nblocks} block calls; the decode launches that follow are not listed)",
             "per-dispatch query: select name, grid_x, workgroup_x, grid_y, duration from kernels order by start",
             f"sources_sha256_16 ({', '.join(BLOCK_SOURCES)}): {sources_hash(BLOCK_SOURCES)}", "",
             f"{'kernel':26} {'grid (wg)':>12} {'calls':>6} {'avg_us':>9} {'us/block':>9}  role"]
    tot = 0.0
    for key, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        s = sum(v) / 1e3
        tot += s
        r = role.get(key)
        lines.append(f"{key[0]:26} {f'({key[1]},{key[2]})':>12} {len(v):6d} {s / len(v):9.2f} {s / nblocks:9.1f}  "
                     f"{r[0] + ' GEMM' if r else ''}")
    lines += ["", f"sum of kernel time per 64-token block: {tot / nblocks:.1f} us "
                  f"({64 / (tot / nblocks * 1e-6):.0f} tokens/s)"]
    for key, (rname, n_w) in role.items():
        us = sum(agg[key]) / len(agg[key]) / 1e3
        b = n_w * (2 if rname == "logits" else eb)  # the output head is bf16 in every format
        lines.append(f"{rname} GEMM: {b:.0f} weight bytes per call / {us:.2f} us = {b / us / 1e3:.0f} GB/s "
                     f"({b / us / 1e3 / PEAK_GBS:.3f} of 8000 GB/s)")
    path = os.path.join(out, f"block_{name}_kernel_trace.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    return path


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", action="append", required=True)
    ap.add_argument("--what", default="trace,pmc,stages")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--raw", required=True, help="directory for the profiler's databases and logs")
    ap.add_argument("--executor", default="megakernel", choices=["megakernel", "graph"],
                    help="graph: a mixture-of-experts workload's per-op kernels replayed as a graph")
    a = ap.parse_args(argv)
    os.makedirs(a.out, exist_ok=True)
    os.makedirs(a.raw, exist_ok=True)
    graph = a.executor == "graph"
    fns = {"trace": lambda n, o, r: trace(n, o, r, graph), "pmc": lambda n, o, r: pmc(n, o, r, graph),
           "stages": stages, "block": block}
    for name in a.config:
        moe = bool(_cfg(name).n_experts)
        for w in a.what.split(","):
            if (moe and w == "block") or (graph and w in ("stages", "block")):
                continue  # no block forward for MoE; no stage trace off the persistent kernel
            _say(f"{name}: {w}")
            path = fns[w](name, a.out, a.raw)
            _say(f"{name}: {w} -> {os.path.relpath(path, ROOT)}")
            print(open(path).read(), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
