"""Builds libtd.so (the HIP library behind include/td.h) in-tree for gfx950, and
td_bench, the native driver of the decode step (linked to libtd.so and libsynth.so)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SO = os.path.join(PKG, "libtd.so")
BENCH = os.path.join(PKG, "td_bench")
SYNTH_DIR = os.path.join(ROOT, "synth")
SOURCES = ["td_kernels.hip", "td_ops.hip", "td_block.hip", "td_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17",
         # packed fp32 instructions stay off: ordinary float code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # no implicit a*b+c contraction: every fused multiply-add is an explicit
         # fmaf, so the persistent kernel and the per-op kernels round alike
         "-ffp-contract=off",
         "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compiles each source to an object in parallel (each carries its own
    device code), then links libtd.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    objs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", *inc, "-o", obj, os.path.join(CSRC, s)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = False
    for s, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed to compile libtd.so's sources")
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to link libtd.so")
    os.replace(tmp, SO)
    build_bench(verbose)
    return SO


def build_bench(verbose: bool = False) -> str:
    """td_bench: host-only C++ against the C ABI; needs synth/libsynth.so built."""
    synth_so = os.path.join(SYNTH_DIR, "libsynth.so")
    if not os.path.exists(synth_so):
        sys.path.insert(0, ROOT)
        import synth
        synth.build()
    tmp = BENCH + ".tmp"
    cmd = [HIPCC, "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), "-o", tmp,
           os.path.join(CSRC, "td_bench.cpp"), "-L", PKG, "-ltd", "-L", SYNTH_DIR, "-lsynth",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,$ORIGIN/../synth"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build td_bench")
    os.replace(tmp, BENCH)
    return BENCH


if __name__ == "__main__":
    print(build(verbose=True))
