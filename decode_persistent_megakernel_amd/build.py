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
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
         # packed fp32 instructions stay off: ordinary float code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # no implicit a*b+c contraction: every fused multiply-add is an explicit
         # fmaf, so the persistent kernel and the per-op kernels round alike
         "-ffp-contract=off",
         "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libtd.so")
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
