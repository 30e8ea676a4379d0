"""The kernels issue some global loads with inline assembly and wait for them
with their own counted s_waitcnt.  The compiler sees such a load's result as
written when the asm statement issues, so if the result is dead (never read) it
may hand those registers to another value while the load is still in flight,
and the late data then corrupts that value (an address, say).  This test builds
the device code to assembly and checks, within each basic block, that no
register an asm load writes is overwritten before it is read or before a
vmcnt(0) wait, and that none is read (a copy the compiler makes of the value,
say) before any counted wait.  Dword loads and the 16-bit loads of the QKV
biases are covered.  CPU only: hipcc cross-compiles for gfx950."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_persistent_megakernel_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=off", "-Wno-unused-function", "--cuda-device-only", "-S"]

NO_VGPR_DEST = ("global_store", "ds_write", "buffer_store", "global_load_lds", "scratch_store", "s_", "ds_add",
                "global_atomic", "buffer_atomic")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def check_asm(text):
    """Returns (asm loads seen, list of findings) for one assembly file."""
    findings, seen = [], 0
    for fn in re.split(r"\n(?=_Z\S+:)", text):
        name = fn.split(":", 1)[0].strip()
        ins, in_asm = [], False
        for raw in fn.split("\n"):
            line = raw.strip()
            if line.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if line.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not line or line.startswith(";") or (line.startswith(".") and not line.startswith(".LBB")):
                continue
            if line.startswith(".LBB") or line.startswith("s_cbranch") or line.startswith("s_branch"):
                ins.append(("<block>", False))
                continue
            ins.append((line, in_asm))
        for i, (line, from_asm) in enumerate(ins):
            if not from_asm or not re.match(r"(global|buffer)_load_(dword(x2|x3|x4)?|ushort|ubyte|sshort|sbyte)\s", line):
                continue
            seen += 1
            dest = _regs(line.split(None, 1)[1].split(",")[0].strip())
            waited = False  # a counted wait (any vmcnt) seen since the load
            for later, _ in ins[i + 1:]:
                if later == "<block>" or later.startswith("s_waitcnt vmcnt(0)"):
                    break
                if later.startswith("s_waitcnt") and "vmcnt" in later:
                    waited = True
                parts = later.split(None, 1)
                if len(parts) < 2:
                    continue
                op, ops = parts[0], [o.strip() for o in parts[1].split(",")]
                srcs = ops if op.startswith(NO_VGPR_DEST) else ops[1:]
                if set().union(*[_regs(o) for o in srcs]) & dest:
                    if not waited:  # e.g. a copy the compiler made of the not yet loaded value
                        findings.append(f"{name[:80]}: '{line}' read by '{later}' before any wait")
                    break
                if not op.startswith(NO_VGPR_DEST) and _regs(ops[0]) & dest:
                    findings.append(f"{name[:80]}: '{line}' overwritten by '{later}' before it is read")
                    break
    return seen, findings


def test_checker_flags_a_dead_or_early_read_destination():
    bad = """_Zk:
\t;;#ASMSTART
\tglobal_load_dwordx4 v[0:3], v[4:5], off
\t;;#ASMEND
\tv_lshl_add_u64 v[0:1], v[8:9], 0, s[4:5]
\tglobal_load_lds_dwordx4 v[0:1], off
"""
    good = """_Zk:
\t;;#ASMSTART
\tglobal_load_dwordx4 v[0:3], v[4:5], off
\t;;#ASMEND
\ts_waitcnt vmcnt(2)
\tv_add_f32_e32 v6, v0, v1
\tv_lshl_add_u64 v[0:1], v[8:9], 0, s[4:5]
"""
    copied = """_Zk:
\t;;#ASMSTART
\tglobal_load_ushort v2, v[4:5], off
\t;;#ASMEND
\tv_mov_b32_e32 v7, v2
\ts_waitcnt vmcnt(0)
"""
    assert check_asm(bad)[1] and check_asm(bad)[0] == 1
    assert check_asm(good) == (1, [])
    assert check_asm(copied)[0] == 1 and "before any wait" in check_asm(copied)[1][0]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src,min_loads", [("td_block.hip", 100), ("td_kernels.hip", 20)])
def test_no_asm_load_destination_is_reused_in_flight(tmp_path, src, min_loads):
    out = tmp_path / (src + ".s")
    r = subprocess.run([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(out),
                        os.path.join(CSRC, src)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    seen, findings = check_asm(out.read_text())
    assert seen >= min_loads, seen
    assert not findings, "\n".join(findings[:10])
