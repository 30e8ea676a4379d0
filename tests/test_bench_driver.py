"""The native driver td_bench builds the same workloads as the Python side."""
import dataclasses
import json
import os
import subprocess

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "decode_persistent_megakernel_amd", "td_bench")


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_driver_workload_table_matches_synth(name):
    if not os.path.exists(BENCH):
        pytest.skip("td_bench not built")
    out = subprocess.run([BENCH, "--config", name, "--print-config"], capture_output=True, text=True, check=True)
    got = json.loads(out.stdout)
    want = dataclasses.asdict(synth.CONFIGS[name])
    for k, v in want.items():
        if isinstance(v, float):
            assert got[k] == pytest.approx(v, rel=1e-15), k
        else:
            assert int(got[k]) == int(v) if not isinstance(v, str) else got[k] == v, k
