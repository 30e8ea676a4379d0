"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the persistent kernel behind td_decode_step).

The long prompts (512 / 256 / 1024 tokens) would take the CPU oracle minutes to
prefill, so a seeded random bf16 K/V prefix of the same length (N(0, 1), the
scale of the projected keys of these random-init models) stands in for the
prefilled cache; the long-context stress case uses its own random prefix of
8192 positions.  Both sides decode 32 greedy steps from the same cache state,
teacher-forced with the oracle's tokens, and every step's logits (all V of
them) and greedy token are compared.
"""
import sys

import pytest

import synth
from tests.test_gpu_parity import run_compare, td  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

TOL = {synth.WF_BF16: 2e-2, synth.WF_INT4_G64: 5e-2}


@pytest.mark.parametrize("name", ["llama1b", "tinyllama_int4", "qwen1p5b", "llama1b_int4_long"])
def test_fullsize_decode_matches_oracle(td, name):  # noqa: F811
    cfg = synth.CONFIGS[name]
    print(f"{name}: generating the model", flush=True)
    m = synth.make_model(cfg)
    if cfg.kv_prefix:
        k, v = synth.kv_cache(cfg)
    else:
        k, v = synth.random_kv_prefix(cfg, cfg.start_pos)
    print(f"{name}: 32 teacher-forced steps from position {cfg.start_pos}", flush=True)
    sys.stdout.flush()
    run_compare(td, cfg, m, k, v, synth.first_token(cfg), cfg.start_pos, 32, TOL[cfg.weight_format], name)
