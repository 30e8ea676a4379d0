"""The per-op and graph executors: the same arithmetic as the persistent
kernel, one launch per fused op (and the same launches captured once into a
hipGraph and replayed).  They must agree with the oracle like the persistent
kernel, and with the persistent kernel bit for bit: every GEMV row, norm,
attention tile, merge and argmax is computed by the same routine in the same
order.  Graph replays are interleaved with eager steps and host
synchronisations, and every replay is checked."""
import numpy as np
import pytest

import synth
from tests.test_gpu_parity import run_compare, td, torch, _say  # noqa: F401  (fixture)
from tests.test_gpu_edges import SPLITK, SPLITK128, RAGGED4, MHA64, MHA128

pytestmark = pytest.mark.gpu

MEGA, PER_OP, GRAPH = 0, 1, 2


def _steps(td, cfg, model, k, v, first, start, n, executor, eager_between=False):
    """Greedy steps from a K/V state; returns the logits bits and tokens per step."""
    dm = td.DeviceModel(model)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx, executor=executor)
    tok = torch.tensor([int(first)], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    outs, toks = [], []
    for i in range(n):
        dec.step(tok.data_ptr() if i == 0 else dec.token_ptr(), start + i, kv, logits)
        if eager_between:
            scratch = torch.arange(4096, device="cuda", dtype=torch.float32)
            _ = (scratch * 2).sum().item()  # eager work and a host sync between replays
        torch.cuda.synchronize()
        assert dec.status() == 0
        outs.append(logits.cpu().numpy().view(np.uint32).copy())
        toks.append(td.read_device_i32(dec.token_ptr()))
    dec.close()
    return outs, toks


# 8 kv heads over a 4096-position cache: 128-position chunks (two tiles each)
# and, at position 2100, 17 chunks to merge
MULTITILE = synth.shrink(SPLITK, name="multitile", n_q_heads=16, n_kv_heads=8, max_ctx=4096, seed=2004)


@pytest.mark.parametrize("cfg,start,n", [(SPLITK, 60, 12), (SPLITK128, 120, 12), (RAGGED4, 40, 8),
                                         (MULTITILE, 2100, 6), (MHA64, 20, 8), (MHA128, 120, 8)],
                         ids=["d64", "d128_bias", "int4", "multitile", "mha_d64", "mha_d128"])
def test_executors_agree_bit_for_bit(td, cfg, start, n):
    _say(f"executors on {cfg.name}")
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, start, seed_tag="exec")
    ref_l, ref_t = _steps(td, cfg, m, k, v, synth.first_token(cfg), start, n, MEGA)
    for ex in (PER_OP, GRAPH):
        got_l, got_t = _steps(td, cfg, m, k, v, synth.first_token(cfg), start, n, ex, eager_between=(ex == GRAPH))
        assert got_t == ref_t, (ex, got_t, ref_t)
        for i, (a, b) in enumerate(zip(got_l, ref_l)):
            assert np.array_equal(a, b), (ex, i, int(np.sum(a != b)))


def test_per_op_matches_oracle_fullsize_llama(td):
    cfg = synth.CONFIGS["llama1b"]
    _say("per-op executor, llama1b, 8 steps from a random 512-position prefix")
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, cfg.start_pos)
    run_compare(td, cfg, m, k, v, synth.first_token(cfg), cfg.start_pos, 8, 2e-2, "llama1b/per-op", executor=PER_OP)


def test_graph_matches_oracle_fullsize_long_int4(td):
    cfg = synth.CONFIGS["llama1b_int4_long"]
    _say("graph executor, llama1b_int4_long, 4 steps at 8192")
    m = synth.make_model(cfg)
    k, v = synth.kv_cache(cfg)
    run_compare(td, cfg, m, k, v, synth.first_token(cfg), cfg.start_pos, 4, 5e-2, "long/graph", executor=GRAPH)
