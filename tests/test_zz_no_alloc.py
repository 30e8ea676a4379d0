"""td_decode_step_noalloc, the entry point for callers that cannot allocate,
against the entry point it varies: td_decode_step on a TD_EXEC_PER_OP context
(the same per-op kernels).  Both must give the same logits bits, the same
greedy token, the same K/V rows and the same error word.  Two calls in a row
share the library's fixed scratch array: a 20-layer model (two launches of
the layer-table setup) and then a smaller one, so a stale table entry, RoPE
row or activation from the first call would show in the second.  A config
that needs more scratch than the array holds is refused before any launch."""
import ctypes

import numpy as np
import pytest

import synth
from tests.test_gpu_parity import td, torch, _say  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

BIG = synth.shrink(synth.CONFIGS["llama1b"], name="noalloc_big", n_layers=20, hidden=256, n_q_heads=8, n_kv_heads=2,
                   head_dim=64, intermediate=512, vocab=5000, max_ctx=256, prompt_len=0, kv_prefix=0,
                   decode_steps=0, seed=3001)
SMALL = synth.CONFIGS["tiny"]
QWENISH = synth.shrink(synth.CONFIGS["qwen1p5b"], name="noalloc_d128", n_layers=3, hidden=256, n_q_heads=4,
                       n_kv_heads=2, head_dim=128, intermediate=512, vocab=3000, max_ctx=200, prompt_len=0,
                       kv_prefix=0, decode_steps=0, seed=3002)


def _per_op(td, cfg, m, k, v, token, pos):
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx, executor=td.TD_EXEC_PER_OP)
    tok = torch.tensor([token], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    dec.step(tok.data_ptr(), pos, kv, logits)
    torch.cuda.synchronize()
    st = dec.status()
    out = (logits.cpu().numpy().view(np.uint32).copy(), td.read_device_i32(dec.token_ptr()), st, *kv.host())
    dec.close()
    return out


def _noalloc(td, cfg, m, k, v, token, pos):
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    tok = torch.tensor([token], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    tok_out = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    err = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    td.decode_step_noalloc(dm, cfg.max_ctx, tok.data_ptr(), pos, kv, logits, tok_out, err)
    torch.cuda.synchronize()
    return (logits.cpu().numpy().view(np.uint32).copy(), int(tok_out.item()), int(err.item()), *kv.host())


def _compare(td, cfg, pos, seed_tag, nan_row=None):
    m = synth.make_model(cfg)
    if nan_row is not None:
        m.head = m.head.copy() if not cfg.tied else m.head
        m.head[nan_row, :] = 0x7FC0  # bf16 NaN: that logit is NaN
    k, v = synth.random_kv_prefix(cfg, pos, seed_tag=seed_tag)
    token = synth.first_token(cfg)
    ref_l, ref_t, ref_st, ref_k, ref_v = _per_op(td, cfg, m, k, v, token, pos)
    got_l, got_t, got_err, got_k, got_v = _noalloc(td, cfg, m, k, v, token, pos)
    assert np.array_equal(got_l, ref_l), int(np.sum(got_l != ref_l))
    assert got_t == ref_t
    assert np.array_equal(got_k, ref_k) and np.array_equal(got_v, ref_v)
    return ref_st, got_err


def test_noalloc_step_equals_per_op_step_twice(td):
    _say("no-allocation step: 20-layer model, then the tiny model")
    st, err = _compare(td, BIG, 120, "noalloc1")
    assert st == 0 and err == 0
    st, err = _compare(td, SMALL, 9, "noalloc2")
    assert st == 0 and err == 0


def test_noalloc_step_head_dim_128_bias_and_nonfinite(td):
    from decode_persistent_megakernel_amd import _lib
    _say("no-allocation step: d = 128 with bias; a NaN logit")
    st, err = _compare(td, QWENISH, 150, "noalloc3")
    assert st == 0 and err == 0
    cfg = synth.shrink(SMALL, tied=False)
    st, err = _compare(td, cfg, 5, "noalloc4", nan_row=7)
    assert st == _lib.TD_E_NONFINITE and err == 1


def test_noalloc_refuses_a_config_beyond_its_scratch(td):
    from decode_persistent_megakernel_amd import _lib
    # a vocabulary of 32M rows needs 8 MiB of greedy candidates alone
    cfg = _lib.TdConfig(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
                        vocab=32 << 20, max_ctx=16, rope_theta=1e4, rms_eps=1e-5, weight_format=0, qkv_bias=0)
    fake = 1 << 20  # never dereferenced: the size check comes before any launch
    layer = (_lib.TdLayerWeights * 1)()
    layer[0] = _lib.TdLayerWeights(attn_norm=fake, w_qkv=fake, w_o=fake, mlp_norm=fake, w_gu=fake, w_d=fake)
    w = _lib.TdWeights(embed=fake, final_norm=fake, head=fake, layers=layer)
    kvbuf = torch.zeros(2 * 16 * 64, dtype=torch.int16, device="cuda")
    kv = _lib.TdKV(k=kvbuf.data_ptr(), v=kvbuf.data_ptr(), max_ctx=16)
    rc = _lib.lib().td_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(w), fake, 0, ctypes.byref(kv), fake, fake,
                                           fake, None)
    assert rc == _lib.TD_E_UNSUPPORTED
    assert "scratch" in _lib.last_error()
