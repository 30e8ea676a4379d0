"""The block forward (td_forward_block): n tokens of one sequence in one pass
over the weights, the prefill / draft-verify path whose linears run as
matrix-core GEMMs.

Row i of the block must be what the oracle's decode step computes for token i
at position pos0 + i, given the same K/V cache before pos0 (teacher forcing:
both sides see the same tokens).  Compared: every row's logits (all V of them)
within the decode-step tolerance (2e-2 for bf16 weights, 5e-2 for int4), every
row's greedy token (a flip is allowed only where the oracle's top-2 gap is
below twice the observed error), and the K/V rows the block writes (within one
bf16 ulp of the oracle's, rarely differing at all), with the rows before pos0
and after the block untouched.

Shapes: the tiny model's whole prompt from position 0; the split-K model across
the 63/64 chunk edge; head dim 128 with a QKV bias and 40 rows (three 16-row
MFMA tiles, a ragged last one); int4 with a ragged K (intermediate 640) and 33
rows; the largest block (64 rows) over 2000 cached positions; a single row.
At full size against the oracle: Llama-3.2-1B (bf16) and TinyLlama (int4), 16
rows at position 100; Qwen2.5-1.5B (d = 128, bias), 24 rows at 1000; the
long-context int4 Llama shape, 33 rows at 8192; and 64 rows against 64 greedy
decode steps of the megakernel (a verify of the megakernel's own draft accepts
every token).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.test_gpu_parity import bf16_to_f64, td, torch, _say  # noqa: F401  (fixture)
from tests.test_gpu_edges import SPLITK, SPLITK128, RAGGED4
from tests.test_gpu_executors import MULTITILE

pytestmark = pytest.mark.gpu

TOL = {synth.WF_BF16: 2e-2, synth.WF_INT4_G64: 5e-2}


def _tokens(cfg, n, tag="block"):
    return synth.i32_uniform(n, synth.key(cfg.seed, -1, tag), cfg.vocab)


def _block(td, cfg, m, k, v, toks, pos0, all_logits=True):
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    n = len(toks)
    t = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    logits = torch.full((n if all_logits else 1, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((n if all_logits else 1,), -7, dtype=torch.int32, device="cuda")
    dec.forward_block(t, pos0, kv, logits, all_logits=all_logits, argmax=am)
    torch.cuda.synchronize()
    st = dec.status()
    word = td.read_device_i32(dec.token_ptr())
    out = (logits.cpu().numpy().astype(np.float64), am.cpu().numpy().tolist(), word, st) + kv.host()
    dec.close()
    return out


def _kv_close(a2, b2, label, atol_rel=2 ** -12):
    """Block K/V rows against reference rows, both bf16 (as float64).

    The block's pre-rounding values carry fp32-level errors that the matrix
    unit makes larger than the decode step's: it sums each MFMA's 32 products
    toward zero at about fp32 precision relative to the largest product (a
    measured property of v_mfma_f32_16x16x32_bf16), and these errors pass
    through the layers.  So: within one bf16 ulp, plus an absolute allowance
    of 2^-12 of the tensor's largest value where the projection cancels to
    near zero (still far below a wrong term, head or position, which moves
    values by O(0.1)); and at most 5% of the entries one ulp apart at all."""
    np.testing.assert_allclose(a2, b2, rtol=2 ** -7, atol=atol_rel * np.abs(b2).max(), err_msg=label)
    frac = float(np.mean(a2 != b2))
    assert frac < 0.05, (label, frac)
    return frac


def _check_kv(gk, gv, ok, ov, k0, v0, pos0, n, label, atol_rel=2 ** -12):
    lo, hi = pos0, pos0 + n
    for a, b in ((gk, ok), (gv, ov)):
        frac = _kv_close(bf16_to_f64(a[:, :, lo:hi]), bf16_to_f64(b[:, :, lo:hi]), label, atol_rel)
        _say(f"{label}: K/V entries one bf16 ulp from the oracle's: {100 * frac:.2f}%")
    for a, b in ((gk, k0), (gv, v0)):
        assert np.array_equal(a[:, :, :lo], b[:, :, :lo]), (label, "rows before pos0 changed")
        assert np.array_equal(a[:, :, hi:], b[:, :, hi:]), (label, "rows after the block changed")


def _compare(td, cfg, m, k, v, toks, pos0, label, kv_atol_rel=2 ** -12):
    n = len(toks)
    _say(f"{label}: block of {n} rows at position {pos0}")
    got, am, word, st, gk, gv = _block(td, cfg, m, k, v, toks, pos0)
    assert st == 0, (label, st)
    o = oracle.Oracle(m)
    o.set_kv(k, v)
    tol = TOL[cfg.weight_format]
    worst, min_gap = 0.0, math.inf
    for i, t in enumerate(toks):
        r, ref = o.step(int(t), pos0 + i)
        assert r >= 0
        diff = float(np.max(np.abs(got[i] - ref)))
        worst = max(worst, diff)
        assert diff <= tol, (label, i, diff)
        top2 = np.sort(ref)[-2:]
        gap = top2[1] - top2[0]
        min_gap = min(min_gap, gap)
        if am[i] != r:
            assert gap <= 2 * diff, (label, i, am[i], r, gap, diff)
        assert am[i] == int(np.argmax(got[i])), (label, i)  # lowest id among equal values
    assert word == am[-1]
    _check_kv(gk, gv, o.k, o.v, k, v, pos0, n, label, kv_atol_rel)
    _say(f"{label}: max|dlogit| = {worst:.3g}, min top-2 gap = {min_gap:.3g}")


MHA1 = synth.shrink(SPLITK, name="mha_d64", n_q_heads=4, n_kv_heads=4, seed=2011)
MHA1_LONG = synth.shrink(MHA1, name="mha_d64_long", max_ctx=2304, seed=2012)


@pytest.mark.parametrize("cfg,pos0,n", [
    (SPLITK, 58, 20),        # positions 58..77 across the 63/64 edge, two 16-row tiles
    (SPLITK128, 100, 40),    # d = 128 + bias, three tiles (the last ragged), across 127/128
    (RAGGED4, 40, 33),       # int4, K = 640 in the down projection, 33 rows
    (MULTITILE, 2000, 64),   # the largest block over 2000 cached positions
    (SPLITK, 0, 1),          # a single row at position 0
    (SPLITK, 255 - 15, 16),  # ends at the last cache position
    (MHA1, 70, 24),          # one query head per kv head (the attention's group-1 instance)
    (MHA1_LONG, 2100, 22),   # group 1 past 2048 cached keys (33 key tiles per token)
    (SPLITK, 100, 57),       # the streamed GEMM (49..64 rows) with a ragged last token tile
    (RAGGED4, 40, 64),       # int4 weights at the largest block, K = 640 in the down projection
    (RAGGED4, 10, 49),       # int4 weights, 49 rows (a ragged fourth token tile)
], ids=["d64_edge", "d128_bias", "int4_ragged", "max_block", "single_row", "last_position", "group1",
        "group1_long", "stream_bf16_57", "int4_64", "int4_49"])
def test_block_matches_oracle(td, cfg, pos0, n):
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, pos0, seed_tag="block")
    _compare(td, cfg, m, k, v, _tokens(cfg, n), pos0, cfg.name)


def test_tiny_prompt_block_matches_oracle(td):
    """The tiny model's whole prompt from an empty cache."""
    cfg = synth.CONFIGS["tiny"]
    m = synth.make_model(cfg)
    k, v = synth.kv_cache(cfg)
    _compare(td, cfg, m, k, v, synth.prompt(cfg), 0, "tiny_prompt")


def test_last_row_logits_only(td):
    """all_logits = 0: the last row's logits, its greedy token in argmax[0] and in
    the token word; the same values as row n - 1 of an all-rows call."""
    cfg = SPLITK
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, 30, seed_tag="block")
    toks = _tokens(cfg, 9)
    full, am_full, _, st1, gk1, gv1 = _block(td, cfg, m, k, v, toks, 30, all_logits=True)
    last, am_last, word, st2, gk2, gv2 = _block(td, cfg, m, k, v, toks, 30, all_logits=False)
    assert st1 == 0 and st2 == 0
    assert np.array_equal(full[-1], last[0])
    assert am_last == [am_full[-1]] and word == am_full[-1]
    assert np.array_equal(gk1, gk2) and np.array_equal(gv1, gv2)


def test_block_then_decode_continues(td):
    """A block prefill followed by decode steps on the same context: the decode
    steps read the block's cache rows and agree with the oracle continuing from
    its own prefill."""
    cfg = synth.CONFIGS["tiny"]
    m = synth.make_model(cfg)
    p = synth.prompt(cfg)
    k, v = synth.kv_cache(cfg)
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    dec.forward_block(torch.from_numpy(p).cuda(), 0, kv, logits)
    o = oracle.Oracle(m)
    o.prefill(p[:-1])
    r, ref = o.step(int(p[-1]), len(p) - 1)
    torch.cuda.synchronize()
    assert dec.status() == 0
    diff = np.max(np.abs(logits.cpu().numpy() - ref))
    assert diff <= 2e-2
    g = td.read_device_i32(dec.token_ptr())
    top2 = np.sort(ref)[-2:]
    assert g == r or top2[1] - top2[0] <= 2 * diff
    r = g  # both sides continue from the GPU's token
    n = cfg.max_ctx - len(p)
    for i in range(n):
        pos = len(p) + i
        dec.step(dec.token_ptr(), pos, kv, logits)
        torch.cuda.synchronize()
        assert dec.status() == 0
        g = td.read_device_i32(dec.token_ptr())
        r2, ref = o.step(r, pos)
        diff = np.max(np.abs(logits.cpu().numpy() - ref))
        assert diff <= 2e-2, (i, diff)
        top2 = np.sort(ref)[-2:]
        assert g == r2 or top2[1] - top2[0] <= 2 * diff
        r = g
    dec.close()


def test_bad_token_sets_range_error(td):
    from decode_persistent_megakernel_amd import _lib
    cfg = SPLITK
    m = synth.make_model(cfg)
    k, v = synth.kv_cache(cfg)
    toks = _tokens(cfg, 5)
    toks[2] = cfg.vocab
    _, _, _, st, _, _ = _block(td, cfg, m, k, v, toks, 0)
    assert st == _lib.TD_E_RANGE


def test_nonfinite_logit_sets_error(td):
    from decode_persistent_megakernel_amd import _lib
    cfg = synth.shrink(SPLITK, tied=False)
    m = synth.make_model(cfg)
    m.head = m.head.copy()
    m.head[5, :] = 0x7FC0  # bf16 NaN: logit 5 is NaN in every row
    k, v = synth.kv_cache(cfg)
    got, am, word, st, _, _ = _block(td, cfg, m, k, v, _tokens(cfg, 3), 0)
    assert st == _lib.TD_E_NONFINITE
    assert np.isnan(got[:, 5]).all() and np.isfinite(np.delete(got, 5, axis=1)).all()


def test_argument_checks(td):
    from decode_persistent_megakernel_amd import _lib
    cfg = SPLITK
    m = synth.make_model(cfg)
    dec = td.Decoder(td.DeviceModel(m), cfg.max_ctx)
    kv = td.KVCache(cfg, cfg.max_ctx)
    logits = torch.empty((_lib.TD_MAX_BLOCK + 1, cfg.vocab), dtype=torch.float32, device="cuda")
    L = _lib.lib()
    kvs = kv.td_kv()
    import ctypes
    t = torch.zeros(_lib.TD_MAX_BLOCK + 1, dtype=torch.int32, device="cuda")
    call = lambda n, pos0, kvp=ctypes.byref(kvs), tp=t.data_ptr(), lp=logits.data_ptr(): L.td_forward_block(  # noqa
        dec.handle, tp, n, pos0, kvp, lp, 1, None, None)
    assert call(0, 0) == _lib.TD_E_INVALID_ARG
    assert call(_lib.TD_MAX_BLOCK + 1, 0) == _lib.TD_E_INVALID_ARG
    assert call(4, -1) == _lib.TD_E_RANGE
    assert call(4, cfg.max_ctx - 3) == _lib.TD_E_RANGE
    assert call(4, 0, tp=None) == _lib.TD_E_INVALID_ARG
    assert call(4, 0, lp=None) == _lib.TD_E_INVALID_ARG
    bad = _lib.TdKV(k=kvs.k, v=kvs.v, max_ctx=cfg.max_ctx - 1)
    assert call(4, 0, kvp=ctypes.byref(bad)) == _lib.TD_E_INVALID_ARG
    # a K or V cache pointer that is not 16-byte aligned is refused on the host by
    # every entry point that takes the cache (no kernel is launched)
    for mk in (dict(k=kvs.k + 8, v=kvs.v), dict(k=kvs.k, v=kvs.v + 2)):
        mis = _lib.TdKV(max_ctx=cfg.max_ctx, **mk)
        assert call(4, 0, kvp=ctypes.byref(mis)) == _lib.TD_E_INVALID_ARG
        assert L.td_decode_step(dec.handle, t.data_ptr(), 0, ctypes.byref(mis), logits.data_ptr(),
                                None) == _lib.TD_E_INVALID_ARG
        assert L.td_decode_loop(dec.handle, t.data_ptr(), 0, 2, -1, ctypes.byref(mis), logits.data_ptr(), None, None,
                                None) == _lib.TD_E_INVALID_ARG
        assert b"16-byte aligned" in L.td_last_error()
    assert call(4, cfg.max_ctx - 4) == _lib.TD_OK
    torch.cuda.synchronize()
    assert dec.status() == 0
    dec.close()


@pytest.mark.parametrize("name,pos0,n,kv_atol_rel", [
    ("llama1b", 100, 16, 2 ** -12),
    ("tinyllama_int4", 100, 16, 2 ** -12),
    ("qwen1p5b", 1000, 24, 2 ** -12),  # d = 128, QKV bias, 28 layers, two 16-row tiles
    ("tinyllama_int4", 60, 52, 2 ** -12),  # int4 weights at full size, 52 rows
    # int4, 33 rows over an 8192-position random N(0, 1) prefix.  Attention over
    # 8192 random rows cancels heavily, and fp32 arithmetic (the decode kernel's
    # as much as the block's) then differs from the fp64 oracle by up to one bf16
    # ulp of the largest K/V values on entries near zero: measured max |d| 3.1e-2
    # (|v| ~ 5) for both paths, while their logits agree with the oracle to 1e-4.
    # Near zero the allowance is therefore one bf16 ulp of the tensor's largest value.
    ("llama1b_int4_long", 8192, 33, 2 ** -7),
])
def test_fullsize_block_matches_oracle(td, name, pos0, n, kv_atol_rel):
    cfg = synth.CONFIGS[name]
    _say(f"{name}: generating the model")
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, pos0, seed_tag="block")
    _compare(td, cfg, m, k, v, _tokens(cfg, n), pos0, name, kv_atol_rel)


def test_fullsize_verify_accepts_own_draft(td):
    """Llama-3.2-1B shape: 64 greedy megakernel decode steps, then one block over
    the same 64 input tokens from the same cache state.  Row i's logits agree
    with step i's and its greedy token is step i's output (the next draft token),
    so a verify of the megakernel's own draft accepts all of it; the cache rows
    agree within one bf16 ulp."""
    cfg = synth.CONFIGS["llama1b"]
    _say("llama1b: generating the model")
    m = synth.make_model(cfg)
    pos0, n = 300, 64
    k, v = synth.random_kv_prefix(cfg, pos0, seed_tag="block")
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    tok = torch.tensor([synth.first_token(cfg)], dtype=torch.int32, device="cuda")
    step_logits = torch.empty((n, cfg.vocab), dtype=torch.float32, device="cuda")
    ins = [synth.first_token(cfg)]
    for i in range(n):
        dec.step(tok.data_ptr() if i == 0 else dec.token_ptr(), pos0 + i, kv, step_logits[i])
        torch.cuda.synchronize()
        ins.append(td.read_device_i32(dec.token_ptr()))
    assert dec.status() == 0
    sk, sv = kv.host()
    outs = ins[1:]
    ins = np.asarray(ins[:n], np.int32)
    dec.close()
    _say("llama1b: block verify of the 64 drafted tokens")
    got, am, word, st, gk, gv = _block(td, cfg, m, k, v, ins, pos0)
    assert st == 0
    ref = step_logits.cpu().numpy().astype(np.float64)
    worst = 0.0
    for i in range(n):
        diff = float(np.max(np.abs(got[i] - ref[i])))
        worst = max(worst, diff)
        assert diff <= 2e-2, (i, diff)
        if am[i] != outs[i]:
            top2 = np.sort(ref[i])[-2:]
            assert top2[1] - top2[0] <= 2 * diff, (i, am[i], outs[i])
    for a, b in ((gk, sk), (gv, sv)):
        _kv_close(bf16_to_f64(a[:, :, pos0:pos0 + n]), bf16_to_f64(b[:, :, pos0:pos0 + n]), "verify")
    accepted = next((i for i in range(n) if am[i] != outs[i]), n)
    _say(f"llama1b verify: max|dlogit| vs the decode steps = {worst:.3g}, accepted {accepted} of {n}")

