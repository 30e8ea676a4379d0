"""The in-kernel token loop (td_decode_loop): several greedy steps in one
launch, the token of each step decided on the device.  Every step computes what
one td_decode_step computes, in the same order, so a loop of n steps must give
the same tokens, the same K/V cache and the same last logits, bit for bit, as
n single steps (which the parity tests check against the oracle).  Covered: the
attention split changing inside one launch (a chunk gains its first row), head
dim 128 with a QKV bias, int4, several tiles per chunk, two loops chained
through the token word, the stop on an end-of-sequence token, the stop on a
non-finite logit, and the argument checks."""
import numpy as np
import pytest

import synth
from tests.test_gpu_parity import td, torch, _say  # noqa: F401  (fixture)
from tests.test_gpu_edges import SPLITK, SPLITK128, RAGGED4
from tests.test_gpu_executors import MULTITILE

pytestmark = pytest.mark.gpu


def _setup(td, cfg, start, seed_tag="loop"):
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, start, seed_tag=seed_tag)
    return m, k, v


def _singles(td, cfg, m, k, v, first, start, n):
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    tok = torch.tensor([int(first)], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    toks, outs = [], []
    for i in range(n):
        dec.step(tok.data_ptr() if i == 0 else dec.token_ptr(), start + i, kv, logits)
        torch.cuda.synchronize()
        assert dec.status() == 0
        toks.append(td.read_device_i32(dec.token_ptr()))
        outs.append(logits.cpu().numpy().view(np.uint32).copy())
    kh, vh = kv.host()
    dec.close()
    return toks, outs, kh, vh


def _loop(td, cfg, m, k, v, first, start, splits, eos=-1):
    """Loops of the given lengths back to back (each starting from the last one's token)."""
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    tok = torch.tensor([int(first)], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    toks, count, pos = [], 0, start
    for j, n in enumerate(splits):
        out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        dec.loop(tok.data_ptr() if j == 0 else dec.token_ptr(), pos, n, kv, logits, out, cnt, eos=eos)
        torch.cuda.synchronize()
        st = dec.status()
        c = int(cnt.item())
        got = out.cpu().numpy().tolist()
        assert 1 <= c <= n and got[c:] == [-1] * (n - c), (c, got)
        toks += got[:c]
        count += c
        pos += c
        if c < n:
            break
    last = logits.cpu().numpy().view(np.uint32).copy()
    kh, vh = kv.host()
    tok_word = td.read_device_i32(dec.token_ptr())
    dec.close()
    return toks, count, last, kh, vh, tok_word, st


@pytest.mark.parametrize("cfg,start,splits", [
    (SPLITK, 58, [12]),           # positions 58..69: the split grows from one chunk to two
    (SPLITK128, 120, [10]),       # d = 128 + bias, across 127/128
    (RAGGED4, 40, [8]),           # int4, ragged rows
    (MULTITILE, 2100, [3, 3]),    # two tiles per chunk, 17 chunks; two chained loops
], ids=["d64_split_grows", "d128_bias", "int4", "multitile_chained"])
def test_loop_equals_single_steps(td, cfg, start, splits):
    n = sum(splits)
    _say(f"loop vs single steps on {cfg.name}, {splits} from {start}")
    m, k, v = _setup(td, cfg, start)
    first = synth.first_token(cfg)
    ref_t, ref_l, ref_k, ref_v = _singles(td, cfg, m, k, v, first, start, n)
    got_t, count, last, gk, gv, tok_word, st = _loop(td, cfg, m, k, v, first, start, splits)
    assert st == 0
    assert count == n
    assert got_t == ref_t
    assert tok_word == ref_t[-1]
    assert np.array_equal(last, ref_l[-1]), int(np.sum(last != ref_l[-1]))
    assert np.array_equal(gk, ref_k) and np.array_equal(gv, ref_v)


def test_loop_fullsize_llama1b_equals_single_steps(td):
    cfg = synth.CONFIGS["llama1b"]
    start, n = cfg.start_pos, 6
    _say(f"loop vs single steps, llama1b, {n} steps from {start}")
    m, k, v = _setup(td, cfg, start)
    first = synth.first_token(cfg)
    ref_t, ref_l, ref_k, ref_v = _singles(td, cfg, m, k, v, first, start, n)
    got_t, count, last, gk, gv, tok_word, st = _loop(td, cfg, m, k, v, first, start, [n])
    assert st == 0 and count == n and got_t == ref_t
    assert np.array_equal(last, ref_l[-1])
    assert np.array_equal(gk, ref_k) and np.array_equal(gv, ref_v)


def test_loop_stops_at_eos(td):
    cfg, start, n = SPLITK, 60, 8
    _say("loop stops at the end-of-sequence token")
    m, k, v = _setup(td, cfg, start)
    first = synth.first_token(cfg)
    ref_t, ref_l, ref_k, ref_v = _singles(td, cfg, m, k, v, first, start, n)
    stop_at = 3
    eos = ref_t[stop_at]
    expect = ref_t.index(eos) + 1  # the first step whose token is eos is the last
    got_t, count, last, gk, gv, tok_word, st = _loop(td, cfg, m, k, v, first, start, [n], eos=eos)
    assert st == 0
    assert count == expect and got_t == ref_t[:expect]
    assert np.array_equal(last, ref_l[expect - 1])
    # rows of the positions not run are untouched
    k0, v0 = k.copy(), v.copy()
    for arr, ref, orig in ((gk, ref_k, k0), (gv, ref_v, v0)):
        assert np.array_equal(arr[:, :, :start + expect], ref[:, :, :start + expect])
        assert np.array_equal(arr[:, :, start + expect:], orig[:, :, start + expect:])


def test_loop_stops_on_nonfinite_logit(td):
    from decode_persistent_megakernel_amd import _lib
    cfg = synth.shrink(SPLITK, tied=False)
    _say("loop stops on a non-finite logit")
    m = synth.make_model(cfg)
    m.head = m.head.copy()
    m.head[5, :] = 0x7FC0  # bf16 NaN: logit 5 is NaN in every step
    k, v = synth.random_kv_prefix(cfg, 30, seed_tag="loop")
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    tok = torch.tensor([1], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    out = torch.full((5,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    dec.loop(tok.data_ptr(), 30, 5, kv, logits, out, cnt)
    torch.cuda.synchronize()
    assert dec.status() == _lib.TD_E_NONFINITE
    assert int(cnt.item()) == 1 and out.cpu().numpy().tolist()[1:] == [-1] * 4
    dec.close()


def test_loop_argument_checks(td):
    from decode_persistent_megakernel_amd import _lib
    cfg = SPLITK
    _say("loop argument checks")
    m = synth.make_model(cfg)
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    dec = td.Decoder(dm, cfg.max_ctx)
    cases = [(0, 0, -1, _lib.TD_E_INVALID_ARG),
             (0, _lib.TD_MAX_LOOP_STEPS + 1, -1, _lib.TD_E_INVALID_ARG),
             (cfg.max_ctx - 2, 3, -1, _lib.TD_E_RANGE), (-1, 1, -1, _lib.TD_E_RANGE),
             (0, 2, cfg.vocab, _lib.TD_E_INVALID_ARG), (0, 2, -2, _lib.TD_E_INVALID_ARG)]
    for pos, n, eos, code in cases:
        with pytest.raises(_lib.TdError) as ei:
            dec.loop(tok.data_ptr(), pos, n, kv, logits, eos=eos)
        assert ei.value.code == code, (pos, n, eos)
    # the last window that fits is accepted
    dec.loop(tok.data_ptr(), cfg.max_ctx - 3, 3, kv, logits)
    torch.cuda.synchronize()
    assert dec.status() == 0
    dec.close()
    per_op = td.Decoder(dm, cfg.max_ctx, executor=td.TD_EXEC_PER_OP)
    with pytest.raises(_lib.TdError) as ei:
        per_op.loop(tok.data_ptr(), 0, 2, kv, logits)
    assert ei.value.code == _lib.TD_E_UNSUPPORTED
    per_op.close()


def test_step_clock_and_stream_yardstick(td):
    """The measurement hooks: the in-kernel step clock of a loop (one stamp at
    the launch's start, then one per step decided, none past the buffer), and
    the stream-read yardstick's rate, between a plausible floor and the
    device's published 8 TB/s."""
    cfg, start = SPLITK, 20
    _say("step clock of a loop launch, and the stream-read yardstick")
    m, k, v = _setup(td, cfg, start)
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx)
    tok = torch.tensor([int(synth.first_token(cfg))], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    for n, slots in ((6, 7), (6, 4)):  # a buffer for every step, then one that holds only three
        clk = torch.zeros(slots + 2, dtype=torch.int64, device="cuda")
        dec.set_step_clock(clk[:slots])
        dec.loop(tok.data_ptr(), start, n, kv, logits)
        torch.cuda.synchronize()
        assert dec.status() == 0
        c = clk.cpu().numpy()
        assert np.all(c[:slots] > 0) and np.all(np.diff(c[:slots]) > 0), c
        assert np.all(c[slots:] == 0), c  # nothing past the buffer
        assert np.all(np.diff(c[:slots]) < 100_000_000), c  # each step well under a second (100 MHz ticks)
        start += n
    dec.set_step_clock(None)
    dec.loop(tok.data_ptr(), start, 2, kv, logits)
    torch.cuda.synchronize()
    assert dec.status() == 0 and np.all(clk.cpu().numpy()[:4] == c[:4])  # off: the old buffer is not written
    dec.close()
    buf = torch.ones(64 << 20, dtype=torch.int32, device="cuda")  # 256 MiB
    gbps = td.measure_stream(buf, reps=3)
    _say(f"stream-read yardstick over 256 MiB: {gbps:.0f} GB/s")
    assert 500.0 < gbps < 8000.0 * 1.05
