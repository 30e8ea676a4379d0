"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Every compute call goes through the C ABI (libtd.so).  Floating-point results
are compared within a bound derived from the arithmetic (fp32 accumulation of
K products: |err| <= gamma_K * sum |w x|, gamma_K = K u / (1 - K u), u = 2^-24)
or, end to end, within the logits tolerance of the decode-step contract
(max |diff| <= 2e-2 for bf16 weights, 5e-2 for int4).  Dequantisation of int4
is checked bit-exactly with one-hot inputs.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_persistent_megakernel_amd as td
    from decode_persistent_megakernel_amd import _lib
    _lib.lib()  # loud failure if the library is missing
    return td


RNG = np.random.default_rng(1234)
U = 2.0 ** -24


def gamma(k):
    return k * U / (1 - k * U)


def bf16_from_f32(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


# ------------------------------------------------------------------ GEMV hook

@pytest.mark.parametrize("rows,cols", [(333, 1112), (512, 256), (3072, 2048), (2048, 8192), (1536, 8960), (7, 520)])
def test_gemv_bf16_matches_oracle(td, rows, cols):
    _say(f"gemv bf16 {rows}x{cols}")
    W = bf16_from_f32(RNG.normal(size=(rows, cols)) * 0.02)
    x = RNG.normal(size=cols).astype(np.float32)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    td.gemv(td.TD_WF_BF16, dev(W), None, rows, cols, torch.from_numpy(x).cuda(), y)
    got = y.cpu().numpy().astype(np.float64)
    ref = oracle.linear(W, None, oracle.WF_BF16, rows, cols, x.astype(np.float64))
    bound = gamma(cols) * (np.abs(bf16_to_f64(W)) @ np.abs(x.astype(np.float64))) + 1e-30
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)


@pytest.mark.parametrize("rows,cols", [(96, 1408), (2560, 2048), (2048, 5632), (2048, 8192), (5, 128)])
def test_gemv_int4_matches_oracle(td, rows, cols):
    _say(f"gemv int4 {rows}x{cols}")
    w = RNG.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s = (np.abs(RNG.normal(size=(rows, cols // 64)) * 0.003)).astype(np.float16).view(np.uint16)
    x = RNG.normal(size=cols).astype(np.float32)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    td.gemv(td.TD_WF_INT4_G64, dev(w), dev(s), rows, cols, torch.from_numpy(x).cuda(), y)
    got = y.cpu().numpy().astype(np.float64)
    ref = oracle.linear(w, s, oracle.WF_INT4_G64, rows, cols, x.astype(np.float64))
    # |w| <= 8 * scale; the scale multiply adds one more rounding
    absw = 8.0 * np.repeat(s.view(np.float16).astype(np.float64), 64, axis=1)
    bound = gamma(cols + 2) * (absw @ np.abs(x.astype(np.float64))) + 1e-30
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)


def test_gemv_int4_one_hot_is_bit_exact_dequant(td):
    _say("gemv int4 one-hot")
    rows, cols = 64, 2048
    codes = RNG.integers(0, 16, size=(rows, cols))
    w = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    svals = np.array([0x0001, 0x03FF, 0x0400, 0x1A3D, 0x3C00, 0x7BFF, 0x8123, 0x2E66], dtype=np.uint16)
    s = svals[RNG.integers(0, len(svals), size=(rows, cols // 64))]
    W, S = dev(w), dev(s)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    for k in (0, 1, 31, 32, 63, 64, 1000, 2047):
        e = np.zeros(cols, np.float32)
        e[k] = 1.0
        td.gemv(td.TD_WF_INT4_G64, W, S, rows, cols, torch.from_numpy(e).cuda(), y)
        ref = oracle.linear(w, s, oracle.WF_INT4_G64, rows, cols, e.astype(np.float64))
        assert np.array_equal(y.cpu().numpy().astype(np.float64), ref), k


# ------------------------------------------------------------------ attention hook

# (positions, head dim, chunk length): one row, ragged single tiles, several tiles per
# chunk, many chunks with a ragged last one, the largest chunk count (64), head dim 128
ATTN_CASES = [(1, 64, 0), (5, 64, 0), (63, 64, 64), (64, 64, 64), (65, 64, 64), (200, 64, 0), (200, 64, 64),
              (1000, 64, 128), (4095, 64, 64), (129, 128, 64), (1, 128, 0), (777, 128, 192), (513, 128, 0)]


# waves per query head: the forms the step takes (1; 4 for group 1 at head dim 64, 8 at
# head dim 128) and 2, which the routine supports as well
ATTN_WAVE_CASES = [(n, d, c, w) for n, d, c in ATTN_CASES for w in ((1, 2, 4) if d == 64 else (1, 2, 4, 8))]


@pytest.mark.parametrize("n,d,chunk,waves", ATTN_WAVE_CASES,
                         ids=[f"n{n}_d{d}_c{c}_w{w}" for n, d, c, w in ATTN_WAVE_CASES])
def test_attention_hook_matches_oracle(td, n, d, chunk, waves):
    """The step's own tile routine, its fold of a head's wave states and its
    split-K merge (through td_test_attention) against the oracle's two-pass
    softmax in fp64: within 2e-5 of the output's scale (fp32 exponentials and
    sums over at most 4096 positions), and exactly V when there is a single
    position (the head's other waves then hold no position and add nothing)."""
    _say(f"attention hook n={n} d={d} chunk={chunk} waves={waves}")
    q = RNG.normal(size=d).astype(np.float32)
    K = bf16_from_f32(RNG.normal(size=(n, d)))
    V = bf16_from_f32(RNG.normal(size=(n, d)))
    out = torch.empty(d, dtype=torch.float32, device="cuda")
    td.attention(torch.from_numpy(q).cuda(), dev(K), dev(V), n, d, out, chunk_len=chunk, waves=waves)
    ref = oracle.attention(q.astype(np.float64), K, V)
    got = out.cpu().numpy().astype(np.float64)
    if n == 1:
        assert np.array_equal(got, ref)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-5 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("waves", [1, 2, 4])
def test_attention_hook_one_dominant_key_and_equal_keys(td, waves):
    """Closed forms: with all keys equal the output is the mean of V; with one
    key far ahead of the others it is that key's V row (for each wave split:
    the dominant key sits in one wave's rows, the other waves' states fold in
    with weight e^-64)."""
    d, n = 64, 300
    q = np.ones(d, dtype=np.float32)
    K = bf16_from_f32(np.full((n, d), 0.25))
    V = bf16_from_f32(RNG.normal(size=(n, d)))
    out = torch.empty(d, dtype=torch.float32, device="cuda")
    td.attention(torch.from_numpy(q).cuda(), dev(K), dev(V), n, d, out, chunk_len=64, waves=waves)
    np.testing.assert_allclose(out.cpu().numpy(), bf16_to_f64(V).mean(axis=0), rtol=0, atol=1e-5)
    K2 = bf16_from_f32(np.zeros((n, d)))
    K2[137] = bf16_from_f32(np.full(d, 8.0))  # score 8 * 64 / 8 = 64 above the rest: e^-64 weights
    td.attention(torch.from_numpy(q).cuda(), dev(K2), dev(V), n, d, out, chunk_len=64, waves=waves)
    np.testing.assert_allclose(out.cpu().numpy(), bf16_to_f64(V[137]), rtol=0, atol=1e-6)


def test_attention_hook_argument_checks(td):
    from decode_persistent_megakernel_amd import _lib
    d = 64
    q = torch.zeros(d, dtype=torch.float32, device="cuda")
    kv = torch.zeros((5000, d), dtype=torch.int16, device="cuda")
    out = torch.empty(d, dtype=torch.float32, device="cuda")
    for n, dd, c, w in ((10, 64, 32, 1), (10, 96, 0, 1), (0, 64, 0, 1), (4097, 64, 64, 1), (10, 64, 0, 3),
                        (10, 64, 0, 8), (10, 64, 0, 0)):
        with pytest.raises(_lib.TdError) as ei:
            td.attention(q, kv, kv, n, dd, out, chunk_len=c, waves=w)
        assert ei.value.code == _lib.TD_E_INVALID_ARG, (n, dd, c, w)


# ------------------------------------------------------------------ whole step (megakernel)

def run_compare(td, cfg, model, kv_k, kv_v, first_token, start_pos, n_steps, tol, label, executor=0):
    """Teacher-forced comparison: both sides start from the same K/V state; at
    every step both receive the same input token (the oracle's greedy choice)
    and their logits and greedy tokens are compared."""
    o = oracle.Oracle(model)
    o.set_kv(kv_k, kv_v)
    dm = td.DeviceModel(model)
    kv = td.KVCache(cfg, cfg.max_ctx, k=kv_k, v=kv_v)
    dec = td.Decoder(dm, cfg.max_ctx, executor=executor)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    t = int(first_token)
    worst = 0.0
    min_gap = math.inf
    for i in range(n_steps):
        pos = start_pos + i
        tok.fill_(t)
        dec.step(tok.data_ptr(), pos, kv, logits)
        torch.cuda.synchronize()
        st = dec.status()
        assert st == 0, (label, i, st)
        g_tok = td.read_device_i32(dec.token_ptr())
        r, ref = o.step(t, pos)
        assert r >= 0
        got = logits.cpu().numpy().astype(np.float64)
        diff = np.max(np.abs(got - ref))
        worst = max(worst, diff)
        top2 = np.sort(ref)[-2:]
        gap = top2[1] - top2[0]
        min_gap = min(min_gap, gap)
        assert diff <= tol, (label, i, diff)
        if g_tok != r:
            # only a near-tie may flip: the oracle's top-2 gap must be below the observed error
            assert gap <= 2 * diff, (label, i, g_tok, r, gap, diff)
        t = r
    _say(f"{label}: {n_steps} steps, max|dlogit| = {worst:.3g}, min top-2 gap = {min_gap:.3g}")
    dec.close()
    return worst


def test_tiny_decode_matches_oracle(td):
    _say("tiny: oracle prefill, 16 teacher-forced decode steps")
    cfg = synth.CONFIGS["tiny"]
    m = synth.make_model(cfg)
    o = oracle.Oracle(m)
    p = synth.prompt(cfg)
    o.prefill(p[:-1])
    run_compare(td, cfg, m, o.k.copy(), o.v.copy(), p[-1], len(p) - 1, cfg.decode_steps + 1, 2e-2, "tiny")


def test_tiny_gpu_prefill_matches_oracle_cache(td):
    """The GPU runs the prompt through its own decode step; its K/V cache and
    the next token agree with the oracle's."""
    _say("tiny: GPU prefill vs oracle prefill")
    cfg = synth.CONFIGS["tiny"]
    m = synth.make_model(cfg)
    o = oracle.Oracle(m)
    p = synth.prompt(cfg)
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx)
    dec = td.Decoder(dm, cfg.max_ctx)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    for i, t in enumerate(p):
        tok.fill_(int(t))
        dec.step(tok.data_ptr(), i, kv, logits)
        r, ref = o.step(int(t), i)
    torch.cuda.synchronize()
    assert dec.status() == 0
    gk, gv = kv.host()
    P = len(p)
    for a, b in ((gk, o.k), (gv, o.v)):
        a = bf16_to_f64(a[:, :, :P])
        b = bf16_to_f64(b[:, :, :P])
        # fp32 vs fp64 before the bf16 rounding: at most one bf16 ulp apart, rarely
        np.testing.assert_allclose(a, b, rtol=2 ** -7, atol=1e-6)
        assert np.mean(a != b) < 0.02
    assert td.read_device_i32(dec.token_ptr()) == r
    assert np.max(np.abs(logits.cpu().numpy() - ref)) <= 2e-2
    dec.close()


def test_bit_reproducible_across_runs(td):
    """Fixed reduction orders: the same step twice gives the same logits bits."""
    _say("tiny: reproducibility")
    cfg = synth.CONFIGS["tiny"]
    m = synth.make_model(cfg)
    dm = td.DeviceModel(m)
    dec = td.Decoder(dm, cfg.max_ctx)
    outs = []
    for _ in range(3):
        kv = td.KVCache(cfg, cfg.max_ctx)
        tok = torch.tensor([17], dtype=torch.int32, device="cuda")
        logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
        for pos in range(5):
            dec.step(tok.data_ptr(), pos, kv, logits)
        torch.cuda.synchronize()
        outs.append(logits.cpu().numpy().view(np.uint32).copy())
    assert dec.status() == 0
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    dec.close()
