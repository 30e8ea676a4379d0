"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks one oracle function against something other than itself: a
closed form, an invariant, a special case that reduces to a library routine,
brute force in a different formulation (tests/ref_fullseq.py), or the byte
counts the pages print.  A plausible slip (a dropped term, a wrong sign, a
swapped nibble, an off-by-one position) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from tests import ref_fullseq as R

RNG = np.random.default_rng(7)


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- formats

def test_bf16_value_matches_bit_view():
    bits = RNG.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_value(b) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_value_exhaustive_against_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(b) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_round_bf16_matches_torch_rne():
    vals = np.concatenate([RNG.normal(size=2000) * 10.0 ** RNG.integers(-6, 6, size=2000),
                           [0.0, -0.0, 1.0, -1.0, 1e-40, 3.0e38]])
    # exact ties between two bf16 values: odd and even mantissas
    ties = (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32)
            .view(np.float32).astype(np.float64))
    vals = np.concatenate([vals, ties])
    ref = bf16_bits(vals.astype(np.float32))
    got = np.array([oracle.round_bf16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_synth_roundings_match_libraries():
    L = synth.lib()
    f = np.concatenate([RNG.normal(size=3000).astype(np.float32) * np.float32(0.003),
                        (RNG.normal(size=1000) * 1e-6).astype(np.float32),   # fp16 subnormal range
                        np.array([65504.0, 65520.0, 1e5, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8], np.float32)])
    got16 = np.array([L.synth_f32_to_f16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got16, f.astype(np.float16).view(np.uint16))
    gotb = np.array([L.synth_f32_to_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(gotb, bf16_bits(f))


def test_synth_stream_is_splitmix64():
    def splitmix(state, n):
        out = []
        M = (1 << 64) - 1
        for _ in range(n):
            state = (state + 0x9E3779B97F4A7C15) & M
            z = state
            z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
            z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
            out.append(z ^ (z >> 31))
        return out
    k = synth.key(1234, 3, "w")
    assert [synth.lib().synth_stream_at(k, i) for i in range(8)] == splitmix(k, 8)


def test_synth_distributions():
    k = synth.key(1, 0, "t")
    w = R.bf16_to_f64(synth.bf16_normal(200000, k, 0.02))
    assert abs(w.mean()) < 2e-4 and abs(w.std() - 0.02) < 2e-4
    s = R.f16_to_f64(synth.f16_absnormal(200000, k, 0.003))
    assert s.min() >= 0 and abs(s.mean() - 0.003 * math.sqrt(2 / math.pi)) < 3e-5
    u = synth.u8_uniform(200000, k)
    for nib in (u & 15, u >> 4):
        c = np.bincount(nib, minlength=16)
        assert c.min() > 11500 and c.max() < 13500
    t = synth.i32_uniform(100000, k, 4096)
    assert t.min() >= 0 and t.max() < 4096


# --------------------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("c", [0.5, -3.0, 1e-3])
def test_rmsnorm_constant_vector_closed_form(c):
    n, eps = 2048, 1e-5
    g = bf16_bits(RNG.normal(size=n))
    y = oracle.rmsnorm(np.full(n, c), g, eps)
    expect = c / math.sqrt(c * c + eps) * R.bf16_to_f64(g)
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance_and_rms_one():
    x = RNG.normal(size=1536) * 3.7
    g = bf16_bits(np.ones(1536))
    y = oracle.rmsnorm(x, g, 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14
    np.testing.assert_allclose(oracle.rmsnorm(x * 123.0, g, 0.0), y, rtol=1e-13)
    assert np.all(oracle.rmsnorm(np.zeros(64), g[:64], 1e-6) == 0)


# --------------------------------------------------------------------------- GEMV

def test_linear_identity_returns_x_exactly():
    n = 300
    W = np.zeros((n, n), dtype=np.uint16)
    W[np.arange(n), np.arange(n)] = 0x3F80  # bf16 1.0
    x = RNG.normal(size=n)
    assert np.array_equal(oracle.linear(W, None, oracle.WF_BF16, n, n, x), x)


def test_linear_one_hot_returns_column():
    rows, cols = 333, 1100
    W = bf16_bits(RNG.normal(size=(rows, cols)))
    Wf = R.bf16_to_f64(W)
    for k in (0, 1, 517, cols - 1):
        e = np.zeros(cols)
        e[k] = 1.0
        assert np.array_equal(oracle.linear(W, None, oracle.WF_BF16, rows, cols, e), Wf[:, k])


def test_linear_bf16_brute_force_numpy():
    rows, cols = 333, 1108  # odd shapes (tinyinfer tests odd shapes such as 333 x 11008)
    W = bf16_bits(RNG.normal(size=(rows, cols)) * 0.02)
    x = RNG.normal(size=cols)
    y = oracle.linear(W, None, oracle.WF_BF16, rows, cols, x, nthreads=3)
    ref = R.bf16_to_f64(W) @ x
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


def test_int4_nibble_order_hand_built():
    # one row, K = 64: bytes 0x21, 0x43 -> elements 0..3 carry codes 1,2,3,4 (q = -7..-4)
    w = np.full((1, 32), 0x88, dtype=np.uint8)  # code 8 = q 0 elsewhere
    w[0, 0], w[0, 1] = 0x21, 0x43
    s = np.array([[0x3C00]], dtype=np.uint16)  # fp16 1.0
    got = [oracle.weight(w, s, oracle.WF_INT4_G64, 64, 0, k) for k in range(6)]
    assert got == [-7.0, -6.0, -5.0, -4.0, 0.0, 0.0]


def test_int4_one_hot_is_exact_dequant_all_codes_and_scales():
    # every code 0..15 at every position parity, scales incl. fp16 subnormals and the max
    scales = np.array([0x0001, 0x03FF, 0x0400, 0x1A3D, 0x3C00, 0x7BFF, 0x8400 | 0x0123], dtype=np.uint16)
    rows, cols = len(scales), 128
    codes = np.tile(np.arange(16), (rows, cols // 16))
    w = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = np.repeat(scales[:, None], cols // 64, axis=1)
    for k in range(cols):
        e = np.zeros(cols)
        e[k] = 1.0
        y = oracle.linear(w, s, oracle.WF_INT4_G64, rows, cols, e)
        expect = R.f16_to_f64(scales) * float(codes[0, k] - 8)
        assert np.array_equal(y, expect), k


def test_linear_int4_brute_force_numpy():
    rows, cols = 96, 5632 // 4
    scales = (np.abs(RNG.normal(size=(rows, cols // 64)) * 0.003)).astype(np.float16).view(np.uint16)
    lin = synth.Linear(w=RNG.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8), s=scales,
                       rows=rows, cols=cols)
    x = RNG.normal(size=cols)
    y = oracle.linear(lin.w, lin.s, oracle.WF_INT4_G64, rows, cols, x)
    np.testing.assert_allclose(y, R.dequant(lin) @ x, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    v = RNG.normal(size=128)
    assert np.array_equal(oracle.rope(v, 0, 1e6), v)


def test_rope_preserves_pair_norms():
    d = 64
    v = RNG.normal(size=d)
    r = oracle.rope(v, 517, 500000.0)
    n0 = v[:d // 2] ** 2 + v[d // 2:] ** 2
    n1 = r[:d // 2] ** 2 + r[d // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_rope_relative_position():
    d = 64
    q, k = RNG.normal(size=d), RNG.normal(size=d)
    a = oracle.rope(q, 40, 10000.0) @ oracle.rope(k, 13, 10000.0)
    b = oracle.rope(q, 40 + 1000, 10000.0) @ oracle.rope(k, 13 + 1000, 10000.0)
    assert abs(a - b) < 1e-11


def test_rope_d2_is_plane_rotation_and_pairs_are_half_split():
    # d = 2: theta_0 = 1, so position p rotates (a, b) by p radians
    r = oracle.rope(np.array([1.0, 0.0]), 3, 10000.0)
    np.testing.assert_allclose(r, [math.cos(3), math.sin(3)], rtol=0, atol=1e-15)
    # d = 8, element 1 pairs with element 5 (not with element 2): frequency base^(-2/8)
    v = np.zeros(8)
    v[1] = 1.0
    r = oracle.rope(v, 7, 10000.0)
    ang = 7 * 10000.0 ** (-2.0 / 8)
    expect = np.zeros(8)
    expect[1], expect[5] = math.cos(ang), math.sin(ang)
    np.testing.assert_allclose(r, expect, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- attention

def test_attention_single_entry_returns_v_exactly():
    d = 64
    K = bf16_bits(RNG.normal(size=(1, d)))
    V = bf16_bits(RNG.normal(size=(1, d)))
    assert np.array_equal(oracle.attention(RNG.normal(size=d), K, V), R.bf16_to_f64(V[0]))


def test_attention_equal_keys_give_mean_of_v():
    d, n = 64, 37
    K = np.tile(bf16_bits(RNG.normal(size=d)), (n, 1))
    V = bf16_bits(RNG.normal(size=(n, d)))
    np.testing.assert_allclose(oracle.attention(RNG.normal(size=d), K, V), R.bf16_to_f64(V).mean(0),
                               rtol=0, atol=1e-14)


def test_attention_dominant_key_returns_its_v():
    d, n = 64, 50
    K = bf16_bits(RNG.normal(size=(n, d)) * 0.01)
    K[17] = bf16_bits(np.full(d, 4.0))
    V = bf16_bits(RNG.normal(size=(n, d)))
    q = np.full(d, 100.0)  # score of key 17 exceeds the others by > 3000
    assert np.array_equal(oracle.attention(q, K, V), R.bf16_to_f64(V[17]))


@pytest.mark.parametrize("n", [2, 5, 129])
def test_attention_brute_force_scipy_softmax(n):
    d = 128
    q = RNG.normal(size=d)
    K = bf16_bits(RNG.normal(size=(n, d)))
    V = bf16_bits(RNG.normal(size=(n, d)))
    p = scipy.special.softmax(R.bf16_to_f64(K) @ q / math.sqrt(d))
    np.testing.assert_allclose(oracle.attention(q, K, V), p @ R.bf16_to_f64(V), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- SiLU

def test_silu_properties_and_library():
    assert oracle.silu(0.0) == 0.0
    for z in (-30.0, -2.5, -0.1, 0.3, 1.0, 7.0):
        assert abs((oracle.silu(z) - oracle.silu(-z)) - z) < 1e-14     # sigma(z) + sigma(-z) = 1
        assert abs(oracle.silu(z) - z * scipy.special.expit(z)) < 1e-15
    assert oracle.silu(60.0) == 60.0


# --------------------------------------------------------------------------- argmax

def test_argmax_lowest_id_on_ties_and_errors():
    x = np.array([0.1, 3.0, -1.0, 3.0, 3.0])
    assert oracle.argmax(x) == (1, False)
    assert oracle.argmax(np.zeros(10)) == (0, False)
    # values equal after rounding to fp32 are ties as well
    y = np.array([1.0, 1.0 + 1e-12, 0.5])
    assert oracle.argmax(y) == (0, False)
    z = np.array([0.0, np.nan, 5.0])
    assert oracle.argmax(z)[1] is True
    assert oracle.argmax(np.array([np.inf, 1.0]))[1] is True


# --------------------------------------------------------------------------- whole step

def tiny_cfg(**over):
    return synth.shrink(synth.CONFIGS["tiny"], **over)


def test_zero_block_model_reduces_to_embedding_dot():
    """W_o = W_d = 0 leaves x = E[t]; with a tied head the logits are
    E . RMSNorm(E[t]) and the self-dot wins, so the next token is t."""
    cfg = tiny_cfg()
    m = synth.make_model(cfg)
    for L in m.layers:
        L.o.w[...] = 0
        L.down.w[...] = 0
    o = oracle.Oracle(m)
    for t in (0, 77, 4095):
        nxt, logits = o.step(t, 0)
        h = R.rmsnorm(R.bf16_to_f64(m.embed[t]), 1.0, cfg.rms_eps)
        np.testing.assert_allclose(logits, R.bf16_to_f64(m.embed) @ h, rtol=0, atol=1e-12)
        assert nxt == t


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("gqa4_bias_int4", dict(n_q_heads=8, n_kv_heads=2, qkv_bias=True, weight_format=synth.WF_INT4_G64,
                            tied=False, hidden=128, intermediate=192, vocab=500, head_dim=32)),
    ("mha_d128", dict(n_q_heads=2, n_kv_heads=2, head_dim=128, hidden=256, intermediate=320, vocab=300,
                      rope_theta=1e6, rms_eps=1e-6)),
])
def test_decode_matches_full_sequence_reference(name, over):
    """Incremental decode with a bf16 K/V cache == full-sequence causal forward."""
    cfg = tiny_cfg(**over)
    m = synth.make_model(cfg)
    toks = synth.i32_uniform(20, synth.key(5, 0, name), cfg.vocab)
    ref_logits, ks, vs = R.forward(m, toks)
    o = oracle.Oracle(m, max_ctx=24)
    for p, t in enumerate(toks):
        nxt, logits = o.step(int(t), p)
        np.testing.assert_allclose(logits, ref_logits[p], rtol=0, atol=1e-9)
        assert nxt == oracle.argmax(ref_logits[p])[0]
    for l in range(cfg.n_layers):
        got_k = R.bf16_to_f64(o.k[l, :, :len(toks)]).transpose(1, 0, 2)
        got_v = R.bf16_to_f64(o.v[l, :, :len(toks)]).transpose(1, 0, 2)
        # both round to bf16 from fp64 values that agree to ~1e-15: allow a rare 1-ulp flip
        assert np.mean(got_k != ks[l]) < 1e-3 and np.mean(got_v != vs[l]) < 1e-3
        np.testing.assert_allclose(got_k, ks[l], rtol=2 ** -7, atol=1e-30)
        np.testing.assert_allclose(got_v, vs[l], rtol=2 ** -7, atol=1e-30)


def test_result_independent_of_thread_count():
    cfg = tiny_cfg()
    m = synth.make_model(cfg)
    outs = []
    for nt in (1, 5):
        o = oracle.Oracle(m, nthreads=nt)
        o.prefill(synth.prompt(cfg)[:8])
        outs.append(o.step(11, 8)[1])
    assert np.array_equal(outs[0], outs[1])


def test_step_errors():
    cfg = tiny_cfg()
    m = synth.make_model(cfg)
    o = oracle.Oracle(m)
    assert o.step(cfg.vocab, 0)[0] == oracle.E_ARG
    assert o.step(-1, 0)[0] == oracle.E_ARG
    assert o.step(0, cfg.max_ctx)[0] == oracle.E_ARG
    m.embed[3, 5] = 0x7FC0  # NaN in the embedding row of token 3
    assert o.step(3, 0)[0] == oracle.E_NONFINITE


def test_tiny_greedy_regression_file():
    """The committed oracle run of the tiny config (tests/golden/make_golden.py) still reproduces."""
    import json
    import os
    from tests.golden import make_golden
    ref = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_greedy.json")))
    got = make_golden.tiny_run()
    assert got["prompt"] == ref["prompt"] and got["greedy"] == ref["greedy"]
    np.testing.assert_allclose(got["max_logit"], ref["max_logit"], rtol=1e-12)


# --------------------------------------------------------------------------- MoE routing and MLP

def test_route_closed_form_example():
    """Router logits ln 4, ln 2, 0, 0: the softmax is 1/2, 1/4, 1/8, 1/8 exactly in
    closed form; the top 3 are experts 0, 1, then 2 (the tie of 2 and 3 goes to
    the lower id)."""
    z = np.array([math.log(4.0), math.log(2.0), 0.0, 0.0])
    r, ids, w = oracle.route(z, 3)
    assert r == 0
    assert ids.tolist() == [0, 1, 2]
    np.testing.assert_allclose(w, [0.5, 0.25, 0.125], rtol=1e-15)
    # order follows the logits, not the ids
    r, ids, w = oracle.route(np.array([0.0, 0.0, math.log(4.0), math.log(2.0)]), 2)
    assert ids.tolist() == [2, 3]
    np.testing.assert_allclose(w, [0.5, 0.25], rtol=1e-15)
    # equal after rounding to fp32: a tie, the lower id first
    r, ids, w = oracle.route(np.array([1.0 + 1e-12, 1.0, -5.0]), 1)
    assert ids.tolist() == [0]
    r, ids, w = oracle.route(np.array([1.0, 1.0 + 1e-12, -5.0]), 1)
    assert ids.tolist() == [0]
    # all experts: the weights are the whole softmax and sum to 1
    zz = RNG.normal(size=16)
    r, ids, w = oracle.route(zz, 16)
    assert sorted(ids.tolist()) == list(range(16))
    np.testing.assert_allclose(w.sum(), 1.0, rtol=1e-14)
    np.testing.assert_allclose(w, scipy.special.softmax(zz)[ids], rtol=1e-14)


def test_route_errors():
    assert oracle.route(np.array([0.0, np.nan]), 1)[0] == oracle.E_NONFINITE
    assert oracle.route(np.array([0.0, np.inf]), 1)[0] == oracle.E_NONFINITE
    assert oracle.route(np.array([0.0, 1.0]), 3)[0] == oracle.E_ARG
    assert oracle.route(np.array([0.0, 1.0]), 0)[0] == oracle.E_ARG


def _moe_from_dense(dense, n_experts, top_k, poison_from=None):
    """A MoE copy of a dense model: every expert is the dense MLP, the router is
    zero (all logits equal, so the uniform softmax and the lowest ids win);
    experts from `poison_from` on have NaN weights."""
    cfg = synth.shrink(dense.cfg, n_experts=n_experts, top_k=top_k)
    m = synth.make_model(cfg)
    m.embed, m.head, m.final_norm = dense.embed, dense.head, dense.final_norm
    for Ld, Lm in zip(dense.layers, m.layers):
        Lm.attn_norm, Lm.qkv, Lm.qkv_bias, Lm.o, Lm.mlp_norm = Ld.attn_norm, Ld.qkv, Ld.qkv_bias, Ld.o, Ld.mlp_norm
        Lm.router = np.zeros_like(Lm.router)
        Lm.gate_up.w = np.ascontiguousarray(np.concatenate([Ld.gate_up.w] * n_experts))
        Lm.down.w = np.ascontiguousarray(np.concatenate([Ld.down.w] * n_experts))
        if poison_from is not None:
            I, H = cfg.intermediate, cfg.hidden
            Lm.gate_up.w[poison_from * 2 * I:] = 0x7FC0
            Lm.down.w[poison_from * H:] = 0x7FC0
    return m


def test_moe_identical_experts_reduce_to_dense():
    """A zero router over E identical experts routes to experts 0..k-1 with
    weight 1/E each, so the MLP is k/E times the dense one.  With k = E the step
    is the dense step; with E = 2k (the unrouted half poisoned with NaN) it is
    the dense step with W_d halved (exact in bf16)."""
    dense = synth.make_model(tiny_cfg())
    toks = synth.i32_uniform(6, synth.key(9, 0, "moe"), dense.cfg.vocab)
    ref = oracle.Oracle(dense)
    moe = oracle.Oracle(_moe_from_dense(dense, 4, 4))
    for p, t in enumerate(toks):
        r0, l0 = ref.step(int(t), p)
        r1, l1 = moe.step(int(t), p)
        assert r0 == r1
        np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)
    half = synth.make_model(tiny_cfg())
    for L in half.layers:
        L.down.w = bf16_bits(R.bf16_to_f64(L.down.w) * 0.5)
    ref2 = oracle.Oracle(half)
    moe2 = oracle.Oracle(_moe_from_dense(dense, 8, 4, poison_from=4))
    for p, t in enumerate(toks):
        r0, l0 = ref2.step(int(t), p)
        r1, l1 = moe2.step(int(t), p)
        assert r0 == r1 and np.isfinite(l1).all()
        np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,over", [
    ("moe_bf16", dict(n_experts=8, top_k=2)),
    ("moe_int4", dict(n_experts=6, top_k=3, weight_format=synth.WF_INT4_G64, hidden=128, intermediate=192,
                      tied=False)),
])
def test_moe_decode_matches_full_sequence_reference(name, over):
    """Incremental MoE decode == the full-sequence forward with torch.topk routing,
    and the routed experts the oracle reports are torch's."""
    cfg = tiny_cfg(**over)
    m = synth.make_model(cfg)
    toks = synth.i32_uniform(12, synth.key(5, 1, name), cfg.vocab)
    ref_logits, _, _ = R.forward(m, toks)
    o = oracle.Oracle(m, max_ctx=16)
    for p, t in enumerate(toks):
        nxt, tr = o.step_traced(int(t), p)
        np.testing.assert_allclose(tr["logits"], ref_logits[p], rtol=0, atol=1e-9)
        assert nxt == oracle.argmax(ref_logits[p])[0]
        assert len(set(tr["expert_ids"][0].tolist())) == cfg.top_k
