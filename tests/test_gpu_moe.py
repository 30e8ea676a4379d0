"""Mixture-of-experts decode on the persistent kernel and on the per-op and
graph executors.

On the per-op and graph executors the router writes each layer's chosen
experts into a device tensor (td_expert_ids) and the expert kernels read
their weights through it, so one recorded graph serves every routing.  The
persistent kernel routes inside the launch: a router stage publishes the
logits, every CU makes the same choice and streams the chosen experts' rows
("One launch per token", its 64-expert MoE section); it runs bf16 weights.  Every step is compared with the
oracle's teacher-forced step from the same K/V state: the V logits within the
decode-step tolerance (2e-2 for bf16 weights, 5e-2 for int4), the greedy token
(a flip only at a near-tie), and the routing itself: the same experts in the
same order and their probabilities within 1e-3 (relative; a probability's
relative error is its router logit's absolute error, which carries the
residual stream's fp32 error through the layers: observed 1.4e-5 at 16 layers,
while a wrong normalisation or a dropped weight is off by a factor).  The routing is an
integer decided on floating point; both sides decide on fp32 router logits,
and with these seeded models no two candidates come within the fp32 error of
each other, so the choices must be identical.

Shapes: bf16 with 16 experts / top 4 and GQA; int4 with 8 / top 2; the OLMoE
head layout (query heads = kv heads, d = 128) with 64 experts / top 8; 10 / top 3,
5 / top 1 and the largest, 256 / top 16; and the
full OLMoE-1B-7B shape (16 layers, hidden 2048, 64 experts of 1024, top 8,
vocab 50304) from a random K/V prefix of 512 positions.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.test_gpu_parity import td, torch, _say  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

TOL = {synth.WF_BF16: 2e-2, synth.WF_INT4_G64: 5e-2}
BASE = dict(n_layers=2, vocab=1000, prompt_len=0, kv_prefix=0, decode_steps=0, max_ctx=96, tied=False)
MOE_BF16 = synth.shrink(synth.CONFIGS["llama1b"], name="moe_bf16", hidden=256, n_q_heads=8, n_kv_heads=2,
                        head_dim=64, intermediate=256, n_experts=16, top_k=4, seed=3001, **BASE)
MOE_INT4 = synth.shrink(synth.CONFIGS["tinyllama_int4"], name="moe_int4", hidden=256, n_q_heads=4, n_kv_heads=2,
                        head_dim=64, intermediate=384, n_experts=8, top_k=2, seed=3002, **BASE)
MOE_D128 = synth.shrink(synth.CONFIGS["olmoe"], name="moe_d128", hidden=256, n_q_heads=2, n_kv_heads=2,
                        head_dim=128, intermediate=128, n_experts=64, top_k=8, seed=3003, **BASE)
# expert counts that are not a multiple of 4 (the padded tail of the staged router
# logits), top-1, and the largest shapes the kernels take (TD_MAX_EXPERTS experts,
# TD_MAX_TOPK chosen: two groups of eight rows in the down kernel)
MOE_ODD = synth.shrink(synth.CONFIGS["llama1b"], name="moe_e10k3", hidden=256, n_q_heads=4, n_kv_heads=2,
                       head_dim=64, intermediate=192, n_experts=10, top_k=3, seed=3004, **BASE)
MOE_TOP1 = synth.shrink(synth.CONFIGS["llama1b"], name="moe_e5k1", hidden=256, n_q_heads=4, n_kv_heads=2,
                        head_dim=64, intermediate=128, n_experts=5, top_k=1, seed=3005, **BASE)
MOE_MAX = synth.shrink(synth.CONFIGS["llama1b"], name="moe_e256k16", hidden=256, n_q_heads=4, n_kv_heads=2,
                       head_dim=64, intermediate=64, n_experts=256, top_k=16, seed=3006, **BASE)
# one query head per kv head at d = 64: the persistent kernel spreads each head's
# attention over 4 waves (8 at d = 128, MOE_D128), each taking a slice of every
# tile's rows, the states folded in wave order
MOE_MHA64 = synth.shrink(synth.CONFIGS["llama1b"], name="moe_mha64", hidden=256, n_q_heads=4, n_kv_heads=4,
                         head_dim=64, intermediate=192, n_experts=8, top_k=2, seed=3007, **BASE)


def _run(td, cfg, m, k, v, first, start, n, executor, label):
    o = oracle.Oracle(m)
    o.set_kv(k, v)
    dm = td.DeviceModel(m)
    kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
    dec = td.Decoder(dm, cfg.max_ctx, executor=executor)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    t = int(first)
    worst = 0.0
    outs = []
    for i in range(n):
        pos = start + i
        tok.fill_(t)
        dec.step(tok.data_ptr(), pos, kv, logits)
        torch.cuda.synchronize()
        assert dec.status() == 0, (label, i)
        g = td.read_device_i32(dec.token_ptr())
        ids, wts = dec.routing()
        r, tr = o.step_traced(t, pos)
        assert r >= 0
        ref = tr["logits"]
        got = logits.cpu().numpy().astype(np.float64)
        outs.append(logits.cpu().numpy().view(np.uint32).copy())
        assert np.array_equal(ids, tr["expert_ids"]), (label, i, ids, tr["expert_ids"])
        np.testing.assert_allclose(wts, tr["expert_w"], rtol=1e-3, atol=0, err_msg=label)
        diff = float(np.max(np.abs(got - ref)))
        worst = max(worst, diff)
        assert diff <= TOL[cfg.weight_format], (label, i, diff)
        if g != r:
            top2 = np.sort(ref)[-2:]
            assert top2[1] - top2[0] <= 2 * diff, (label, i, g, r)
        t = r
    dec.close()
    _say(f"{label}: {n} steps, max|dlogit| = {worst:.3g}")
    return outs


@pytest.mark.parametrize("cfg,start", [(MOE_BF16, 30), (MOE_INT4, 10), (MOE_D128, 60), (MOE_ODD, 20), (MOE_TOP1, 5),
                                       (MOE_MAX, 40), (MOE_MHA64, 58)],
                         ids=["bf16_e16k4", "int4_e8k2", "d128_e64k8", "e10k3", "e5k1", "e256k16", "mha64_e8k2"])
@pytest.mark.parametrize("executor", ["megakernel", "per_op", "graph"])
def test_moe_matches_oracle(td, cfg, start, executor):
    from decode_persistent_megakernel_amd import _lib
    ex = {"per_op": td.TD_EXEC_PER_OP, "graph": td.TD_EXEC_GRAPH, "megakernel": td.TD_EXEC_MEGAKERNEL}[executor]
    m = synth.make_model(cfg)
    if ex == td.TD_EXEC_MEGAKERNEL and cfg.weight_format != synth.WF_BF16:
        with pytest.raises(td.TdError) as ei:  # the persistent kernel runs MoE layers on bf16 weights
            td.Decoder(td.DeviceModel(m), cfg.max_ctx, executor=ex)
        assert ei.value.code == _lib.TD_E_UNSUPPORTED
        return
    k, v = synth.random_kv_prefix(cfg, start, seed_tag="moe")
    _run(td, cfg, m, k, v, synth.first_token(cfg), start, 12, ex, f"{cfg.name}/{executor}")


@pytest.mark.parametrize("cfg", [MOE_D128, MOE_BF16, MOE_MAX, MOE_MHA64],
                         ids=["d128_e64k8", "bf16_e16k4", "e256k16", "mha64_e8k2"])
def test_executors_agree_across_routings(td, cfg):
    """The graph executor replays one recording and the persistent kernel routes
    inside its launch; the logits of both equal the per-op executor's bit for
    bit over steps whose routing differs, and so do the routings."""
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, 20, seed_tag="moe")
    dm = td.DeviceModel(m)
    res = {}
    for ex in (td.TD_EXEC_PER_OP, td.TD_EXEC_GRAPH, td.TD_EXEC_MEGAKERNEL):
        kv = td.KVCache(cfg, cfg.max_ctx, k=k, v=v)
        dec = td.Decoder(dm, cfg.max_ctx, executor=ex)
        tok = torch.tensor([synth.first_token(cfg)], dtype=torch.int32, device="cuda")
        logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
        bits, routes = [], []
        for i in range(8):
            dec.step(tok.data_ptr() if i == 0 else dec.token_ptr(), 20 + i, kv, logits)
            torch.cuda.synchronize()
            assert dec.status() == 0
            bits.append(logits.cpu().numpy().view(np.uint32).copy())
            routes.append(dec.routing()[0].copy())
        res[ex] = (bits, routes)
        dec.close()
    (b0, r0) = res[td.TD_EXEC_PER_OP]
    for ex in (td.TD_EXEC_GRAPH, td.TD_EXEC_MEGAKERNEL):
        b1, r1 = res[ex]
        assert all(np.array_equal(a, b) for a, b in zip(r0, r1)), ex
        assert all(np.array_equal(a, b) for a, b in zip(b0, b1)), ex
    assert len({x.tobytes() for x in r0}) > 1  # the routing changed between steps
    for ids in r0:
        for row in ids:
            assert len(set(row.tolist())) == cfg.top_k and row.min() >= 0 and row.max() < cfg.n_experts


def test_moe_errors(td):
    from decode_persistent_megakernel_amd import _lib
    cfg = MOE_BF16
    m = synth.make_model(cfg)
    dm = td.DeviceModel(m)
    m4 = synth.make_model(MOE_INT4)
    with pytest.raises(td.TdError) as ei:  # int4 experts: per-op and graph executors only
        td.Decoder(td.DeviceModel(m4), MOE_INT4.max_ctx, executor=td.TD_EXEC_MEGAKERNEL)
    assert ei.value.code == _lib.TD_E_UNSUPPORTED
    dec = td.Decoder(dm, cfg.max_ctx, executor=td.TD_EXEC_PER_OP)
    kv = td.KVCache(cfg, cfg.max_ctx)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    toks = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(td.TdError) as ei:
        dec.forward_block(toks, 0, kv, logits)
    assert ei.value.code == _lib.TD_E_UNSUPPORTED
    dec.close()
    # a NaN router row: a non-finite router logit is reported, and the step stays in bounds
    m.layers[1].router = m.layers[1].router.copy()
    m.layers[1].router[3, :] = 0x7FC0
    dmn = td.DeviceModel(m)
    for ex in (td.TD_EXEC_PER_OP, td.TD_EXEC_MEGAKERNEL):
        dec = td.Decoder(dmn, cfg.max_ctx, executor=ex)
        tok = torch.tensor([5], dtype=torch.int32, device="cuda")
        dec.step(tok.data_ptr(), 0, kv, logits)
        torch.cuda.synchronize()
        assert dec.status() == _lib.TD_E_NONFINITE, ex
        ids, wts = dec.routing()
        assert ids[1].tolist() == list(range(cfg.top_k)) and not wts[1].any(), ex  # in-bounds fallback routing
        dec.close()


@pytest.mark.parametrize("executor", ["megakernel", "graph"])
def test_fullsize_olmoe_matches_oracle(td, executor):
    cfg = synth.CONFIGS["olmoe"]
    ex = {"graph": td.TD_EXEC_GRAPH, "megakernel": td.TD_EXEC_MEGAKERNEL}[executor]
    _say("olmoe: generating the model")
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, cfg.start_pos)
    _say(f"olmoe: 8 teacher-forced steps from position {cfg.start_pos} ({executor})")
    _run(td, cfg, m, k, v, synth.first_token(cfg), cfg.start_pos, 8, ex, f"olmoe/{executor}")


def test_tied_router_logits_take_the_lower_id_first(td):
    """Equal router logits: the lower expert id takes the earlier slot.  The top
    expert's router row is copied to two other experts of layer 0, so from the
    first step on three experts share the largest logit bit for bit (the rows are
    identical, so both sides compute identical logits for them); the kernel must
    then order them by id, as the oracle does, on every step."""
    cfg = MOE_BF16
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, 30, seed_tag="moe")
    o = oracle.Oracle(m)
    o.set_kv(k, v)
    _, tr = o.step_traced(synth.first_token(cfg), 30)
    top = int(tr["expert_ids"][0][0])
    twins = sorted({(top + 3) % cfg.n_experts, (top + cfg.n_experts - 5) % cfg.n_experts})
    m.layers[0].router = m.layers[0].router.copy()
    for e in twins:
        m.layers[0].router[e, :] = m.layers[0].router[top, :]
    o = oracle.Oracle(m)
    o.set_kv(k, v)
    _, tr = o.step_traced(synth.first_token(cfg), 30)
    assert sorted(tr["expert_ids"][0][:3].tolist()) == sorted([top] + twins)
    assert tr["expert_ids"][0][:3].tolist() == sorted([top] + twins)  # the oracle's own tie order
    for ex in (td.TD_EXEC_PER_OP, td.TD_EXEC_GRAPH, td.TD_EXEC_MEGAKERNEL):
        _run(td, cfg, m, k, v, synth.first_token(cfg), 30, 4, ex, f"ties/{ex}")


@pytest.mark.parametrize("cfg,start", [(MOE_MAX, 40), (MOE_BF16, 30), (MOE_D128, 60)],
                         ids=["e256k16", "bf16_e16k4", "d128_e64k8"])
def test_moe_down_reads_no_stale_input(td, cfg, start):
    """Regression: a MoE down row shorter than its whole chunks meets zero
    weights in its padded lanes, against the activations after its slot, and
    the last slot's reach runs past top_k I.  The persistent kernel zeroes its
    input area out to that reach; before, the stage read whatever an earlier
    kernel had left in LDS there, and a stale NaN made the router logits of the
    next layer NaN (0 x NaN).  Here an earlier kernel leaves NaN in every CU's
    LDS on purpose: the GEMV hook, on a grid of one workgroup per CU, stages a
    NaN input of 32768 values (LDS bytes 0 to 128 Ki) and packs NaN weight
    chunks just above it (where the d = 64 shapes keep their input area); then
    the MoE step must still match the oracle.  These shapes have top_k I a
    multiple of 512 (no zero padding past top_k I without the reach) and down
    rows of 64 to 256 values."""
    rows, cols = 2048, 32768
    w = torch.full((rows, cols), -1, dtype=torch.int16, device="cuda")  # 0xFFFF: a bf16 NaN
    x = torch.full((cols,), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    m = synth.make_model(cfg)
    k, v = synth.random_kv_prefix(cfg, start, seed_tag="moe")
    for rep in range(2):
        td.gemv(synth.WF_BF16, w, None, rows, cols, x, y)
        torch.cuda.synchronize()
        assert torch.isnan(y).all()  # the hook ran on the NaN input
        _run(td, cfg, m, k, v, synth.first_token(cfg), start, 2, td.TD_EXEC_MEGAKERNEL, f"{cfg.name}/stale-lds{rep}")
