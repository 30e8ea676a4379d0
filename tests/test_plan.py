"""The work plan on the host, without a device: the plan the library builds for
every workload validates, and a corrupted plan is refused with TD_E_PLAN before
anything is launched ("Decoding in tiles", sec. 4: the schedule is built and
checked once, and the runtime rejects an invalid one).  Covered corruptions:
a unit with two owners (overlapping CU ranges), a unit without an owner (a
gap), a range past the end of the matrix, a descending range, a table that
does not start at 0 or end at the unit count.  A config the attention split
cannot place (more kv heads than CUs) is refused with TD_E_UNSUPPORTED, not a
division by zero."""
import ctypes

import numpy as np
import pytest

import synth
from decode_persistent_megakernel_amd import _lib

NCU = 256
NSP = 6  # unit spaces: QKV row pairs, hidden rows, intermediate rows, vocabulary rows, router rows, expert units


def _cfg(c, **over):
    kw = dict(n_layers=c.n_layers, hidden=c.hidden, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
              head_dim=c.head_dim, intermediate=c.intermediate, vocab=c.vocab, max_ctx=c.max_ctx,
              rope_theta=c.rope_theta, rms_eps=c.rms_eps, weight_format=c.weight_format,
              qkv_bias=int(c.qkv_bias), n_experts=c.n_experts, top_k=c.top_k)
    kw.update(over)
    return _lib.TdConfig(**kw)


def _partition(cfg, ncu=NCU):
    part = np.zeros(NSP * (ncu + 1), dtype=np.int32)
    rc = _lib.lib().td_plan_partition(ctypes.byref(cfg), ncu, part.ctypes.data, part.size)
    assert rc == _lib.TD_OK, _lib.last_error()
    return part


def _check(cfg, part=None, ncu=NCU):
    if part is None:
        return _lib.lib().td_plan_check(ctypes.byref(cfg), ncu, None, 0)
    part = np.ascontiguousarray(part, dtype=np.int32)
    return _lib.lib().td_plan_check(ctypes.byref(cfg), ncu, part.ctypes.data, part.size)


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_every_workload_plan_validates(name):
    cfg = _cfg(synth.CONFIGS[name])
    assert _check(cfg) == _lib.TD_OK, _lib.last_error()
    part = _partition(cfg).reshape(NSP, NCU + 1)
    c = synth.CONFIGS[name]
    units = [c.qkv_rows // 2, c.hidden, c.intermediate, c.vocab, c.n_experts, c.top_k * c.intermediate]
    for sp in range(NSP):
        assert part[sp, 0] == 0 and part[sp, -1] == units[sp]
        assert np.all(np.diff(part[sp]) >= 0)
    # the plan's own table, passed back in, validates too
    assert _check(cfg, part.ravel()) == _lib.TD_OK


def _corrupt(p, space, kind):
    """A copy of partition table p (NSP x (NCU + 1)) with one unit space corrupted."""
    p = p.copy()
    r = p[space]
    if kind == "overlap":          # CU 20's range ends after CU 21's begins: boundaries out of order
        r[21], r[22] = r[22] + 1, r[21]
    elif kind == "start_gap":      # unit 0 has no owner
        r[0] = 1
    elif kind == "end_gap":        # the last unit has no owner
        r[NCU] -= 1
    elif kind == "past_end":       # the last CU's range runs past the matrix
        r[NCU] += 1
    elif kind == "negative":       # a range starting before unit 0
        r[0] = -1
    return p


@pytest.mark.parametrize("kind", ["overlap", "start_gap", "end_gap", "past_end", "negative"])
@pytest.mark.parametrize("space", range(NSP))
def test_corrupted_partition_is_refused(space, kind):
    cfg = _cfg(synth.CONFIGS["llama1b"])
    base = _partition(cfg).reshape(NSP, NCU + 1)
    bad = _corrupt(base, space, kind)
    assert not np.array_equal(bad, base)
    assert _check(cfg, bad.ravel()) == _lib.TD_E_PLAN, _lib.last_error()


def test_another_exact_tiling_is_accepted():
    """The validator checks ownership, not equality with the plan's own table:
    moving one boundary by a unit still gives every unit one owner."""
    cfg = _cfg(synth.CONFIGS["llama1b"])
    p = _partition(cfg).reshape(NSP, NCU + 1).copy()
    for sp in range(4):  # the spaces a dense model uses
        assert p[sp, 101] > p[sp, 100]
        p[sp, 101] -= 1
    assert _check(cfg, p.ravel()) == _lib.TD_OK, _lib.last_error()


def test_moe_plan_keeps_each_cu_in_one_expert_slot():
    """The expert gate/up units are top_k slots of I; every CU's range lies in one
    slot (its waves stream one chosen expert's rows), so a table in which a CU's
    range crosses a slot boundary is refused with TD_E_PLAN.  The router's rows
    are a unit space of their own; int4 experts are refused by the persistent
    kernel (the per-op executors run them)."""
    c = synth.CONFIGS["olmoe"]
    cfg = _cfg(c)
    part = _partition(cfg).reshape(NSP, NCU + 1)
    ei = part[5]
    per_slot = NCU // c.top_k
    for j in range(c.top_k + 1):
        assert ei[j * per_slot] == j * c.intermediate
    for cu in range(NCU):
        if ei[cu + 1] > ei[cu]:
            assert ei[cu] // c.intermediate == (ei[cu + 1] - 1) // c.intermediate
    bad = part.copy()
    b = per_slot  # the first CU of slot 1 starts one unit early: the previous CU ends inside slot 0 ...
    bad[5, b] -= 1  # ... and this CU's range now crosses from slot 0 into slot 1
    assert _check(cfg, bad.ravel()) == _lib.TD_E_PLAN
    assert "slot" in _lib.last_error()
    for corrupt in ("overlap", "start_gap", "end_gap", "past_end", "negative"):
        for sp in (4, 5):
            assert _check(cfg, _corrupt(part, sp, corrupt).ravel()) == _lib.TD_E_PLAN, (sp, corrupt)
    c4 = _cfg(c, weight_format=synth.WF_INT4_G64)
    assert _check(c4) == _lib.TD_E_UNSUPPORTED
    # odd expert counts and top-1 plan too (the logits hand-off pads to a pair)
    assert _check(_cfg(c, n_experts=5, top_k=1)) == _lib.TD_OK, _lib.last_error()


def test_more_kv_heads_than_cus_is_unsupported_not_a_crash():
    # 64 kv heads on a device of 32 CUs: the attention split has no CU per head
    cfg = _lib.TdConfig(n_layers=1, hidden=4096, n_q_heads=64, n_kv_heads=64, head_dim=64, intermediate=512,
                        vocab=1000, max_ctx=64, rope_theta=1e4, rms_eps=1e-5, weight_format=0, qkv_bias=0)
    assert _check(cfg, ncu=32) == _lib.TD_E_UNSUPPORTED
    assert "kv heads" in _lib.last_error()
    assert _check(cfg, ncu=256) == _lib.TD_OK


def test_bad_arguments():
    cfg = _cfg(synth.CONFIGS["tiny"])
    L = _lib.lib()
    assert L.td_plan_check(None, NCU, None, 0) == _lib.TD_E_INVALID_ARG
    part = np.zeros(10, dtype=np.int32)
    assert L.td_plan_check(ctypes.byref(cfg), NCU, part.ctypes.data, part.size) == _lib.TD_E_INVALID_ARG
    assert L.td_plan_partition(ctypes.byref(cfg), NCU, part.ctypes.data, part.size) == _lib.TD_E_INVALID_ARG
    assert _check(cfg, ncu=12) == _lib.TD_E_UNSUPPORTED  # not a multiple of 8
    bad = _cfg(synth.CONFIGS["tiny"], head_dim=96)
    assert _check(bad) == _lib.TD_E_INVALID_ARG
