"""Kernel-level parity of the step's RoPE rotation and greedy selection
(through td_test_rope and td_test_argmax) against the oracle.

RoPE: the step rotates fp32 pairs with a host-built fp32 (cos, sin) row; the
oracle rotates in fp64 with exact cos/sin.  Each output is a two-term sum of
products of values rounded to fp32, so |GPU - oracle| <= 4 * 2^-24 * (|a| + |b|)
for the pair (a, b).  Position 0 is the identity, bit for bit.
Argmax: integer result, compared exactly; ties go to the lowest id, a
non-finite logit is left out of the choice and raises the flag (the oracle
decides on the same fp32 values).
"""
import numpy as np
import pytest

import oracle
from tests.test_gpu_parity import td, torch, _say  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(4321)


@pytest.mark.parametrize("d,pos,theta", [(64, 0, 1e4), (64, 1, 1e4), (64, 639, 5e5), (64, 8255, 5e5),
                                         (128, 1087, 1e6), (128, 3, 1e4)])
def test_rope_hook_matches_oracle(td, d, pos, theta):
    _say(f"rope hook d={d} pos={pos} theta={theta}")
    nh = 12
    x = RNG.normal(size=(nh, d)).astype(np.float32)
    out = torch.empty((nh, d), dtype=torch.float32, device="cuda")
    td.rope(torch.from_numpy(x).cuda(), nh, d, pos, theta, out)
    got = out.cpu().numpy().astype(np.float64)
    half = d // 2
    for h in range(nh):
        ref = oracle.rope(x[h].astype(np.float64), pos, theta)
        scale = np.abs(x[h, :half]).astype(np.float64) + np.abs(x[h, half:])
        bound = 4 * 2.0 ** -24 * np.concatenate([scale, scale])
        assert np.all(np.abs(got[h] - ref) <= bound), (h, np.max(np.abs(got[h] - ref) / bound))
        # each pair's norm is preserved
        n_in = x[h, :half].astype(np.float64) ** 2 + x[h, half:].astype(np.float64) ** 2
        n_out = got[h, :half] ** 2 + got[h, half:] ** 2
        np.testing.assert_allclose(n_out, n_in, rtol=1e-6, atol=1e-12)
    if pos == 0:
        assert np.array_equal(out.cpu().numpy(), x)


def _argmax(td, logits, groups):
    n = logits.size
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    work = torch.empty(3 * groups, dtype=torch.int32, device="cuda")
    tok = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    bad = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    td.argmax(lg, n, groups, work, tok, bad)
    return int(tok.item()), int(bad.item())


@pytest.mark.parametrize("n,groups", [(128256, 256), (32000, 256), (4096, 256), (1000, 7), (257, 256), (1, 1)])
def test_argmax_hook_matches_oracle(td, n, groups):
    _say(f"argmax hook n={n} groups={groups}")
    z = RNG.normal(size=n).astype(np.float32)
    tok, bad = _argmax(td, z, groups)
    r, rbad = oracle.argmax(z.astype(np.float64))
    assert (tok, bad) == (r, int(rbad))


def test_argmax_hook_ties_take_the_lowest_id(td):
    n, groups = 128256, 256
    z = RNG.normal(size=n).astype(np.float32)
    top = np.float32(z.max() + 1.0)
    # equal maxima in different workgroups, in one workgroup's different waves and lanes
    for ids in ([90000, 5, 128255], [70001, 70000], [3000, 3008, 3001], [128255, 0]):
        zz = z.copy()
        zz[ids] = top
        tok, bad = _argmax(td, zz, groups)
        assert (tok, bad) == (min(ids), 0), ids
        assert oracle.argmax(zz.astype(np.float64)) == (min(ids), False)
    tok, _ = _argmax(td, np.zeros(n, np.float32), groups)
    assert tok == 0


def test_argmax_hook_nonfinite(td):
    n, groups = 50000, 256
    z = RNG.normal(size=n).astype(np.float32)
    best = int(np.argmax(z))
    for bad_val, at in ((np.nan, 10), (np.inf, 49999), (-np.inf, 123), (np.nan, best)):
        zz = z.copy()
        zz[at] = bad_val
        tok, bad = _argmax(td, zz, groups)
        r, rbad = oracle.argmax(zz.astype(np.float64))
        assert bad == 1 and rbad
        assert tok == r, (bad_val, at, tok, r)
    tok, bad = _argmax(td, np.full(300, np.nan, np.float32), 4)
    assert (tok, bad) == (0, 1)
