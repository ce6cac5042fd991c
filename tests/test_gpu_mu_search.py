"""Choosing mu per matrix for a target energy (ExTernD §3.3), on the GPU.

One decomposition at mu_max gives, through its residual trace and the greedy
prefix property, the energy of every shorter decomposition (every whole
number of blocks in block mode).  Checked here: ||A||^2 as reported matches
the fp64 oracle; the rank chosen from the trace, run on its own, gives
exactly the prefix of the long run's factors (bit-identical), reaches the
target (within 1e-5: the trace is predicted from the exact decrease, the
energy of the separate run recomputed from its fp32 residual), and one step
less does not.
"""
import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu


CASES = [  # (m, n, mu_max, block, mode, targets)
    (256, 256, 2.0, 0, 1, (0.3, 0.8, 0.95)),     # resident sequential
    (300, 200, 1.0, 0, 0, (0.3, 0.8)),           # streaming sequential
    (512, 384, 1.0, 32, -1, (0.3, 0.7, 0.9)),    # block, b = 32
]


@pytest.mark.parametrize("m,n,mu_max,block,mode,targets", CASES)
def test_rank_for_energy_reproduces_prefix(lib, m, n, mu_max, block, mode, targets):
    A_h = synthetic.gaussian(m, n, 21)
    A = torch.from_numpy(A_h).cuda()
    big = lib.decompose(A, mu_max, 0.7, 15, block, 3, mode=mode, trace=True)
    torch.cuda.synchronize()
    a2 = float(big.norm_a2.item())
    ref_a2 = float(np.sum(A_h.astype(np.float64) ** 2))
    assert abs(a2 - ref_a2) <= 1e-12 * ref_a2
    tr = big.trace.cpu().numpy()
    step = big.block
    assert np.all(np.diff(tr) <= 1e-9 * a2)
    for target in targets:
        c = lib.rank_for_energy(tr, big.k, step, a2, target)
        assert c > 0 and c % step == 0, (target, c)
        mu = c / min(m, n)
        assert lib.rank(m, n, mu) == c
        small = lib.decompose(A, mu, 0.7, 15, block, 3, mode=mode, stats=True)
        torch.cuda.synchronize()
        assert small.k == c
        assert torch.equal(small.B2, big.B2[:c]), target
        assert torch.equal(small.C2, big.C2[:c]), target
        assert torch.equal(small.D, big.D[:c]), target
        e = float(small.energy.item())
        assert e >= target - 1e-5
        assert abs(e - (1.0 - tr[c // step - 1] / a2)) <= 1e-5
        if c > step:
            assert 1.0 - tr[c // step - 2] / a2 < target


def test_mu_for_energy_helper(lib):
    A = torch.from_numpy(synthetic.gaussian(256, 192, 8)).cuda()
    got = lib.mu_for_energy(A, 0.75, 2.0, 0.7, seed=1)
    assert got is not None
    mu, c, e = got
    assert c == lib.rank(256, 192, mu) and e >= 0.75
    assert lib.mu_for_energy(A, 0.9999, 0.1, 0.7, seed=1) is None
