"""Refinement sweeps (ExTernD §2.4, refinement) on the GPU against the fp64
oracle.  As for block extraction, the fp32 and fp64 trajectories part once a
near-threshold entry flips, so energies are compared within 2e-3; the energy
the GPU reports must equal an fp64 recomputation from its own factors to
1e-5; the per-sweep trace never rises; repeated runs are bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _factors(res):
    B = oracle.unpack2(res.B2.cpu().numpy().view(np.uint32), res.m).T
    C = oracle.unpack2(res.C2.cpu().numpy().view(np.uint32), res.n)
    D = res.D.cpu().numpy().astype(np.float64)
    return B, C, D


@pytest.mark.parametrize("m,n,mu,tau,b,sweeps", [(256, 256, 1.0, 0.7, 32, 3), (300, 200, 1.3, 1.0, 16, 2),
                                                 (200, 180, 0.9, 0.7, 16, 2), (900, 1000, 0.3, 0.7, 100, 1)])
def test_sweeps_vs_oracle(lib, m, n, mu, tau, b, sweeps):
    A = synthetic.gaussian(m, n, 7)
    Ad = _dev(A)
    base = lib.decompose(Ad, mu, tau, 15, b, 3)
    res = lib.decompose(Ad, mu, tau, 15, b, 3, trace=True, stats=True, sweeps=sweeps)
    torch.cuda.synchronize()
    E, E0 = float(res.energy.item()), float(base.energy.item())
    ref = oracle.decompose_block(A, mu, tau, 15, b, 3, sweeps=sweeps)
    assert abs(E - ref.E) <= 2e-3, (E, ref.E)
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    a2 = float(res.norm_a2.item())
    tr = res.sweep_trace.cpu().numpy()
    assert tr.size == sweeps
    assert tr[0] <= float(res.trace[-1].item()) + 1e-6 * a2
    assert np.all(np.diff(tr) <= 1e-6 * a2)
    assert abs(1.0 - tr[-1] / a2 - E) <= 1e-5
    assert E >= E0 - 1e-6
    assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)
    again = lib.decompose(Ad, mu, tau, 15, b, 3, sweeps=sweeps)
    torch.cuda.synchronize()
    assert torch.equal(again.B2, res.B2) and torch.equal(again.C2, res.C2)
    assert torch.equal(again.D, res.D) and torch.equal(again.energy, res.energy)


def test_zero_sweeps_is_plain_extraction(lib):
    Ad = _dev(synthetic.gaussian(256, 192, 3))
    a = lib.decompose(Ad, 1.0, 0.7, 15, 32, 1)
    z = lib.decompose(Ad, 1.0, 0.7, 15, 32, 1, sweeps=0)
    torch.cuda.synchronize()
    assert torch.equal(a.B2, z.B2) and torch.equal(a.C2, z.C2) and torch.equal(a.D, z.D)
    assert torch.equal(a.energy, z.energy)


@pytest.mark.parametrize("seed,iters", [(2, 15), (8, 15), (16, 15), (1, 3)])
def test_single_block_sweep_continues_the_iterations(lib, seed, iters):
    # one block: the sweep adds it back (R returns to A up to fp32 rounding)
    # and continues its iterations, so the result is the better of the runs
    # with iters and 2 * iters iterations
    A = synthetic.gaussian(160, 128, 40 + seed)
    Ad = _dev(A)
    mu = 16 / 128   # k = 16 = b: a single block
    e1 = float(lib.decompose(Ad, mu, 0.7, iters, 16, seed).energy.item())
    e2 = float(lib.decompose(Ad, mu, 0.7, 2 * iters, 16, seed).energy.item())
    sw = lib.decompose(Ad, mu, 0.7, iters, 16, seed, sweeps=1, stats=True)
    assert sw.k == 16
    assert abs(float(sw.energy.item()) - max(e1, e2)) <= 1e-4
    ref1 = oracle.decompose_block(A, mu, 0.7, iters, 16, seed)
    ref2 = oracle.decompose_block(A, mu, 0.7, iters, 16, seed, sweeps=1)
    assert abs(e1 - ref1.E) <= 2e-3 and abs(float(sw.energy.item()) - ref2.E) <= 2e-3


def test_sweeps_need_block_mode(lib):
    Ad = _dev(synthetic.gaussian(64, 64, 1))
    with pytest.raises(lib.ExterndError) as ei:
        lib.decompose(Ad, 1.0, 0.7, 15, 0, 0, sweeps=1)
    assert ei.value.status == 1


def test_sweeps_llm2560_full_size(lib):
    # the 2560 x 2560 LLM-shaped matrix, mu = 2, tau = 0.7, b = 64: one sweep
    # raises the energy and keeps the report consistent with the factors
    A = synthetic.workload_matrix("llm2560")
    Ad = _dev(A)
    base = lib.decompose(Ad, 2.0, 0.7, 15, 64, 0)
    res = lib.decompose(Ad, 2.0, 0.7, 15, 64, 0, trace=True, stats=True, sweeps=1)
    torch.cuda.synchronize()
    E, E0 = float(res.energy.item()), float(base.energy.item())
    assert E > E0
    assert abs(float(lib.energy(Ad, res.B2, res.C2, res.D).item()) - E) <= 1e-5
    a2 = float(res.norm_a2.item())
    assert abs(1.0 - float(res.sweep_trace[0].item()) / a2 - E) <= 1e-5
