"""The single-entry safeguard of the pages' appendix (§7) on the GPU.

The appendix states that the safeguard never activates in practice: the ALS
decrease is far above the single-entry bound max_ij w_j R_ij^2.  Every path
counts the components (blocks) where it would, and the sequential streaming
path can apply it.  A dense fit (tau = 0 keeps every nonzero entry, one
iteration) of a matrix with one dominant entry falls far below that bound,
so the count and the replacement are checked there against the oracle, and
the counts are compared with the oracle's on inputs where they are mixed.
"""
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
    return B, C, res.D.cpu().numpy().astype(np.float64)


def _spiky():
    A = synthetic.gaussian(12, 10, 1, std=0.01)
    A[3, 7] = 5.0
    return A


@pytest.mark.parametrize("mode", ["streaming", "auto"])
def test_safeguard_replaces_a_dense_fit(lib, mode):
    A = _spiky()
    md = lib.MODE_STREAMING if mode == "streaming" else lib.MODE_AUTO
    res = lib.decompose(_dev(A), 0.2, 0.0, 1, 0, 0, mode=md, stats=True, trace=True, safeguard=True)
    ref = oracle.decompose_seq(A, 0.2, 0.0, 1, 0, safeguard=True)
    assert res.stat("mode") == 0   # the replacement runs in streaming mode
    B, C, D = _factors(res)
    assert np.array_equal(np.nonzero(B[:, 0])[0], [3]) and B[3, 0] == 1
    assert np.array_equal(np.nonzero(C[0])[0], [7]) and C[0, 7] == 1
    assert D[0] == float(A[3, 7])
    assert res.stat("safeguard") == ref.extra["safeguard_would"] >= 1
    assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)
    E = float(res.energy.item())
    assert abs(E - ref.E) <= 2e-3
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    tr = res.trace.cpu().numpy()
    assert np.allclose(tr, ref.trace, rtol=1e-5, atol=1e-9 * ref.norm_a2)


@pytest.mark.parametrize("mode", ["resident", "streaming"])
def test_safeguard_counted_not_applied_by_default(lib, mode):
    A = _spiky()
    md = lib.MODE_RESIDENT if mode == "resident" else lib.MODE_STREAMING
    res = lib.decompose(_dev(A), 0.2, 0.0, 1, 0, 0, mode=md, stats=True)
    ref = oracle.decompose_seq(A, 0.2, 0.0, 1, 0)
    assert res.stat("safeguard") == ref.extra["safeguard_would"] >= 1
    B, _, _ = _factors(res)
    assert np.count_nonzero(B[:, 0]) == 12   # the dense fit was kept


def test_safeguard_count_in_block_mode(lib):
    A = synthetic.gaussian(32, 24, 3, std=0.01)
    A[5, 9] = 4.0
    res = lib.decompose(_dev(A), 4 / 24, 0.0, 1, 2, 0, stats=True)   # k = 4, b = 2: two blocks
    ref = oracle.decompose_block(A, 4 / 24, 0.0, 1, 2, 0)
    assert res.stat("mode") == 2
    assert res.stat("safeguard") == ref.extra["safeguard_would"] >= 1


@pytest.mark.parametrize("tau,iters", [(0.0, 1), (2.0, 1)])
def test_safeguard_gives_the_geometric_rate(lib, tau, iters):
    # appendix §7: with the safeguard each component lowers ||R||^2 by at
    # least max R_ij^2 >= ||R||^2 / (m n)
    m, n = 8, 6
    A = synthetic.gaussian(m, n, 9, std=1.0)
    res = lib.decompose(_dev(A), 3.0, tau, iters, 0, 0, trace=True, safeguard=True)
    tr = res.trace.cpu().numpy()
    prev = float(res.norm_a2.item())
    for t in tr:
        assert t <= (1.0 - 1.0 / (m * n)) * prev * (1 + 1e-6)
        prev = t


def _planted(m=96, n=80, spike=16.0, count=4, seed=2):
    A = synthetic.gaussian(m, n, seed, std=1.0)
    rng = np.random.default_rng(seed)
    for q in range(count):
        A[rng.integers(m), rng.integers(n)] = spike * (1 if q % 2 else -1)
    return A


@pytest.mark.parametrize("mode", ["resident", "streaming"])
def test_safeguard_count_matches_oracle_mixed(lib, mode):
    # a Gaussian matrix with four planted entries of magnitude 16: 6 of the
    # first 20 components fall below the single-entry bound (every decision
    # at least 2 % away from the bound), the other 14 stay above it
    A = _planted()
    md = lib.MODE_RESIDENT if mode == "resident" else lib.MODE_STREAMING
    res = lib.decompose(_dev(A), 0.25, 0.7, 15, 0, 0, mode=md, stats=True)
    ref = oracle.decompose_seq(A, 0.25, 0.7, 15, 0)
    assert ref.extra["safeguard_would"] == 6
    assert res.stat("safeguard") == 6


def test_safeguard_count_on_workloads(lib):
    # the pages: never on their (real) weights.  The synthetic Gaussian
    # workload agrees; the 2560 x 2560 LLM-shaped one, with heavy Student-t
    # tails and x10 outlier columns, has entries whose square (max 11.7)
    # exceeds every ALS decrease of its first components (about 6): the
    # oracle counts 32 of the first 32, at least 42 % away from the bound
    c = synthetic.WORKLOADS["gauss256"]
    A = synthetic.workload_matrix("gauss256")
    res = lib.decompose(_dev(A), c["mu"], c["tau"], c["iters"], 0, c["seed"], stats=True)
    assert res.stat("safeguard") == 0
    c = synthetic.WORKLOADS["llm2560"]
    A = synthetic.workload_matrix("llm2560")
    for mode in (lib.MODE_RESIDENT, lib.MODE_STREAMING):
        res = lib.decompose(_dev(A), 32 / 2560, c["tau"], c["iters"], 0, c["seed"], mode=mode, stats=True)
        assert res.k == 32 and res.stat("safeguard") == 32
    res = lib.decompose(_dev(A), c["mu"], c["tau"], c["iters"], c["block"], c["seed"], stats=True)
    assert res.stat("safeguard") == 0   # a whole block's decrease stays above the bound
