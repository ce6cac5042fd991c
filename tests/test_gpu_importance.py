"""Importance-weighted ALS (ExTernD §2.5) on the GPU against the fp64 oracle.

The weights are h / max(h) + lambda over the input columns.  The GPU forms
them in fp32 and the oracle in fp64, so weighted quantities agree to about
1e-7 relative.  End to end, the weighted energy is compared within 2e-3 of
the oracle's (the trajectories part at near-threshold flips, as unweighted).
The reported energy must match an fp64 weighted recomputation from the GPU's
own factors to 1e-5.  Per step on captured inputs, T_tau is bit-exact and the
GEMV and the scale are within 1e-5 of fp64 weighted least squares.  Flat
importance with weights 1 or 4 gives the unweighted result bit for bit.
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
    D = res.D.cpu().numpy().astype(np.float64)
    return B, C, D


def _relnorm(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


CASES = [  # (m, n, mu, tau, block, mode, lam)
    (256, 256, 1.0, 0.7, 0, 1, 0.0),      # resident
    (300, 200, 1.0, 0.7, 0, 0, 0.0),      # streaming
    (300, 200, 1.0, 0.7, 0, 2, 0.05),     # persistent streaming
    (256, 256, 1.0, 0.7, 0, 1, 0.05),
    (256, 256, 1.0, 0.7, 32, -1, 0.0),    # block, NS inverse
    (300, 200, 1.3, 1.0, 16, -1, 0.1),    # block, ragged
    (1100, 1040, 0.25, 0.7, 128, -1, 0.0),  # block, b = 128 (Gauss-Jordan inverse)
]


@pytest.mark.parametrize("m,n,mu,tau,block,mode,lam", CASES)
def test_weighted_vs_oracle(lib, m, n, mu, tau, block, mode, lam):
    A = synthetic.gaussian(m, n, 17)
    h = synthetic.importance(n, 5)
    Ad, hd = _dev(A), _dev(h)
    res = lib.decompose(Ad, mu, tau, 15, block, 2, mode=mode, trace=True, stats=True, importance=hd, lam=lam)
    torch.cuda.synchronize()
    w = oracle.importance_weights(h, lam)
    if block:
        ref = oracle.decompose_block(A, mu, tau, 15, block, 2, weights=w)
    else:
        ref = oracle.decompose_seq(A, mu, tau, 15, 2, weights=w)
    E = float(res.energy.item())
    assert abs(E - ref.E) <= 2e-3, (E, ref.E)
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D, weights=w)) <= 1e-5
    a2 = float(res.norm_a2.item())
    assert abs(a2 - ref.norm_a2) <= 1e-6 * ref.norm_a2
    tr = res.trace.cpu().numpy()
    assert np.all(np.diff(tr) <= 1e-9 * a2)
    assert abs(1 - tr[-1] / a2 - E) <= 1e-4
    assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)
    if mode >= 0:
        assert res.stat("mode") == {0: 0, 1: 1, 2: 3}[mode]
    again = lib.decompose(Ad, mu, tau, 15, block, 2, mode=mode, importance=hd, lam=lam)
    torch.cuda.synchronize()
    assert torch.equal(again.B2, res.B2) and torch.equal(again.D, res.D)
    assert torch.equal(again.energy, res.energy)


@pytest.mark.parametrize("block,mode", [(0, 1), (0, 0), (0, 2), (32, -1), (128, -1)])
@pytest.mark.parametrize("level,lam", [(0.37, 0.0), (5.0, 3.0)])
def test_flat_importance_is_the_plain_algorithm(lib, block, mode, level, lam):
    # weights exactly 1, or exactly 4 (every step scales by a power of two)
    m, n = (1100, 1040) if block == 128 else (256, 192)
    mu = 0.25 if block == 128 else 1.0
    Ad = _dev(synthetic.gaussian(m, n, 3))
    hd = torch.full((n,), level, dtype=torch.float32, device="cuda")
    plain = lib.decompose(Ad, mu, 0.7, 15, block, 1, mode=mode, stats=True)
    wtd = lib.decompose(Ad, mu, 0.7, 15, block, 1, mode=mode, stats=True, importance=hd, lam=lam)
    torch.cuda.synchronize()
    assert torch.equal(plain.B2, wtd.B2) and torch.equal(plain.C2, wtd.C2)
    assert torch.equal(plain.D, wtd.D)
    assert torch.equal(plain.energy, wtd.energy)


@pytest.mark.parametrize("mode", [1, 0, 2])
@pytest.mark.parametrize("comp", [0, 7])
def test_weighted_capture_parity(lib, mode, comp):
    m, n, tau, iters, seed = 256, 200, 0.7, 6, 4
    A = synthetic.gaussian(m, n, 9)
    h = synthetic.importance(n, 6)
    w = oracle.importance_weights(h, 0.0)
    res = lib.decompose(_dev(A), 0.5, tau, iters, 0, seed, mode=mode, capture=comp, stats=True,
                        importance=_dev(h))
    torch.cuda.synchronize()
    assert res.stat("mode") == {0: 0, 1: 1, 2: 3}[mode]
    cap = {k: v.cpu().numpy() for k, v in res.capture.items()}
    R64 = cap["R"].astype(np.float64)
    u = oracle.init_signs(seed, comp, m)
    for t in range(iters):
        y = cap["y"][t]
        assert _relnorm(y, R64.T @ u) <= 1e-5, ("y", t)          # plain target for v
        assert np.array_equal(oracle.ternarize(y.astype(np.float64), tau), cap["v"][t]), ("v", t)
        v = cap["v"][t].astype(np.float64)
        x = cap["x"][t]
        assert _relnorm(x, R64 @ (w * v)) <= 1e-5, ("x", t)      # weighted target for u
        assert np.array_equal(oracle.ternarize(x.astype(np.float64), tau), cap["u"][t]), ("u", t)
        u = cap["u"][t].astype(np.float64)
    d_ref = (u @ R64 @ (w * v)) / (np.count_nonzero(u) * float(w @ (v * v)))
    assert abs(float(cap["d"][0]) - d_ref) <= 1e-5 * abs(d_ref)


@pytest.mark.parametrize("block", [0, 6])
def test_weighting_raises_the_weighted_energy(lib, block):
    A = synthetic.gaussian(256, 192, 13)
    h = synthetic.importance(192, 7, sigma=2.0)
    w = oracle.importance_weights(h, 0.0)
    Ad = _dev(A)
    plain = lib.decompose(Ad, 1.0, 0.7, 15, block, 2)
    wtd = lib.decompose(Ad, 1.0, 0.7, 15, block, 2, importance=_dev(h))
    torch.cuda.synchronize()
    B, C, D = _factors(plain)
    e_plain = oracle.energy_from_factors(A, B, C, D, weights=w)
    assert float(wtd.energy.item()) > e_plain + 0.01


def test_weighted_sweeps(lib):
    A = synthetic.gaussian(256, 256, 21)
    h = synthetic.importance(256, 8)
    w = oracle.importance_weights(h, 0.0)
    Ad, hd = _dev(A), _dev(h)
    base = lib.decompose(Ad, 1.0, 0.7, 15, 32, 1, importance=hd)
    res = lib.decompose(Ad, 1.0, 0.7, 15, 32, 1, importance=hd, sweeps=2, trace=True)
    torch.cuda.synchronize()
    E = float(res.energy.item())
    assert E >= float(base.energy.item()) - 1e-6
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D, weights=w)) <= 1e-5
    ref = oracle.decompose_block(A, 1.0, 0.7, 15, 32, 1, sweeps=2, weights=w)
    assert abs(E - ref.E) <= 2e-3


def test_bad_importance_gives_nan(lib):
    A = _dev(synthetic.gaussian(64, 48, 1))
    for bad in (-1.0, float("nan"), float("inf")):
        h = torch.ones(48, dtype=torch.float32, device="cuda")
        h[5] = bad
        for block, mode in ((0, 1), (0, 0), (6, -1)):
            r = lib.decompose(A, 1.0, 0.7, 15, block, 0, mode=mode, stats=True, importance=h)
            torch.cuda.synchronize()
            assert np.isnan(float(r.energy.item()))
            assert r.stat("nonfinite") >= 1
    with pytest.raises(lib.ExterndError):
        lib.decompose(A, 1.0, 0.7, 15, 0, 0, importance=torch.ones(48, device="cuda"), lam=-1.0)
