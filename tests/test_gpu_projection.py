"""The optimal ternary projection (ExTernD §2.2) as the ternarizer, on the GPU.

The kernel sorts keys in LDS and takes its argmax on exact integers, as the
oracle does, so single vectors are compared bit for bit.  Decompositions
that use it (streaming and block mode) are compared end to end within 2e-3
of the oracle's energy, their reported energy against an fp64 recomputation
from their own factors to 1e-5, and step by step (bit-exact ternarization of
the captured vectors) in streaming mode.
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


def _vectors():
    rng = np.random.default_rng(12)
    out = []
    for N in (1, 2, 3, 15, 16, 17, 100, 1000, 2560, 4096, 4097, 9728, 16384):
        out.append(("normal", rng.standard_normal(N).astype(np.float32)))
    heavy = rng.standard_t(3, 5000).astype(np.float32)
    out.append(("student_t", heavy))
    ties = np.repeat(np.float32([0.5, -0.5, 0.25]), 700)
    rng.shuffle(ties)
    out.append(("ties", ties))
    out.append(("not_unimodal", np.float32([1.0] + [0.3] * 40)))
    z = rng.standard_normal(300).astype(np.float32)
    z[::3] = 0.0
    z[1] = -0.0
    out.append(("zeros", z))
    out.append(("all_zero", np.zeros(77, dtype=np.float32)))
    out.append(("tiny", (rng.standard_normal(64) * 1e-30).astype(np.float32)))
    return out


@pytest.mark.parametrize("name,x", _vectors(), ids=[v[0] + str(v[1].size) for v in _vectors()])
def test_projection_kernel_bit_exact(lib, name, x):
    codes, nnz = lib.project(_dev(x))
    torch.cuda.synchronize()
    got = oracle.unpack2(codes.cpu().numpy().view(np.uint32)[None, :], x.size)[0]
    want, _ = oracle.optimal_projection(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert int(nnz.item()) == np.count_nonzero(want)


def test_projection_length_limit(lib):
    with pytest.raises(lib.ExterndError) as ei:
        lib.project(torch.ones(16385, device="cuda"))
    assert ei.value.status == 4


@pytest.mark.parametrize("m,n,mu,block", [(256, 256, 1.0, 0), (300, 200, 1.0, 0), (256, 256, 1.0, 32),
                                          (300, 200, 1.3, 16)])
def test_projection_decomposition_vs_oracle(lib, m, n, mu, block):
    A = synthetic.gaussian(m, n, 19)
    Ad = _dev(A)
    res = lib.decompose(Ad, mu, 0.7, 15, block, 3, trace=True, stats=True, projection=True)
    torch.cuda.synchronize()
    if block:
        ref = oracle.decompose_block(A, mu, 0.7, 15, block, 3, projection=True)
        assert res.stat("mode") == 2
    else:
        ref = oracle.decompose_seq(A, mu, 0.7, 15, 3, projection=True)
        assert res.stat("mode") == 0   # AUTO takes the streaming path
    E = float(res.energy.item())
    assert abs(E - ref.E) <= 2e-3, (E, ref.E)
    B, C, D = _factors(res)
    assert abs(E - oracle.energy_from_factors(A, B, C, D)) <= 1e-5
    tr = res.trace.cpu().numpy()
    assert np.all(np.diff(tr) <= 1e-9 * ref.norm_a2)
    assert res.stat("nnz_b") == np.count_nonzero(B) and res.stat("nnz_c") == np.count_nonzero(C)
    # §2.2: the projection ties T_0.7
    plain = lib.decompose(Ad, mu, 0.7, 15, block, 3)
    assert abs(float(plain.energy.item()) - E) < 0.02


@pytest.mark.parametrize("comp", [0, 4])
def test_projection_capture_parity(lib, comp):
    m, n, iters, seed = 200, 160, 5, 2
    A = synthetic.gaussian(m, n, 23)
    res = lib.decompose(_dev(A), 0.5, 0.7, iters, 0, seed, capture=comp, projection=True)
    torch.cuda.synchronize()
    cap = {k: v.cpu().numpy() for k, v in res.capture.items()}
    for t in range(iters):
        v, _ = oracle.optimal_projection(cap["y"][t].astype(np.float64))
        assert np.array_equal(v, cap["v"][t]), ("v", t)
        u, _ = oracle.optimal_projection(cap["x"][t].astype(np.float64))
        assert np.array_equal(u, cap["u"][t]), ("u", t)


def test_projection_not_in_resident_mode(lib):
    Ad = _dev(synthetic.gaussian(64, 64, 1))
    with pytest.raises(lib.ExterndError) as ei:
        lib.decompose(Ad, 1.0, 0.7, 15, 0, 0, mode=lib.MODE_RESIDENT, projection=True)
    assert ei.value.status == 4
